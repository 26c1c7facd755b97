"""Probabilities at a temperature and the raw logits mode on the GPU, against the oracle.

ADR-0008 "POST /v1/logits": the response lists each top token with its
probability at the request's temperature, or (raw logits mode) returns the
whole logit vector.  Every path is forced on the same inputs:

* raw logits: every entry within the logit tolerance of the oracle, and bitwise
  the values the same path's top-k ranks (its ids are the top k of the vector);
* probabilities: ids and scores under the acceptance rule, probabilities within
  the bound that the logit tolerance implies (oracle/accept.py), and over a
  whole small vocabulary they sum to one (both sides use the same f32 logits,
  so only the f32 arithmetic of the probabilities enters).
"""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from oracle import accept
from tests.gpu_util import bits, note, table, to_dev

pytestmark = pytest.mark.gpu

F32, BF16, Q8_0, F16 = etg.F32, etg.BF16, etg.Q8_0, etg.F16
VALU, STREAM, GEMM, WIDE, Q8, ROW = (etg.PATH_VALU, etg.PATH_STREAM, etg.PATH_GEMM, etg.PATH_WIDE, etg.PATH_Q8,
                                    etg.PATH_ROW)
ALL = [VALU, STREAM, GEMM, WIDE, ROW]

# (dtype, V, d, B, path): ragged vocabularies, several blocks and passes per path
CASES = [
    (F32, 2049, 100, 3, VALU), (Q8_0, 3001, 96, 9, VALU), (BF16, 5003, 200, 2, VALU),
    (BF16, 5003, 200, 1, STREAM), (BF16, 4099, 896, 5, STREAM), (BF16, 37, 8, 8, STREAM),
    (BF16, 20000, 5376, 3, STREAM),
    (BF16, 5003, 200, 17, WIDE), (BF16, 1536, 1032, 64, WIDE), (BF16, 70000, 512, 33, WIDE),
    (BF16, 5003, 200, 65, GEMM), (BF16, 1001, 64, 130, GEMM), (BF16, 20000, 5376, 70, GEMM),
    (Q8_0, 3001, 768, 3, Q8), (Q8_0, 4099, 5376, 2, Q8), (Q8_0, 777, 288, 1, Q8),
    (BF16, 20000, 5376, 1, ROW), (F32, 2049, 100, 2, ROW), (F16, 4099, 2560, 1, ROW),
]


def _ids(c):
    return f"dt{c[0]}-V{c[1]}-d{c[2]}-B{c[3]}-p{c[4]}"


def _topk_of_vector(x: np.ndarray, k: int) -> np.ndarray:
    """Top k of a float32 vector by (value desc, id asc), -0 tying with +0."""
    v = x.astype(np.float64) + 0.0          # -0.0 + 0.0 = +0.0
    order = np.lexsort((np.arange(v.size), -v))
    return order[:k]


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_raw_logits_every_entry_and_topk_consistency(case):
    dtype, V, d, B, path = case
    host = synth.make_table(dtype, V, d, seed=700 + V)
    R = synth.residuals(B, d, seed=800 + B)
    t = table(host, dtype, V, d)
    note(f"raw dtype={dtype} V={V} d={d} B={B} path={path}")
    raw = t.logits_raw(to_dev(R), path=path)
    k = min(10, V)
    ids, sc = t.logits_topk(to_dev(R), k, path=path)
    torch.cuda.synchronize()
    raw = raw.cpu().numpy()
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    L, A = oracle.logits(host, dtype, V, d, R)
    c = accept.tol_coeff(dtype)
    err = np.abs(raw.astype(np.float64) - L)
    bad = np.argwhere(err > c * A)
    assert bad.size == 0, f"{len(bad)} raw logits beyond tolerance, first at {bad[0].tolist()}"
    for b in range(B):
        assert np.array_equal(bits(raw[b, ids[b]]), bits(sc[b])), f"row {b}: scores differ from raw logits"
        assert np.array_equal(_topk_of_vector(raw[b], k), ids[b]), f"row {b}: ids are not the raw top {k}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("T", [0.5, 1.0, 3.0])
def test_probs_against_oracle(case, T):
    dtype, V, d, B, path = case
    host = synth.make_table(dtype, V, d, seed=700 + V)
    R = synth.residuals(B, d, seed=900 + B)
    t = table(host, dtype, V, d)
    k = min(10, V)
    note(f"probs dtype={dtype} V={V} d={d} B={B} k={k} T={T} path={path}")
    ids, sc, pr = t.logits_topk_probs(to_dev(R), k, temperature=T, path=path)
    torch.cuda.synchronize()
    ids, sc, pr = ids.cpu().numpy(), sc.cpu().numpy(), pr.cpu().numpy()
    L, A = oracle.logits(host, dtype, V, d, R)
    oids, _ = oracle.topk(L, k)
    c = accept.tol_coeff(dtype)
    fails = accept.check_full(ids, sc, L, A, oids, c)
    fails += accept.check_probs(ids, pr, T, c, L, A)
    assert not fails, fails[:5]
    # the probabilities follow the scores (non-increasing)
    assert np.all(np.diff(pr.astype(np.float64), axis=1) <= 0)


@pytest.mark.parametrize("path", ALL)
def test_probs_of_whole_small_vocabulary_sum_to_one(path):
    V, d, B = 64, 256, 5
    dtype = F32 if path == VALU else BF16
    host = synth.make_table(dtype, V, d, seed=41)
    R = synth.residuals(B, d, seed=42) * 3.0
    t = table(host, dtype, V, d)
    for T in (0.25, 1.0, 10.0):
        note(f"probs sum V={V} k=64 T={T} path={path}")
        ids, _, pr = t.logits_topk_probs(to_dev(R), 64, temperature=T, path=path)
        torch.cuda.synchronize()
        s = pr.cpu().numpy().astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= 1e-5), s
        assert np.array_equal(np.sort(ids.cpu().numpy(), axis=1), np.tile(np.arange(V), (B, 1)))


@pytest.mark.parametrize("path", ALL)
def test_zero_residual_probs_are_one_over_v(path):
    V, d = 5003, 200
    dtype = F32 if path == VALU else BF16
    host = synth.make_table(dtype, V, d, seed=43)
    t = table(host, dtype, V, d)
    note(f"probs zero residual path={path}")
    ids, sc, pr = t.logits_topk_probs(torch.zeros((2, d), dtype=torch.float32, device="cuda"), 7, 0.7, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(7), (2, 1)))
    assert np.all(sc.cpu().numpy() == 0)
    # every term of the normaliser is exp2(0) = 1: only the f32 sum's rounding enters
    assert np.allclose(pr.cpu().numpy(), 1.0 / V, rtol=1e-5, atol=0)


def test_temperature_out_of_range_is_an_error():
    host = synth.make_table(BF16, 100, 64, seed=44)
    t = table(host, BF16, 100, 64)
    R = torch.ones((1, 64), dtype=torch.float32, device="cuda")
    for T in (0.0, -1.0, float("inf"), float("nan"), 1e-39):
        with pytest.raises(etg.EtgError) as e:
            t.logits_topk_probs(R, 3, temperature=T)
        assert e.value.status == -5
