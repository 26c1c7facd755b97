"""Full-size workloads on the GPU, in the launch configuration the bench times.

The oracle computes full logits only for a few sampled residual rows per call
(each is one f64 pass over the table); every other row is checked through
properties that hold at any size: k distinct ids, scores equal to the oracle's
logits at those ids within tolerance, non-increasing order, and no id whose
logit falls below the oracle's k-th best by more than the tolerance.
"""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from oracle import accept
from tests.gpu_util import note, table, to_dev

pytestmark = pytest.mark.gpu

_cache = {}


def _table(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        cfg = synth.CONFIGS[name]
        note(f"generate {name} table ({cfg.table_bytes / 1e9:.2f} GB)")
        host = cfg.table()
        _cache[name] = (cfg, host, table(host, cfg.dtype, cfg.V, cfg.d))
    return _cache[name]


def _check(name, B, k, sample_rows, path=0):
    cfg, host, t = _table(name)
    R = synth.residuals(B, cfg.d, cfg.residual_seed(B))
    note(f"logits_topk {name} B={B} k={k} path={path}")
    gids, gsc = t.logits_topk(to_dev(R), k, path=path)
    torch.cuda.synchronize()
    gids, gsc = gids.cpu().numpy(), gsc.cpu().numpy()
    c = accept.tol_coeff(cfg.dtype)
    # every row: properties with the oracle's logits at the returned ids
    bs = np.repeat(np.arange(B), k)
    Lg, Ag = oracle.logits_at(host, cfg.dtype, cfg.V, cfg.d, R, bs, gids.reshape(-1))
    Lg, Ag = Lg.reshape(B, k), Ag.reshape(B, k)
    fails = []
    for b in range(B):
        fails += [f"row {b}: {s}" for s in accept.check_row(gids[b], gsc[b], cfg.V, c, Lg[b], Ag[b])]
    # sampled rows: the oracle's own top-k, all of them from one full pass over the table
    rows = sorted(set(sample_rows))
    L, A = oracle.logits(host, cfg.dtype, cfg.V, cfg.d, R[rows])
    oids, _ = oracle.topk(L, k)
    for i, b in enumerate(rows):
        fails += [f"row {b}: {s}" for s in accept.check_full(gids[b:b + 1], gsc[b:b + 1], L[i:i + 1], A[i:i + 1],
                                                             oids[i:i + 1], c)]
        # every returned logit is at least the oracle's k-th best minus the tolerance
        kth = L[i, oids[i, -1]]
        assert np.all(Lg[b] >= kth - c * (Ag[b] + A[i, oids[i, -1]]))
    assert not fails, fails[:5]


def test_qwen05b_logits_b1():
    _check("qwen05b", 1, 10, [0])


# B = 20 takes the rank path (the wide kernel ranking, then exact rescoring); the
# Qwen-shaped table has 297 blocks of 512 rows, an odd count, and k = 1 or 3 keeps
# 1 or 3 keys per block, so the rescoring's key list has an odd length
@pytest.mark.parametrize("k", [1, 3])
def test_qwen05b_logits_b20_rank_odd_block_count(k):
    _check("qwen05b", 20, k, range(20))


# B = 8: every row against the oracle's own top-k; B = 64: rows from each of the
# four 16-row N-tiles of the wide kernel
@pytest.mark.parametrize("B,sample", [(1, [0]), (8, range(8)), (64, [0, 9, 17, 31, 32, 47, 55, 63])])
def test_lm31b_logits(B, sample):
    _check("lm31b", B, 10, sample)


# the 31B-shaped lm_head stored as Q8_0 (1.50 GB): one residual row takes the
# lane-split kernel, two or more the matrix-core kernel (8 rows per table pass)
@pytest.mark.parametrize("B,sample", [(1, [0]), (2, [0, 1]), (8, range(8))])
def test_lm31b_q8_logits(B, sample):
    _check("lm31b_q8", B, 10, sample)


@pytest.mark.parametrize("path", [etg.PATH_STREAM, etg.PATH_ROW])
def test_lm31b_logits_b1_paths(path):
    _check("lm31b", 1, 10, [0], path)


@pytest.mark.parametrize("path", [etg.PATH_GEMM, etg.PATH_WIDE, etg.PATH_RANK])
def test_lm31b_logits_b64_mfma_paths(path):
    _check("lm31b", 64, 10, [0, 9, 17, 31, 32, 47, 55, 63], path)


# past 64 rows: the automatic choice ranks with the wide kernel in one table pass
# of 5 to 8 N-tiles over 512-row blocks (up to 128 rows), then of 9 to 16 over
# 256-row blocks (up to 256 rows)
@pytest.mark.parametrize("B", [96, 128, 200, 256])
def test_lm31b_logits_wide_rank_past_64_rows(B):
    _check("lm31b", B, 10, [0, 15, 16, 63, 64, B // 2 + 1, B - 1])


# rows from each 256-row column tile of the ranking contraction (and of the
# 128-row column tiles of the split one): both ends of every tile
_PREFILL_ROWS = [0, 255, 256, 300, 511, 512, 600, 767, 768, 1023]


def test_prefill_logits_b1024():
    # the automatic choice here is the rank path
    _check("prefill", 1024, 40, _PREFILL_ROWS)


def test_prefill_logits_b1024_split_gemm():
    _check("prefill", 1024, 40, _PREFILL_ROWS + [127, 128, 895, 896], etg.PATH_GEMM)


def test_lm31b_tied_gather_then_logits():
    # tied lm_head: gather rows from the same table, then project them back
    cfg, host, t = _table("lm31b")
    ids = np.array([0, 262143, 199729, 123456], np.int32)
    note("lm31b tied gather")
    x = t.embed_gather(torch.from_numpy(ids).cuda(), check=False)
    ref, _ = oracle.embed_gather(host, cfg.dtype, cfg.V, cfg.d, ids)
    assert torch.equal(x.cpu(), torch.from_numpy(ref))
    gids, gsc = t.logits_topk(x, 1)
    torch.cuda.synchronize()
    # a row's dot product with itself is its squared norm, by far the largest logit here
    assert gids.cpu().numpy()[:, 0].tolist() == ids.tolist()


@pytest.mark.parametrize("B,T", [(1, 1.0), (8, 0.7)])
def test_lm31b_probs_full_pass(B, T):
    # probabilities at the bench's shape: the oracle's full log-partition of row 0
    cfg, host, t = _table("lm31b")
    R = synth.residuals(B, cfg.d, cfg.residual_seed(B))
    note(f"logits_topk_probs lm31b B={B} T={T}")
    ids, sc, pr = t.logits_topk_probs(to_dev(R), 10, temperature=T)
    torch.cuda.synchronize()
    ids, sc, pr = ids.cpu().numpy(), sc.cpu().numpy(), pr.cpu().numpy()
    L, A = oracle.logits(host, cfg.dtype, cfg.V, cfg.d, R[:1])
    oids, _ = oracle.topk(L, 10)
    c = accept.tol_coeff(cfg.dtype)
    fails = accept.check_full(ids[:1], sc[:1], L, A, oids, c)
    fails += accept.check_probs(ids[:1], pr[:1], T, c, L, A)
    assert not fails, fails[:5]
    assert np.all((pr > 0) & (pr <= 1)) and np.all(np.diff(pr, axis=1) <= 0)


def test_lm31b_raw_logits_b1():
    # raw logits mode at the bench's shape: sampled entries against the oracle,
    # and the top-k of the vector against the top-k call
    cfg, host, t = _table("lm31b")
    R = synth.residuals(1, cfg.d, cfg.residual_seed(1))
    note("logits_raw lm31b B=1")
    raw = t.logits_raw(to_dev(R))
    ids, sc = t.logits_topk(to_dev(R), 10)
    torch.cuda.synchronize()
    raw, ids, sc = raw.cpu().numpy()[0], ids.cpu().numpy()[0], sc.cpu().numpy()[0]
    g = np.random.default_rng(5)
    vids = np.concatenate([g.integers(0, cfg.V, 2000), [0, cfg.V - 1], ids]).astype(np.int32)
    Lv, Av = oracle.logits_at(host, cfg.dtype, cfg.V, cfg.d, R, np.zeros(vids.size, np.int64), vids)
    assert np.all(np.abs(raw[vids].astype(np.float64) - Lv) <= accept.tol_coeff(cfg.dtype) * Av)
    assert np.array_equal(raw[ids].view(np.uint32), sc.view(np.uint32))
    order = np.lexsort((np.arange(cfg.V), -(raw.astype(np.float64) + 0.0)))
    assert np.array_equal(order[:10], ids)
