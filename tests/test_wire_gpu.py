"""Residual wire codecs on the GPU (ADR-0009 "Wire Layout"), against the oracle.

* embed_gather_wire: the encoded rows are bit-exact to the oracle's encoding of
  the oracle's gathered f32 rows (f16 and per-position i8, every storage dtype,
  scaled and not, zero rows, values past the f16 range, bad ids);
* logits_topk_wire: ids and scores are bitwise those of logits_topk on the same
  path fed the oracle's decoding of the same wire rows, and accepted against the
  oracle's logits of those rows.
"""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from oracle import accept
from tests.gpu_util import bits, ids_dev, note, table, to_dev

pytestmark = pytest.mark.gpu

F32, BF16, Q8_0, F16 = etg.F32, etg.BF16, etg.Q8_0, etg.F16
WIRES = [etg.WIRE_F16, etg.WIRE_I8]


@pytest.mark.parametrize("dtype,d", [(F32, 100), (BF16, 896), (BF16, 2048), (F16, 2560), (Q8_0, 768), (Q8_0, 96)])
@pytest.mark.parametrize("wire", WIRES)
@pytest.mark.parametrize("scaled", [False, True])
def test_gather_wire_bit_exact(dtype, d, wire, scaled):
    V, n = 3001, 77
    host = synth.make_table(dtype, V, d, seed=1500 + d)
    if dtype == F32:
        host[5, :3] = [1e5, -7e4, 65519.0]        # past the f16 range: clamped to +-65504
        host[6, :] = 0.0                          # an all-zero row: i8 scale 0
    ids = synth.uniform_ids(n, V, seed=1600 + n)
    ids[:3] = [5, 6, V - 1]
    ids[10] = -1                                  # a bad id: all-zero record, counted
    t = table(host, dtype, V, d)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"gather wire dtype={dtype} d={d} wire={wire} scaled={scaled}")
    out = t.embed_gather_wire(ids_dev(ids), wire, scale="sqrt_d" if scaled else None, bad_count=cnt)
    torch.cuda.synchronize()
    x, nbad = oracle.embed_gather(host, dtype, V, d, ids, scale=oracle.sqrt_d(d) if scaled else None)
    want = oracle.wire_encode(x, wire)
    want[10] = 0
    assert int(cnt.item()) == nbad == 1
    got = out.cpu().numpy()
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"first mismatch at {bad[0].tolist()}"


@pytest.mark.parametrize("path,dtype,V,d,B", [
    (etg.PATH_VALU, F32, 2049, 100, 3), (etg.PATH_VALU, Q8_0, 3001, 768, 2),
    (etg.PATH_STREAM, BF16, 5003, 896, 1), (etg.PATH_STREAM, BF16, 5003, 200, 8),
    (etg.PATH_WIDE, BF16, 5003, 896, 33), (etg.PATH_GEMM, BF16, 4099, 512, 70),
    (etg.PATH_Q8, Q8_0, 3001, 768, 3), (etg.PATH_ROW, BF16, 5003, 896, 1), (etg.PATH_ROW, F32, 2049, 100, 2),
    (etg.PATH_RANK, BF16, 4099, 512, 70), (etg.PATH_RANK, BF16, 4099, 512, 200), (etg.PATH_RANK, BF16, 4099, 512, 300),
])
@pytest.mark.parametrize("wire", WIRES)
def test_logits_wire_equals_logits_of_decoded_rows(path, dtype, V, d, B, wire):
    host = synth.make_table(dtype, V, d, seed=1700 + V)
    R = synth.residuals(B, d, seed=1800 + B) * np.float32(3.0)
    R[0, :5] = 0.0
    enc = oracle.wire_encode(R, wire)
    dec = oracle.wire_decode(enc, d, wire)
    t = table(host, dtype, V, d)
    k = 10
    note(f"logits wire path={path} dtype={dtype} V={V} d={d} B={B} wire={wire}")
    gi, gs = t.logits_topk_wire(torch.from_numpy(enc).cuda(), wire, k, path=path)
    ri, rs = t.logits_topk(to_dev(dec), k, path=path)
    torch.cuda.synchronize()
    gi, gs, ri, rs = gi.cpu().numpy(), gs.cpu().numpy(), ri.cpu().numpy(), rs.cpu().numpy()
    assert np.array_equal(gi, ri)
    assert np.array_equal(bits(gs), bits(rs))
    L, A = oracle.logits(host, dtype, V, d, dec)
    oids, _ = oracle.topk(L, k)
    fails = accept.check_full(gi, gs, L, A, oids, accept.tol_coeff(dtype))
    assert not fails, fails[:3]


def test_embed_then_logits_over_i8_wire():
    # the service's two calls with the residual travelling as i8 in between
    V, d = 5003, 896
    host = synth.make_table(BF16, V, d, seed=1900)
    t = table(host, BF16, V, d)
    ids = synth.uniform_ids(6, V, seed=1901)
    note("embed -> i8 wire -> logits")
    enc = t.embed_gather_wire(ids_dev(ids), etg.WIRE_I8, scale="sqrt_d")
    gi, gs = t.logits_topk_wire(enc, etg.WIRE_I8, 5)
    torch.cuda.synchronize()
    x, _ = oracle.embed_gather(host, BF16, V, d, ids, scale=oracle.sqrt_d(d))
    dec = oracle.wire_decode(oracle.wire_encode(x, etg.WIRE_I8), d, etg.WIRE_I8)
    L, A = oracle.logits(host, BF16, V, d, dec)
    oids, _ = oracle.topk(L, 5)
    fails = accept.check_full(gi.cpu().numpy(), gs.cpu().numpy(), L, A, oids, accept.tol_coeff(BF16))
    assert not fails, fails[:3]
