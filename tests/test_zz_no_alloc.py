"""etg_logits_topk_noalloc (the library's own device scratch as the workspace)
against etg_logits_topk with a caller's workspace, through the C-ABI.

Two calls in a row on the same scratch, the second with a smaller input, must
each give bitwise the answer of the existing entry point (the same kernels),
and that answer must pass the oracle's acceptance rule."""
import ctypes

import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from oracle import accept
from tests.gpu_util import note, table, to_dev

pytestmark = pytest.mark.gpu


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(t, R, k):
    """(noalloc ids, scores), (etg_logits_topk ids, scores) for device residuals R."""
    L = etg.lib()
    B = R.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ids_n = torch.full((B, k), -1, dtype=torch.int32, device=R.device)
    sc_n = torch.full((B, k), float("nan"), dtype=torch.float32, device=R.device)
    note(f"noalloc V={t.vocab} d={t.hidden} B={B} k={k}")
    st = L.etg_logits_topk_noalloc(t.handle, _vp(R), B, k, _vp(ids_n), _vp(sc_n), stream)
    assert st == 0, L.etg_last_error()
    ws = torch.empty(max(t.workspace_bytes(B, k), 256), dtype=torch.uint8, device=R.device)
    ids_w = torch.empty((B, k), dtype=torch.int32, device=R.device)
    sc_w = torch.empty((B, k), dtype=torch.float32, device=R.device)
    note(f"with workspace V={t.vocab} d={t.hidden} B={B} k={k}")
    st = L.etg_logits_topk(t.handle, _vp(R), B, k, _vp(ids_w), _vp(sc_w), _vp(ws), ws.numel(), stream)
    assert st == 0, L.etg_last_error()
    torch.cuda.synchronize()
    return (ids_n.cpu().numpy(), sc_n.cpu().numpy()), (ids_w.cpu().numpy(), sc_w.cpu().numpy())


# (first batch, second smaller batch): the rank path's contraction then its wide
# kernel over 256-row blocks (16 N-tiles), the wide kernel at 8 then 3 N-tiles, the
# wide kernel then the stream kernel, the stream kernel with 8 then 1 row
@pytest.mark.parametrize("B1,B2", [(300, 256), (128, 40), (64, 5), (8, 1)])
def test_noalloc_matches_the_workspace_entry_point(B1, B2):
    V, d, k = 20011, 896, 10
    host = synth.make_table(synth.BF16, V, d, seed=41)
    t = table(host, synth.BF16, V, d)
    for B, seed in ((B1, 42), (B2, 43)):
        R = synth.residuals(B, d, seed=seed + B)
        (gi, gs), (wi, wsc) = _both(t, to_dev(R), k)
        assert np.array_equal(gi, wi)
        assert np.array_equal(gs.view(np.uint32), wsc.view(np.uint32))
        L, A = oracle.logits(host, synth.BF16, V, d, R)
        oids, _ = oracle.topk(L, k)
        fails = accept.check_full(gi, gs, L, A, oids, accept.tol_coeff(synth.BF16))
        assert not fails, fails[:3]


def test_noalloc_other_dtypes_and_the_binding():
    # an f32 table (row path) then a Q8_0 table (matrix-core kernel), on the same scratch
    for dt, V, d, B in ((synth.F32, 4096, 256, 4), (synth.Q8_0, 3001, 768, 3)):
        host = synth.make_table(dt, V, d, seed=44 + dt)
        t = table(host, dt, V, d)
        R = synth.residuals(B, d, seed=45)
        (gi, gs), (wi, wsc) = _both(t, to_dev(R), 5)
        assert np.array_equal(gi, wi) and np.array_equal(gs.view(np.uint32), wsc.view(np.uint32))
        oi = torch.empty((B, 5), dtype=torch.int32, device="cuda")
        os_ = torch.empty((B, 5), dtype=torch.float32, device="cuda")
        t.logits_topk_noalloc(to_dev(R), 5, oi, os_)
        torch.cuda.synchronize()
        assert np.array_equal(oi.cpu().numpy(), gi)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # nothing is launched: the size check comes first (zero-filled rows suffice)
    t = etg.Table(torch.zeros((300000, 64), dtype=torch.int16, device="cuda"), synth.BF16, 300000, 64)
    B, k = 16384, 64
    assert t.workspace_bytes(B, k) > 32 << 20
    R = torch.zeros((B, 64), dtype=torch.float32, device="cuda")
    oi = torch.empty((B, k), dtype=torch.int32, device="cuda")
    os_ = torch.empty((B, k), dtype=torch.float32, device="cuda")
    with pytest.raises(etg.EtgError, match="scratch"):
        t.logits_topk_noalloc(R, k, oi, os_)
