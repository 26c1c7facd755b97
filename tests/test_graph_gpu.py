"""The library's calls inside a captured HIP graph.

Every call only enqueues kernels on the caller's stream: no allocation, no
synchronisation, no host-side wait and no memset node.  So a serving loop can
capture a whole step (gather + logits + top-k) once per shape and replay it.
Each test captures the calls on a side stream, then replays the graph three
times with new inputs copied into the captured buffers, with eager work and
synchronisations between the replays, and checks every replay bitwise against
the same calls run eagerly (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import synth
from tests.gpu_util import bits, note, table, to_dev

pytestmark = pytest.mark.gpu


def _eager(t, ids, R, k, path, T):
    x = t.embed_gather(ids, scale="sqrt_d", check=False)
    i, s = t.logits_topk(R, k, path=path)
    i2, s2, p2 = t.logits_topk_probs(R, k, temperature=T, path=path)
    raw = t.logits_raw(R, path=path)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (x, i, s, i2, s2, p2, raw)]


@pytest.mark.parametrize("dtype,V,d,B,path", [
    (etg.F32, 4096, 256, 4, etg.PATH_VALU),
    (etg.BF16, 5003, 896, 1, etg.PATH_STREAM),
    (etg.BF16, 5003, 896, 8, etg.PATH_STREAM),
    (etg.BF16, 5003, 896, 16, etg.PATH_WIDE),
    (etg.BF16, 5003, 896, 70, etg.PATH_GEMM),
    (etg.Q8_0, 3001, 768, 3, etg.PATH_VALU),
    (etg.Q8_0, 3001, 768, 3, etg.PATH_Q8),
    (etg.BF16, 5003, 896, 1, etg.PATH_ROW),
])
def test_captured_step_replays_match_eager(dtype, V, d, B, path):
    host = synth.make_table(dtype, V, d, seed=1200 + V)
    t = table(host, dtype, V, d)
    k, T, n = 10, 0.9, 37
    dev = torch.device("cuda")
    ids_buf = torch.zeros(n, dtype=torch.int32, device=dev)
    R_buf = torch.zeros((B, d), dtype=torch.float32, device=dev)
    ws = t.workspace(B, k, path)
    wsr = torch.empty(max(t.workspace_bytes(B, 1, path), 256), dtype=torch.uint8, device=dev)
    x_buf = torch.empty((n, d), dtype=torch.float32, device=dev)
    o = [torch.empty((B, k), dtype=torch.int32, device=dev), torch.empty((B, k), device=dev),
         torch.empty((B, k), dtype=torch.int32, device=dev), torch.empty((B, k), device=dev),
         torch.empty((B, k), device=dev)]
    raw_buf = torch.empty((B, V), dtype=torch.float32, device=dev)

    def step():
        t.embed_gather(ids_buf, scale="sqrt_d", out=x_buf, check=False)
        t.logits_topk(R_buf, k, path=path, workspace=ws, out_ids=o[0], out_scores=o[1])
        etg.lib().etg_logits_topk_probs(t.handle, R_buf.data_ptr(), B, k, T, o[2].data_ptr(), o[3].data_ptr(),
                                         o[4].data_ptr(), ws.data_ptr(), ws.numel(), path,
                                         torch.cuda.current_stream().cuda_stream)
        t.logits_raw(R_buf, path=path, out=raw_buf, workspace=wsr)

    note(f"graph capture dtype={dtype} V={V} d={d} B={B} path={path}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        ids = synth.uniform_ids(n, V, seed=1300 + rep)
        R = synth.residuals(B, d, seed=1400 + rep)
        ids_buf.copy_(torch.from_numpy(ids))
        R_buf.copy_(torch.from_numpy(R))
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = [x_buf.cpu().numpy()] + [a.cpu().numpy() for a in o] + [raw_buf.cpu().numpy()]
        want = _eager(t, to_dev(ids), to_dev(R), k, path, T)   # eager work between replays
        for j, (a, b) in enumerate(zip(got, want)):
            if a.dtype == np.int32:
                assert np.array_equal(a, b), (rep, j)
            else:
                assert np.array_equal(bits(a), bits(b)), (rep, j)


@pytest.mark.parametrize("B", [70, 200, 300])
def test_captured_rank_path_replays_match_eager(B):
    # the rank path answers the top-k alone (no probabilities or raw logits):
    # gather + top-k captured, replayed with new inputs, against eager calls
    V, d, k, n = 5003, 896, 10, 37
    host = synth.make_table(etg.BF16, V, d, seed=1250)
    t = table(host, etg.BF16, V, d)
    dev = torch.device("cuda")
    ids_buf = torch.zeros(n, dtype=torch.int32, device=dev)
    R_buf = torch.zeros((B, d), dtype=torch.float32, device=dev)
    ws = t.workspace(B, k, etg.PATH_RANK)
    x_buf = torch.empty((n, d), dtype=torch.float32, device=dev)
    oi = torch.empty((B, k), dtype=torch.int32, device=dev)
    osc = torch.empty((B, k), device=dev)

    def step():
        t.embed_gather(ids_buf, scale="sqrt_d", out=x_buf, check=False)
        t.logits_topk(R_buf, k, path=etg.PATH_RANK, workspace=ws, out_ids=oi, out_scores=osc)

    note(f"graph capture rank path V={V} d={d} B={B}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        ids = synth.uniform_ids(n, V, seed=1350 + rep)
        R = synth.residuals(B, d, seed=1450 + rep)
        ids_buf.copy_(torch.from_numpy(ids))
        R_buf.copy_(torch.from_numpy(R))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [a.cpu().numpy().copy() for a in (x_buf, oi, osc)]
        x = t.embed_gather(ids_buf, scale="sqrt_d", check=False)
        i, s = t.logits_topk(R_buf, k, path=etg.PATH_RANK)
        torch.cuda.synchronize()
        assert np.array_equal(got[1], i.cpu().numpy()), f"replay {rep}: ids differ from eager"
        for a, b in ((got[0], x), (got[2], s)):
            assert np.array_equal(bits(a), bits(b)), f"replay {rep} differs from eager"
