"""The C-ABI library without a GPU: it loads, exports what include/etg.h declares,
and every host-detectable error returns its status and message without a launch."""
import ctypes
import os
import re

import pytest

import embedding_table_gather_amd as etg
from tests.conftest import ROOT, read_golden

H = os.path.join(ROOT, "include", "etg.h")


@pytest.fixture(scope="module")
def L():
    return etg.lib()


def _declared():
    src = open(H).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(etg_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported_and_bound(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
        assert n in etg.SIGNATURES, f"{n} has no ctypes signature in the binding"
    assert set(etg.SIGNATURES) == set(names)


def test_version(L):
    assert L.etg_version() >= 100


def test_row_bytes_matches_page_sizes(L):
    dts = {"f32": etg.F32, "bf16": etg.BF16, "q8_0": etg.Q8_0, "f16": etg.F16}
    for name, dt, V, d, qty, expected, unit, src in read_golden("sizes.txt"):
        if unit == "B" and int(V) == 1:
            assert L.etg_row_bytes(dts[dt], int(d)) == int(expected), (name, src)
    assert L.etg_row_bytes(etg.BF16, 5376) == 10752
    assert L.etg_row_bytes(etg.Q8_0, 768) == 816
    assert L.etg_row_bytes(etg.F16, 2560) == 5120
    for dt, d in [(etg.F32, 6), (etg.BF16, 12), (etg.F16, 12), (etg.Q8_0, 48), (etg.BF16, 0), (etg.F32, 65540),
                  (9, 64)]:
        assert L.etg_row_bytes(dt, d) == -1, (dt, d)


def test_sqrt_d_matches_fixture(L):
    (hidden, hexbits, dec), = read_golden("embed_scale.txt")
    v = L.etg_sqrt_d(int(hidden))
    import struct
    assert struct.unpack("<I", struct.pack("<f", v))[0] == int(hexbits, 16)
    assert L.etg_sqrt_d(0) == 0.0


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced on these paths


def _create(L, ptr, dt, V, d):
    h = ctypes.c_void_p()
    st = L.etg_table_create(ctypes.c_void_p(ptr), dt, V, d, ctypes.byref(h))
    return st, h


def _err(L):
    return L.etg_last_error().decode()


def test_table_create_errors(L):
    assert _create(L, 0, etg.BF16, 10, 64)[0] == -1 and "NULL" in _err(L)
    assert _create(L, FAKE, 7, 10, 64)[0] == -2 and "dtype" in _err(L)
    assert _create(L, FAKE, etg.BF16, 0, 64)[0] == -3 and "vocab" in _err(L)
    assert _create(L, FAKE, etg.BF16, 2 ** 31, 64)[0] == -3
    assert _create(L, FAKE, etg.BF16, 10, 60)[0] == -3 and "hidden" in _err(L)
    assert _create(L, FAKE, etg.Q8_0, 10, 48)[0] == -3
    assert _create(L, FAKE + 8, etg.BF16, 10, 64)[0] == -4 and "aligned" in _err(L)
    assert L.etg_table_create(ctypes.c_void_p(FAKE), 1, 10, 64, None) == -1
    st, h = _create(L, FAKE, etg.Q8_0, 262144, 768)
    assert st == 0 and h.value
    assert L.etg_table_destroy(h) == 0
    assert L.etg_table_destroy(None) == 0


@pytest.fixture
def table(L):
    st, h = _create(L, FAKE, etg.BF16, 262144, 5376)
    assert st == 0
    yield h
    L.etg_table_destroy(h)


def test_gather_errors_without_launch(L, table):
    ids, out = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    assert L.etg_embed_gather(None, ids, 4, 1.0, out, None, None) == -1
    assert L.etg_embed_gather(table, ids, -1, 1.0, out, None, None) == -3
    assert L.etg_embed_gather(table, ids, 2 ** 31, 1.0, out, None, None) == -3
    assert L.etg_embed_gather(table, None, 4, 1.0, out, None, None) == -1
    assert L.etg_embed_gather(table, ids, 4, 1.0, None, None, None) == -1
    assert L.etg_embed_gather(table, ctypes.c_void_p(FAKE + 2), 4, 1.0, out, None, None) == -4
    assert L.etg_embed_gather(table, ids, 4, 1.0, ctypes.c_void_p(FAKE + 4), None, None) == -4
    assert L.etg_embed_gather(table, ids, 4, 1.0, out, ctypes.c_void_p(FAKE + 1), None) == -4
    assert L.etg_embed_gather(table, ids, 4, float("inf"), out, None, None) == -5
    # seq_len 0 enqueues nothing and succeeds, even with null buffers
    assert L.etg_embed_gather(table, None, 0, 1.0, None, None, None) == 0


def test_workspace_is_host_computable(L, table):
    n1 = L.etg_logits_topk_workspace(table, 1, 10)
    n64 = L.etg_logits_topk_workspace(table, 64, 10)
    assert 0 < n1 < n64
    assert n1 % 256 == 0
    assert L.etg_logits_topk_workspace_ex(table, 8, 10, etg.PATH_VALU) > 0
    assert L.etg_logits_topk_workspace(table, 0, 10) == -3
    assert L.etg_logits_topk_workspace(table, 1, 0) == -5
    assert L.etg_logits_topk_workspace(table, 1, 65) == -5
    assert L.etg_logits_topk_workspace_ex(table, 1, 10, 9) == -5
    assert L.etg_logits_topk_workspace(None, 1, 10) == -1


def test_workspace_rejects_stream_path_for_q8_0(L):
    st, h = _create(L, FAKE, etg.Q8_0, 1000, 64)
    assert st == 0
    assert L.etg_logits_topk_workspace_ex(h, 1, 5, etg.PATH_STREAM) == -5
    assert "bf16" in _err(L)
    assert L.etg_logits_topk_workspace_ex(h, 1, 5, etg.PATH_VALU) > 0
    L.etg_table_destroy(h)


def test_k_is_capped_by_vocab(L):
    st, h = _create(L, FAKE, etg.F32, 7, 64)
    assert L.etg_logits_topk_workspace(h, 1, 7) > 0
    assert L.etg_logits_topk_workspace(h, 1, 8) == -5
    L.etg_table_destroy(h)


def test_logits_errors_without_launch(L, table):
    p = ctypes.c_void_p(FAKE)
    ws_n = L.etg_logits_topk_workspace(table, 2, 10)
    f = L.etg_logits_topk
    assert f(None, p, 2, 10, p, p, p, ws_n, None) == -1
    assert f(table, None, 2, 10, p, p, p, ws_n, None) == -1
    assert f(table, p, 2, 10, None, p, p, ws_n, None) == -1
    assert f(table, p, 2, 10, p, p, None, ws_n, None) == -1
    assert f(table, p, 0, 10, p, p, p, ws_n, None) == -3
    assert f(table, p, 2, 0, p, p, p, ws_n, None) == -5
    assert f(table, ctypes.c_void_p(FAKE + 2), 2, 10, p, p, p, ws_n, None) == -4
    assert f(table, p, 2, 10, ctypes.c_void_p(FAKE + 1), p, p, ws_n, None) == -4
    assert f(table, p, 2, 10, p, p, ctypes.c_void_p(FAKE + 16), ws_n, None) == -4
    assert f(table, p, 2, 10, p, p, p, ws_n - 1, None) == -6 and "workspace" in _err(L)
    assert L.etg_logits_topk_ex(table, p, 2, 10, p, p, p, ws_n, 9, None) == -5


def test_to_host_errors_without_launch(L, table):
    p = ctypes.c_void_p(FAKE)
    ws_n = L.etg_logits_topk_workspace(table, 2, 10)
    f = L.etg_logits_topk_to_host
    assert f(table, p, 2, 10, p, p, p, ws_n, 0, None, p, p, None) == -1 and "host" in _err(L)
    assert f(table, p, 2, 10, p, p, p, ws_n, 0, p, None, p, None) == -1
    assert f(table, p, 2, 10, p, None, p, ws_n, 0, p, p, p, None) == -1 and "scores" in _err(L)
    assert f(table, p, 2, 10, p, p, p, ws_n, 0, p, p, None, None) == -1 and "event" in _err(L)
    # the logits call's own checks come first: nothing is copied or recorded then
    assert f(table, p, 0, 10, p, p, p, ws_n, 0, p, p, p, None) == -3
    assert f(table, p, 2, 10, p, p, p, ws_n - 1, 0, p, p, p, None) == -6


def test_probs_and_raw_errors_without_launch(L, table):
    p = ctypes.c_void_p(FAKE)
    ws_n = L.etg_logits_topk_workspace(table, 2, 10)
    f = L.etg_logits_topk_probs
    for T in (0.0, -1.0, float("inf"), float("nan"), 1e-39):
        assert f(table, p, 2, 10, T, p, p, p, p, ws_n, 0, None) == -5, T
        assert "temperature" in _err(L)
    assert f(table, p, 2, 10, 1.0, p, p, None, p, ws_n, 0, None) == -1
    assert f(table, p, 2, 10, 1.0, None, p, p, p, ws_n, 0, None) == -1
    assert f(table, p, 2, 10, 1.0, p, p, ctypes.c_void_p(FAKE + 2), p, ws_n, 0, None) == -4
    assert f(table, p, 2, 10, 1.0, p, p, p, p, ws_n - 1, 0, None) == -6
    rn = L.etg_logits_raw_workspace(table, 3, 0)
    assert rn == L.etg_logits_topk_workspace_ex(table, 3, 1, 0) > 0
    g = L.etg_logits_raw
    assert g(table, p, 3, None, p, rn, 0, None) == -1
    assert g(table, p, 3, ctypes.c_void_p(FAKE + 1), p, rn, 0, None) == -4
    assert g(table, p, 3, p, p, rn - 1, 0, None) == -6
    assert g(table, p, 0, p, p, rn, 0, None) == -3
    assert g(None, p, 3, p, p, rn, 0, None) == -1


def test_rank_path_planning(L, table):
    # the rank path: bf16 tables, top-k only; the auto workspace covers it and the
    # split contraction that probabilities / raw logits take at the same batch
    p = ctypes.c_void_p(FAKE)
    rank = L.etg_logits_topk_workspace_ex(table, 1024, 40, etg.PATH_RANK)
    gemm = L.etg_logits_topk_workspace_ex(table, 1024, 40, etg.PATH_GEMM)
    auto = L.etg_logits_topk_workspace(table, 1024, 40)
    assert rank > 0 and gemm > 0 and auto == max(rank, gemm)
    assert L.etg_logits_topk_probs(table, p, 1024, 40, 1.0, p, p, p, p, auto, etg.PATH_RANK, None) == -5
    assert "rank" in _err(L)
    assert L.etg_logits_raw(table, p, 1024, p, p, auto, etg.PATH_RANK, None) == -5
    for dtype, d in ((etg.F32, 64), (etg.Q8_0, 64), (etg.F16, 64)):
        st, h = _create(L, FAKE, dtype, 1000, d)
        assert st == 0
        assert L.etg_logits_topk_workspace_ex(h, 100, 5, etg.PATH_RANK) == -5 and "bf16" in _err(L)
        L.etg_table_destroy(h)
    # hidden past 16384: the residual row no longer fits the rescoring's LDS
    st, h = _create(L, FAKE, etg.BF16, 1000, 16392)
    assert st == 0
    assert L.etg_logits_topk_workspace_ex(h, 100, 5, etg.PATH_RANK) == -5 and "hidden" in _err(L)
    assert L.etg_logits_topk_workspace(h, 100, 5) == L.etg_logits_topk_workspace_ex(h, 100, 5, etg.PATH_GEMM) > 0
    L.etg_table_destroy(h)


def test_read_probe_errors_without_launch(L):
    p, s = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64)
    f = L.etg_hbm_read_probe
    assert f(None, 1024, s, None) == -1
    assert f(p, 1024, None, None) == -1
    assert f(ctypes.c_void_p(FAKE + 8), 1024, s, None) == -4
    assert f(p, 1024, ctypes.c_void_p(FAKE + 2), None) == -4
    assert f(p, 0, s, None) == -3 and f(p, 1000, s, None) == -3


def test_f16_tables_take_the_row_path_then_valu(L):
    # rows of up to 16 KiB (8,192 binary16 values) take the row path, wider ones VALU
    st, h = _create(L, FAKE, etg.F16, 1000, 64)
    assert st == 0
    assert L.etg_logits_topk_workspace_ex(h, 1, 5, etg.PATH_STREAM) == -5
    assert L.etg_logits_topk_workspace_ex(h, 4, 5, etg.PATH_AUTO) == L.etg_logits_topk_workspace_ex(
        h, 4, 5, etg.PATH_ROW) > 0
    L.etg_table_destroy(h)
    for d in (8192, 8200):
        st, h = _create(L, FAKE, etg.F16, 1000, d)
        assert st == 0
        want = etg.PATH_ROW if d == 8192 else etg.PATH_VALU
        assert L.etg_logits_topk_workspace_ex(h, 4, 5, etg.PATH_AUTO) == L.etg_logits_topk_workspace_ex(
            h, 4, 5, want) > 0
        if d == 8200:
            assert L.etg_logits_topk_workspace_ex(h, 4, 5, etg.PATH_ROW) == -5
        L.etg_table_destroy(h)


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        etg.Table(torch.zeros(16, dtype=torch.int16), etg.BF16, 1, 16)


def test_wire_formats(L, table):
    assert L.etg_wire_row_bytes(etg.WIRE_F32, 5376) == 21504
    assert L.etg_wire_row_bytes(etg.WIRE_F16, 5120) == 10240        # ADR-0009: half of 20 KB
    assert L.etg_wire_row_bytes(etg.WIRE_I8, 5120) == 5128          # 8-byte header + one byte per value
    assert L.etg_wire_row_bytes(3, 64) == -1 and L.etg_wire_row_bytes(etg.WIRE_I8, 0) == -1
    p = ctypes.c_void_p(FAKE)
    g = L.etg_embed_gather_wire
    assert g(table, p, 4, 1.0, 3, p, None, None) == -5
    assert g(table, p, 4, 1.0, etg.WIRE_I8, ctypes.c_void_p(FAKE + 2), None, None) == -4
    assert g(table, p, 4, 1.0, etg.WIRE_I8, None, None, None) == -1
    assert g(table, p, 0, 1.0, etg.WIRE_F16, None, None, None) == 0
    ws_n = L.etg_logits_topk_workspace(table, 2, 10)
    f = L.etg_logits_topk_wire
    assert f(table, p, 3, 2, 10, p, p, p, ws_n, 0, None) == -5
    assert f(table, ctypes.c_void_p(FAKE + 1), etg.WIRE_F16, 2, 10, p, p, p, ws_n, 0, None) == -4
    assert f(table, ctypes.c_void_p(FAKE + 2), etg.WIRE_I8, 2, 10, p, p, p, ws_n, 0, None) == -4
    assert f(table, p, etg.WIRE_I8, 2, 10, None, p, p, ws_n, 0, None) == -1


def test_noalloc_host_errors_without_launch(L, table):
    # host-detectable errors return before the scratch is looked up or anything runs
    p = ctypes.c_void_p(FAKE)
    f = L.etg_logits_topk_noalloc
    assert f(None, p, 1, 10, p, p, None) == -1
    assert f(table, p, 0, 10, p, p, None) == -3
    assert f(table, p, 1, 0, p, p, None) == -5
    # a shape whose workspace exceeds the 32 MiB scratch
    big = 4096
    assert L.etg_logits_topk_workspace(table, big, 64) > 32 << 20
    assert f(table, p, big, 64, p, p, None) == -6
    assert "scratch" in _err(L)


def test_write_probe_errors_without_launch(L):
    p = ctypes.c_void_p(FAKE)
    f = L.etg_hbm_write_probe
    assert f(None, 1024, 0, None) == -1
    assert f(ctypes.c_void_p(FAKE + 8), 1024, 0, None) == -4
    assert f(p, 0, 0, None) == -3 and f(p, 1000, 0, None) == -3


def test_step_cache_host_errors(L, table):
    assert L.etg_step_cache_ids_capacity(1) == 64 and L.etg_step_cache_ids_capacity(64) == 64
    assert L.etg_step_cache_ids_capacity(65) == 128 and L.etg_step_cache_ids_capacity(1024) == 1024
    assert L.etg_step_cache_ids_capacity(1025) == 1280 and L.etg_step_cache_ids_capacity(0) == -1
    assert L.etg_step_cache_workspace(table, 8, 10) == max(L.etg_logits_topk_workspace(table, b, 10)
                                                            for b in range(1, 9))
    assert L.etg_step_cache_workspace(table, 8, 0) == -5
    p = ctypes.c_void_p(FAKE)
    out = ctypes.c_void_p()
    f = L.etg_step_cache_create
    ws = L.etg_step_cache_workspace(table, 4, 5)
    assert f(table, 10, 4, 5, 1, p, p, p, p, p, p, ws, p, p, p, None) == -1
    assert f(table, 10, 4, 5, 1, None, p, p, p, p, p, ws, p, p, p, ctypes.byref(out)) == -1
    assert f(table, 0, 4, 5, 1, p, p, p, p, p, p, ws, p, p, p, ctypes.byref(out)) == -3
    assert f(table, 10, 4, 5, 1, p, p, p, p, p, p, ws - 1, p, p, p, ctypes.byref(out)) == -6
    assert f(table, 10, 4, 5, 1, p, ctypes.c_void_p(FAKE + 4), p, p, p, p, ws, p, p, p, ctypes.byref(out)) == -4
    assert f(table, 10, 4, 5, 1, p, p, p, p, p, p, ws, p, p, p, ctypes.byref(out)) == 0
    c = out.value
    import numpy as np
    ids = np.array([1, 262144], np.int32)  # the second is past the vocabulary
    assert L.etg_step_gather(ctypes.c_void_p(c), ids.ctypes.data_as(ctypes.c_void_p), 2, 1.0, None) == -5
    assert "bad token id" in _err(L)
    assert L.etg_step_gather(ctypes.c_void_p(c), ids.ctypes.data_as(ctypes.c_void_p), 11, 1.0, None) == -3
    assert L.etg_step_logits(ctypes.c_void_p(c), 5, None, None) == -3
    g, r = ctypes.c_int64(-1), ctypes.c_int64(-1)
    assert L.etg_step_cache_stats(ctypes.c_void_p(c), ctypes.byref(g), ctypes.byref(r)) == 0 and (g.value, r.value) == (0, 0)
    assert L.etg_step_cache_destroy(ctypes.c_void_p(c)) == 0


def test_every_valid_shape_has_an_automatic_plan(L):
    # seeded random shapes over the whole accepted range: the automatic path always
    # plans (a positive, 256-byte multiple workspace), and forced paths either plan or
    # return ETG_ERANGE / ETG_ESHAPE with a message
    import numpy as np
    rng = np.random.default_rng(7)
    step = {etg.F32: 4, etg.BF16: 8, etg.F16: 8, etg.Q8_0: 32}
    paths = [etg.PATH_VALU, etg.PATH_STREAM, etg.PATH_GEMM, etg.PATH_WIDE, etg.PATH_Q8, etg.PATH_ROW, etg.PATH_RANK]
    for _ in range(300):
        dt = [etg.F32, etg.BF16, etg.F16, etg.Q8_0][int(rng.integers(4))]
        d = int(rng.choice([step[dt], 64, 256, 768, 896, 2048, 4096, 5120, 5376, 8192, 16384, 65536]))
        d = max(step[dt], d // step[dt] * step[dt])
        V = int(rng.choice([1, 7, 63, 64, 65, 4099, 151936, 262144, 1 << 21]))
        st, h = _create(L, FAKE, dt, V, d)
        assert st == 0, (dt, V, d)
        try:
            k = int(rng.integers(1, min(V, 64) + 1))
            for B in sorted({1, 2, 8, 9, 17, 64, 65, 256, 257, 65536, int(rng.integers(1, 4097))}):
                n = L.etg_logits_topk_workspace(h, B, k)
                assert n > 0 and n % 256 == 0, (dt, V, d, B, k, n, _err(L))
                for p in paths:
                    m = L.etg_logits_topk_workspace_ex(h, B, k, p)
                    assert m > 0 or (m in (-3, -5) and _err(L)), (dt, V, d, B, k, p, m)
        finally:
            L.etg_table_destroy(h)
