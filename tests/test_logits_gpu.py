"""logits_topk on the GPU against the CPU oracle.

Small and ragged shapes compare every row with the oracle's full logits under
the acceptance rule (oracle/accept.py); the special cases (zero and one-hot
residuals, duplicate rows, planted winners) pin exact ids and scores.  Every
path (valu, stream) is forced on the same inputs.
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

F32, BF16, Q8_0, F16 = etg.F32, etg.BF16, etg.Q8_0, etg.F16
VALU, STREAM, GEMM, WIDE, ROW, RANK = (etg.PATH_VALU, etg.PATH_STREAM, etg.PATH_GEMM, etg.PATH_WIDE, etg.PATH_ROW,
                                       etg.PATH_RANK)
ALL = [VALU, STREAM, GEMM, WIDE, ROW, RANK]


def run(t, R, k, path):
    note(f"logits dtype={t.dtype} V={t.vocab} d={t.hidden} B={R.shape[0]} k={k} path={path}")
    ids, sc = t.logits_topk(to_dev(R), k, path=path)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def full_check(host, dtype, V, d, R, k, path, t=None):
    t = t or table(host, dtype, V, d)
    gids, gsc = run(t, R, k, path)
    L, A = oracle.logits(host, dtype, V, d, R)
    oids, osc = oracle.topk(L, k)
    fails = accept.check_full(gids, gsc, L, A, oids, accept.tol_coeff(dtype))
    assert not fails, fails[:5]
    return gids, gsc, oids, osc


def test_tiny_config_f32():
    cfg = synth.CONFIGS["tiny"]
    host = cfg.table()
    R = cfg.residuals(4)
    full_check(host, cfg.dtype, cfg.V, cfg.d, R, cfg.k, etg.PATH_AUTO)


@pytest.mark.parametrize("dtype,V,d", [(F32, 2049, 100), (BF16, 5003, 200), (BF16, 4099, 896),
                                       (Q8_0, 3001, 96), (Q8_0, 2000, 768), (F16, 2049, 104), (F16, 4099, 896)])
@pytest.mark.parametrize("B", [1, 3, 9])
def test_valu_path_ragged(dtype, V, d, B):
    host = synth.make_table(dtype, V, d, seed=100 + V)
    R = synth.residuals(B, d, seed=200 + B)
    full_check(host, dtype, V, d, R, 10, VALU)


@pytest.mark.parametrize("V,d", [(5003, 200), (4099, 896), (1001, 64), (20000, 5376), (37, 8)])
@pytest.mark.parametrize("B", [1, 2, 4, 5, 8, 9, 17])
def test_stream_path_ragged(V, d, B):
    host = synth.make_table(BF16, V, d, seed=300 + V)
    R = synth.residuals(B, d, seed=400 + B)
    k = min(10, V)
    full_check(host, BF16, V, d, R, k, STREAM)


@pytest.mark.parametrize("V,d", [(5003, 200), (4099, 896), (1001, 64), (20000, 5376), (37, 8), (70000, 512)])
@pytest.mark.parametrize("B", [1, 9, 33, 64, 65, 130])
def test_gemm_path_ragged(V, d, B):
    host = synth.make_table(BF16, V, d, seed=500 + V)
    R = synth.residuals(B, d, seed=600 + B)
    full_check(host, BF16, V, d, R, min(10, V), GEMM)


# the rank path: up to 256 rows the wide kernel ranks in one pass (1 to 8 N-tiles
# over 512-row blocks, 9 to 16 over 256-row blocks, 4 keys per block; 65, 100,
# 130, 200 and 256 rows are 5, 7, 9, 13 and 16 N-tiles), past 256 the contraction
# (256-row column tiles, ragged last one, one or many vocabulary ranges, lists of
# fewer keys than k)
@pytest.mark.parametrize("V,d", [(5003, 200), (4099, 896), (1001, 64), (20000, 5376), (37, 8), (70000, 512)])
@pytest.mark.parametrize("B", [1, 9, 17, 33, 64, 65, 100, 128, 130, 200, 256, 257])
def test_rank_path_ragged(V, d, B):
    host = synth.make_table(BF16, V, d, seed=500 + V)
    R = synth.residuals(B, d, seed=600 + B)
    full_check(host, BF16, V, d, R, min(10, V), RANK)


# batches past three 256-row column tiles of the ranking contraction (and past
# six 128-row tiles of the split one): every row of tiles 2 and 3 against the
# oracle's own top-k
@pytest.mark.parametrize("path", [RANK, GEMM])
@pytest.mark.parametrize("V,d,B", [(70000, 512, 769), (5003, 200, 1000)])
def test_mfma_paths_past_three_column_tiles(path, V, d, B):
    host = synth.make_table(BF16, V, d, seed=510 + V)
    R = synth.residuals(B, d, seed=610 + B)
    full_check(host, BF16, V, d, R, 10, path)


# an odd number of 512-row blocks (9) with k = 1 or 3 keys per block: the
# rescoring's list of block keys has an odd length, and its residual row must
# still sit 16-byte aligned in LDS after that list
@pytest.mark.parametrize("k", [1, 3])
@pytest.mark.parametrize("path", [RANK, etg.PATH_AUTO])
def test_rank_path_odd_block_count(k, path):
    V, d, B = 4099, 512, 20
    host = synth.make_table(BF16, V, d, seed=520 + k)
    R = synth.residuals(B, d, seed=620 + k)
    full_check(host, BF16, V, d, R, k, path)


@pytest.mark.parametrize("k", [10, 40, 64])
@pytest.mark.parametrize("B", [2, 70, 140, 300])
def test_rank_path_rescans_a_range_holding_many_winners(k, B):
    # 80 planted winners in rows 256..335, inside one range of the ranking kernel
    # (a 512-row block of the wide kernel keeping 4 keys for B = 2 and 70, a
    # 256-row block keeping 4 for B = 140, a 256-row range of the contraction
    # keeping 16 for B = 300): the certificate must send the whole range to exact
    # rescoring for the answer to hold the other winners
    V, d = 30000, 512
    host = synth.make_table(BF16, V, d, seed=23)
    R = synth.residuals(B, d, seed=24)
    u = R[0] / np.linalg.norm(R[0])
    for j in range(80):
        host[256 + j] = synth.f32_to_bf16_bits((u * (0.9 - 0.005 * j)).astype(np.float32))
    gids, _, oids, _ = full_check(host, BF16, V, d, R, k, RANK)
    assert np.array_equal(gids[0], np.arange(256, 256 + k))
    assert np.array_equal(gids[0], oids[0])


# 256 planted rows filling the tile of rows 256..511 of the split contraction,
# ranked round-robin over 16 row groups of its register layout (wave row, M-tile,
# half-wave; 16 rows each): the first tile's lower bound on the k-th best must
# vouch for k groups (k = 17 fails a bound taking floor(k / 4) of each holder's
# 4-row groups, k > 16 one taking the 16-row groups)
@pytest.mark.parametrize("k", [16, 17, 40, 64])
@pytest.mark.parametrize("B", [2, 70])
def test_split_path_keeps_many_winners_of_one_tile(k, B):
    V, d = 30000, 512
    host = synth.make_table(BF16, V, d, seed=25)
    R = synth.residuals(B, d, seed=26)
    u = R[0] / np.linalg.norm(R[0])
    rows = np.arange(256)
    group = (rows // 128) * 8 + (rows % 128) // 32 * 2 + (rows % 8) // 4
    rank = (4 * ((rows % 32) // 8) + rows % 4) * 16 + group
    for r in rows:
        host[256 + r] = synth.f32_to_bf16_bits((u * (0.9 - 0.002 * rank[r])).astype(np.float32))
    gids, _, oids, _ = full_check(host, BF16, V, d, R, k, GEMM)
    assert np.array_equal(gids[0], 256 + np.argsort(rank)[:k])
    assert np.array_equal(gids[0], oids[0])


# 256 planted rows filling the tile of rows 256..511, ranked round-robin over the 4
# holders of a column's tile rows (wave row, half-wave) first and then over each
# holder's 16 groups of 4 rows: the top k are spread as evenly as possible, so a
# first-tile bound vouching for fewer than ceil(k / 4) groups per holder drops a
# winner whenever 4 does not divide k (split contraction, and the rank path's
# contraction, whose certificate relies on each range's list being its top keys)
@pytest.mark.parametrize("k", [1, 5, 6, 13, 40, 63])
@pytest.mark.parametrize("path,B", [(GEMM, 2), (GEMM, 70), (RANK, 300)])
def test_first_tile_bound_keeps_winners_spread_over_holders(path, B, k):
    V, d = 30000, 512
    host = synth.make_table(BF16, V, d, seed=27)
    R = synth.residuals(B, d, seed=28)
    u = R[0] / np.linalg.norm(R[0])
    rows = np.arange(256)
    holder = (rows // 128) * 2 + (rows % 8) // 4
    group = (rows % 128) // 32 * 4 + (rows % 32) // 8
    rank = 4 * ((rows % 4) * 16 + group) + holder
    for r in rows:
        host[256 + r] = synth.f32_to_bf16_bits((u * (0.9 - 0.002 * rank[r])).astype(np.float32))
    gids, _, oids, _ = full_check(host, BF16, V, d, R, k, path)
    assert np.array_equal(gids[0], 256 + np.argsort(rank)[:k])
    assert np.array_equal(gids[0], oids[0])


# the row path: rows of 16 bytes to 16 KiB (1 to 16 KiB loads, the last one partial),
# f32 / bf16 / f16 tables, one table pass per residual row
@pytest.mark.parametrize("dtype,V,d", [(BF16, 5003, 200), (BF16, 4099, 896), (BF16, 37, 8), (BF16, 20000, 5376),
                                       (BF16, 1500, 8192), (F32, 2049, 100), (F32, 3000, 4096), (F16, 2049, 104),
                                       (F16, 4099, 2560)])
@pytest.mark.parametrize("B", [1, 3])
def test_row_path_ragged(dtype, V, d, B):
    host = synth.make_table(dtype, V, d, seed=700 + V + d)
    R = synth.residuals(B, d, seed=800 + B)
    full_check(host, dtype, V, d, R, min(10, V), ROW)


# f32 and f16 rows too wide for the row path (over 16 KiB) take the VALU path;
# the f32 tables' bound of 1e-5 sum|r e| holds there up to 65,536 values.  The
# residual of row 0 is aligned with table row 3 (every product positive), so its
# rounding errors do not cancel.
@pytest.mark.parametrize("dtype,d", [(F32, 16384), (F16, 16384), (F32, 65536), (F16, 65536)])
@pytest.mark.parametrize("path", [etg.PATH_AUTO, VALU])
def test_wide_f32_f16_rows_within_1e5(dtype, d, path):
    V, B = 1001, 3
    host = synth.make_table(dtype, V, d, seed=900 + d + dtype)
    R = synth.residuals(B, d, seed=901)
    E3 = oracle.f16_to_f64(host[3]) if dtype == F16 else host[3].astype(np.float64)
    R[0] = (np.sign(E3) * (1.0 + np.abs(R[0]) / 8)).astype(np.float32)
    full_check(host, dtype, V, d, R, 10, path)


# the wide path: 512-row blocks (ragged last block), 4-step K chunks (ragged last
# chunk and 64-value step), 1 to 4 N-tiles per pass and several passes
@pytest.mark.parametrize("V,d", [(5003, 200), (4099, 896), (1001, 64), (20000, 5376), (37, 8), (70000, 512),
                                 (1536, 1032)])
@pytest.mark.parametrize("B", [1, 9, 16, 17, 33, 48, 64, 65, 130, 200])
def test_wide_path_ragged(V, d, B):
    host = synth.make_table(BF16, V, d, seed=700 + V)
    R = synth.residuals(B, d, seed=800 + B)
    full_check(host, BF16, V, d, R, min(10, V), WIDE)


@pytest.mark.parametrize("k", [1, 2, 40, 64])
@pytest.mark.parametrize("path", ALL)
def test_k_range(k, path):
    V, d = 7001, 256
    host = synth.make_table(BF16, V, d, seed=17)
    R = synth.residuals(3, d, seed=18)
    full_check(host, BF16, V, d, R, k, path)


@pytest.mark.parametrize("path", ALL)
def test_zero_residual_gives_ids_in_order(path):
    V, d = 3000, 128
    host = synth.make_table(BF16, V, d, seed=5)
    ids, sc = run(table(host, BF16, V, d), np.zeros((2, d), np.float32), 64, path)
    assert np.array_equal(ids, np.tile(np.arange(64), (2, 1)))
    assert np.all(sc == 0)


# all-tie blocks of the wide ranking kernel (every logit 0) take its selection
# rounds over the accumulators, at 1 to 16 N-tiles; rows 16..31 are nonzero so
# that tied and untied columns share a block
@pytest.mark.parametrize("B", [3, 40, 72, 128, 200, 256])
def test_rank_path_all_tie_blocks(B):
    V, d = 3000, 128
    host = synth.make_table(BF16, V, d, seed=5)
    R = np.zeros((B, d), np.float32)
    if B > 16:
        n = min(B, 32) - 16
        R[16:16 + n] = synth.residuals(n, d, seed=7)
    gids, gsc, oids, osc = full_check(host, BF16, V, d, R, 20, RANK)
    assert np.array_equal(gids[0], np.arange(20))
    assert np.all(gsc[0] == 0)


@pytest.mark.parametrize("path", ALL)
@pytest.mark.parametrize("B", [1, 6])
def test_one_hot_residual_selects_column_exactly(path, B):
    V, d = 4000, 192
    host = synth.make_table(BF16, V, d, seed=6)
    R = np.zeros((B, d), np.float32)
    cols = [0, 191, 64, 65, 127, 3][:B]
    for b, j in enumerate(cols):
        R[b, j] = 1.0
    gids, gsc = run(table(host, BF16, V, d), R, 20, path)
    L, _ = oracle.logits(host, BF16, V, d, R)
    oids, osc = oracle.topk(L, 20)
    assert np.array_equal(gids, oids)
    assert np.array_equal(gsc.view(np.uint32), osc.view(np.uint32))


@pytest.mark.parametrize("path", ALL)
def test_duplicate_rows_rank_by_id(path):
    V, d = 5000, 256
    host = synth.make_table(BF16, V, d, seed=9)
    R = synth.residuals(1, d, seed=10)
    best = synth.f32_to_bf16_bits((R[0] / np.linalg.norm(R[0]) * 0.5).astype(np.float32))
    for v in (4999, 17, 2048, 8):
        host[v] = best
    gids, _, oids, _ = full_check(host, BF16, V, d, R, 6, path)
    assert list(gids[0][:4]) == [8, 17, 2048, 4999]
    assert np.array_equal(gids, oids)


@pytest.mark.parametrize("path", ALL)
def test_planted_winners_exact_order(path):
    V, d = 30000, 512
    host = synth.make_table(BF16, V, d, seed=11)
    R = synth.residuals(2, d, seed=12)
    planted = [[29999, 5, 12345, 777], [0, 15000, 29998, 1]]
    for b in range(2):
        u = R[b] / np.linalg.norm(R[b])
        for j, v in enumerate(planted[b]):
            host[v] = synth.f32_to_bf16_bits((u * (0.6 - 0.1 * j)).astype(np.float32))
    gids, _, oids, _ = full_check(host, BF16, V, d, R, 4, path)
    assert gids.tolist() == planted
    assert np.array_equal(gids, oids)


@pytest.mark.parametrize("k", [1, 10, 16])
def test_merge_threshold_pass_and_its_fallback(k):
    # 70,001 rows on the stream path: 256 per-block lists, so the merge takes its
    # threshold pass (16-list group maxima); rows: a random residual, winners that
    # all sit in one block's list (a whole list prefix at or above the bound), a
    # zero residual (every logit ties: the pass overflows and the rounds answer)
    V, d = 70001, 64
    host = synth.make_table(BF16, V, d, seed=15)
    R = synth.residuals(3, d, seed=16)
    u = R[1] / np.linalg.norm(R[1])
    planted = list(range(40000, 40000 + 16))  # one 273-row block holds them all
    for j, v in enumerate(planted):
        host[v] = synth.f32_to_bf16_bits((u * (2.0 - 0.05 * j)).astype(np.float32))
    R[2] = 0
    gids, gsc, oids, _ = full_check(host, BF16, V, d, R, k, STREAM)
    assert gids[1].tolist() == planted[:k]
    assert gids[2].tolist() == list(range(k)) and np.all(gsc[2] == 0)
    assert np.array_equal(gids[:2], oids[:2])


@pytest.mark.parametrize("path", ALL)
def test_repeatable_bitwise(path):
    V, d = 50000, 896
    host = synth.make_table(BF16, V, d, seed=13)
    R = to_dev(synth.residuals(5, d, seed=14))
    t = table(host, BF16, V, d)
    note(f"logits repeat x20 path={path}")
    i0, s0 = t.logits_topk(R, 10, path=path)
    i0, s0 = i0.clone(), s0.clone()
    for _ in range(20):
        i1, s1 = t.logits_topk(R, 10, path=path)
        assert torch.equal(i0, i1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))


def test_paths_agree_on_bf16():
    V, d = 20011, 1024
    host = synth.make_table(BF16, V, d, seed=15)
    R = synth.residuals(6, d, seed=16)
    t = table(host, BF16, V, d)
    outs = [run(t, R, 10, path) for path in ALL]
    L, A = oracle.logits(host, BF16, V, d, R)
    oids, _ = oracle.topk(L, 10)
    for g in outs:
        assert not accept.check_full(g[0], g[1], L, A, oids, accept.tol_coeff(BF16))


def test_vocab_smaller_than_k_slots():
    # fewer rows than one block's share: blocks with no rows must not leak empty keys
    V, d = 9, 64
    host = synth.make_table(BF16, V, d, seed=19)
    R = synth.residuals(2, d, seed=20)
    for path in ALL:
        full_check(host, BF16, V, d, R, 9, path)


@pytest.mark.parametrize("path", ALL)
@pytest.mark.parametrize("B,d", [(1, 64), (3, 896), (6, 5376), (8, 200)])
def test_residual_at_bf16_midpoints_stays_within_tolerance(path, B, d):
    # r_i = (1 + 2^-8) * sign(e_i) sits halfway between two bf16 values; rounding it
    # once would lose 2^-8 / (1 + 2^-8) = 3.9e-3 of sum|r e|, twice the 2e-3 bound.
    V = 777
    host = synth.make_table(BF16, V, d, seed=21)
    E = oracle.bf16_to_f64(host)
    R = np.empty((B, d), np.float32)
    for b in range(B):
        R[b] = np.where(E[(37 * b) % V] >= 0, 1.0, -1.0) * np.float32(1 + 2 ** -8)
        # one bf16 rounding of this residual misses the bound on the row it is aligned with
        row = E[(37 * b) % V]
        single = oracle.bf16_to_f64(synth.f32_to_bf16_bits(R[b])) @ row
        exact = R[b].astype(np.float64) @ row
        assert abs(single - exact) > 2e-3 * (np.abs(R[b]).astype(np.float64) @ np.abs(row))
    full_check(host, BF16, V, d, R, 5, path)


def test_untied_lm_head_is_a_second_handle():
    # ADR-0008 "Vindex Slice: embed": lm_head.bin is the embeddings when tied, else
    # its own matrix.  Gather from an f16 embedding table, project through a
    # separate bf16 lm_head table of another vocabulary size.
    Ve, Vh, d = 3000, 4099, 256
    emb = synth.make_table(F16, Ve, d, seed=90)
    head = synth.make_table(BF16, Vh, d, seed=91)
    te, th = table(emb, F16, Ve, d), table(head, BF16, Vh, d)
    ids = synth.uniform_ids(5, Ve, seed=92)
    note("untied: gather f16, logits bf16")
    x = te.embed_gather(torch.from_numpy(ids).cuda())
    gids, gsc = th.logits_topk(x, 10)
    torch.cuda.synchronize()
    xr, _ = oracle.embed_gather(emb, F16, Ve, d, ids)
    assert np.array_equal(x.cpu().numpy().view(np.uint32), xr.view(np.uint32))
    L, A = oracle.logits(head, BF16, Vh, d, xr)
    oids, _ = oracle.topk(L, 10)
    fails = accept.check_full(gids.cpu().numpy(), gsc.cpu().numpy(), L, A, oids, accept.tol_coeff(BF16))
    assert not fails, fails[:3]


@pytest.mark.parametrize("B", [1, 8, 33])
def test_logits_to_host_matches_the_device_answer(B):
    # the answer copied to page-locked host memory behind an event equals the
    # device answer of the same call, bit for bit
    V, d = 20011, 896
    host = synth.make_table(BF16, V, d, seed=31)
    R = to_dev(synth.residuals(B, d, seed=32))
    t = table(host, BF16, V, d)
    note(f"logits to host B={B}")
    di, ds = t.logits_topk(R, 10)
    hi, hs, ev = t.logits_topk_to_host(R, 10)
    assert hi.is_pinned() and hs.is_pinned()
    ev.synchronize()
    assert torch.equal(hi, di.cpu()) and torch.equal(hs.view(torch.int32), ds.cpu().view(torch.int32))
    # reused host buffers, a second call in a row
    hi.fill_(-1)
    hi2, hs2, ev2 = t.logits_topk_to_host(R, 10, host_out=(hi, hs))
    ev2.synchronize()
    assert hi2.data_ptr() == hi.data_ptr() and torch.equal(hi2, di.cpu())


def test_logits_to_host_with_pageable_buffers():
    # pageable host memory: the copy is still correct (it blocks instead)
    import ctypes
    V, d, B, k = 5003, 256, 3, 7
    host = synth.make_table(BF16, V, d, seed=33)
    R = to_dev(synth.residuals(B, d, seed=34))
    t = table(host, BF16, V, d)
    ws = t.workspace(B, k)
    ids = torch.empty((B, k), dtype=torch.int32, device=R.device)
    sc = torch.empty((B, k), dtype=torch.float32, device=R.device)
    h_ids = np.full((B, k), -7, np.int32)
    h_sc = np.zeros((B, k), np.float32)
    ev = torch.cuda.Event()
    ev.record()
    note("logits to pageable host buffers")
    st = etg.lib().etg_logits_topk_to_host(t._h, ctypes.c_void_p(R.data_ptr()), B, k, ctypes.c_void_p(ids.data_ptr()),
                                           ctypes.c_void_p(sc.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                           etg.PATH_AUTO, h_ids.ctypes.data_as(ctypes.c_void_p),
                                           h_sc.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(ev.cuda_event),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    ev.synchronize()
    assert np.array_equal(h_ids, ids.cpu().numpy()) and np.array_equal(h_sc.view(np.int32), sc.cpu().numpy().view(np.int32))


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    step = {F32: 4, BF16: 8, F16: 8, Q8_0: 32}
    out = []
    for i in range(n):
        dt = [F32, BF16, F16, Q8_0][int(rng.integers(4))]
        d = int(rng.integers(1, 768 // step[dt] + 1)) * step[dt]
        V = int(rng.choice([1, 5, 63, 64, 65, 257, int(rng.integers(2, 6000))]))
        B = int(rng.choice([1, 2, 3, 8, 9, 16, 17, 33, int(rng.integers(1, 41))]))
        k = int(rng.integers(1, min(V, 64) + 1))
        out.append((i, dt, V, d, B, k))
    return out


@pytest.mark.parametrize("i,dtype,V,d,B,k", _random_shapes(40, 31))
def test_random_shapes_every_path(i, dtype, V, d, B, k):
    # seeded random shapes (dtype, vocabulary from 1 row up, hidden, batch, k): the
    # automatic choice and every path that plans the shape against the oracle
    host = synth.make_table(dtype, V, d, seed=3000 + i)
    R = synth.residuals(B, d, seed=3100 + i)
    t = table(host, dtype, V, d)
    L, A = oracle.logits(host, dtype, V, d, R)
    oids, _ = oracle.topk(L, k)
    for path in [etg.PATH_AUTO] + ALL + [etg.PATH_Q8]:
        if _plans(t, B, k, path):
            gids, gsc = run(t, R, k, path)
            fails = accept.check_full(gids, gsc, L, A, oids, accept.tol_coeff(dtype))
            assert not fails, (path, fails[:3])


def _plans(t, B, k, path):
    try:
        return t.workspace_bytes(B, k, path) > 0
    except etg.EtgError:
        return False
