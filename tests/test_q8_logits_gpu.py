"""The Q8_0 stream path of logits_topk on the GPU against the CPU oracle.

Two kernels serve the path.  Hidden a multiple of 256 (768, 4096, 4608, 5376,
8192 below) takes the matrix-core kernel for two or more residual rows: one MFMA
per 32-value block and 16-row tile, passes of 8 residual rows (2 to 17 rows: one
pass, ragged passes, three passes).  One residual row, and other widths, take the
lane-split kernel; its shapes cover every lane layout, from 1 block per row (64
rows per wave) to 256 (4 blocks per lane; 128, 144 and 168 blocks leave the last
of a lane's blocks to some lanes only), with passes of 2 residual rows.  Ragged
vocabularies throughout.  Special cases pin exact ids and scores.
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

Q8_0, Q8 = etg.Q8_0, etg.PATH_Q8


def run(t, R, k, path=Q8):
    note(f"q8 logits V={t.vocab} d={t.hidden} B={R.shape[0]} k={k} path={path}")
    ids, sc = t.logits_topk(to_dev(R), k, path=path)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def full_check(host, V, d, R, k, path=Q8):
    gids, gsc = run(table(host, Q8_0, V, d), R, k, path)
    L, A = oracle.logits(host, Q8_0, V, d, R)
    oids, osc = oracle.topk(L, k)
    fails = accept.check_full(gids, gsc, L, A, oids, accept.tol_coeff(Q8_0))
    assert not fails, fails[:5]
    return gids, gsc, oids, osc


# blocks per row: 1, 3, 9, 24, 100, 168, 256, 128, 144 -> lanes per row 1, 4, 16, 32, 64, 64, 64, 64, 64
@pytest.mark.parametrize("V,d", [(1001, 32), (3001, 96), (777, 288), (2000, 768), (4099, 3200), (4099, 5376),
                                 (1500, 8192), (2049, 4096), (5000, 4608), (37, 64), (37, 256), (13, 512),
                                 (61, 5376)])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 9, 17])
def test_q8_path_ragged(V, d, B):
    host = synth.make_table(Q8_0, V, d, seed=2000 + V + d)
    R = synth.residuals(B, d, seed=2100 + B)
    full_check(host, V, d, R, min(10, V))


def test_q8_zero_residual_gives_ids_in_order():
    V, d = 3000, 768
    host = synth.make_table(Q8_0, V, d, seed=2200)
    ids, sc = run(table(host, Q8_0, V, d), np.zeros((2, d), np.float32), 64)
    assert np.array_equal(ids, np.tile(np.arange(64), (2, 1)))
    assert np.all(sc == 0)


@pytest.mark.parametrize("d", [96, 768, 5376])
def test_q8_one_hot_residual_selects_column_exactly(d):
    # one product is q * 1 and every other term is +-0: the logit is int8 * scale exactly
    V = 4000
    host = synth.make_table(Q8_0, V, d, seed=2300 + d)
    cols = [0, d - 1, 33, 31 if d > 31 else 1]
    R = np.zeros((len(cols), d), np.float32)
    for b, j in enumerate(cols):
        R[b, j] = 1.0
    gids, gsc = run(table(host, Q8_0, V, d), R, 20)
    L, _ = oracle.logits(host, Q8_0, V, d, R)
    oids, osc = oracle.topk(L, 20)
    assert np.array_equal(gids, oids)
    assert np.array_equal(bits(gsc), bits(osc))


@pytest.mark.parametrize("d", [4096, 4608, 5376, 8192])
def test_q8_one_row_one_hot_in_every_block_round(d):
    # one residual row (the lane-split kernel, 64 lanes per row, lane l taking blocks
    # l, l + 64, ...): a single 1 at the first and last value of each round of 64
    # blocks and in an odd block (both byte alignments of a block) gives the logit
    # int8 * scale exactly
    V = 3001
    host = synth.make_table(Q8_0, V, d, seed=2350 + d)
    t = table(host, Q8_0, V, d)
    nb = d // 32
    cols = sorted({c for s0 in range(0, nb, 64) for c in (32 * s0, 32 * min(s0 + 64, nb) - 1, 32 * s0 + 33)})
    for c in cols:
        R = np.zeros((1, d), np.float32)
        R[0, c] = 1.0
        gids, gsc = run(t, R, 12)
        L, _ = oracle.logits(host, Q8_0, V, d, R)
        oids, osc = oracle.topk(L, 12)
        assert np.array_equal(gids, oids), c
        assert np.array_equal(bits(gsc), bits(osc)), c


def test_q8_duplicate_rows_rank_by_id_and_planted_winners():
    # row 100: codes aligned with R at scale 1; rows 3, 8, 17, 2048, 4999: the same
    # codes at scale 1/2, so they tie exactly for second place and rank by id
    V, d = 5000, 768
    host = synth.make_table(Q8_0, V, d, seed=2400)
    R = synth.residuals(1, d, seed=2401)
    q = np.clip(np.rint(R[0] / np.abs(R[0]).max() * 127), -127, 127).astype(np.int8).reshape(d // 32, 32)
    for v, sc in ((100, 0x3C00), (4999, 0x3800), (17, 0x3800), (2048, 0x3800), (8, 0x3800), (3, 0x3800)):
        blk = host[v].reshape(d // 32, 34)
        blk[:, :2] = np.array([sc], np.uint16).view(np.uint8)
        blk[:, 2:] = q.view(np.uint8)
    gids, gsc, oids, _ = full_check(host, V, d, R, 6)
    assert gids[0].tolist() == [100, 3, 8, 17, 2048, 4999]
    assert np.array_equal(gids, oids)
    assert len(set(bits(gsc[0][1:]).tolist())) == 1


def test_q8_repeatable_and_agrees_with_valu():
    V, d = 20011, 768
    host = synth.make_table(Q8_0, V, d, seed=2500)
    R = synth.residuals(4, d, seed=2501)
    t = table(host, Q8_0, V, d)
    note("q8 repeat x10")
    i0, s0 = t.logits_topk(to_dev(R), 10, path=Q8)
    for _ in range(10):
        i1, s1 = t.logits_topk(to_dev(R), 10, path=Q8)
        assert torch.equal(i0, i1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))
    L, A = oracle.logits(host, Q8_0, V, d, R)
    oids, _ = oracle.topk(L, 10)
    for path in (Q8, etg.PATH_VALU, etg.PATH_AUTO):
        g = run(t, R, 10, path)
        assert not accept.check_full(g[0], g[1], L, A, oids, accept.tol_coeff(Q8_0))


def test_q8_path_rejects_other_dtypes_and_wide_rows():
    hb = synth.make_table(etg.BF16, 100, 64, seed=1)
    with pytest.raises(etg.EtgError):
        table(hb, etg.BF16, 100, 64).logits_topk(torch.zeros((1, 64), device="cuda"), 3, path=Q8)
    hq = synth.make_table(Q8_0, 10, 8224, seed=2)                       # 257 blocks per row
    with pytest.raises(etg.EtgError):
        table(hq, Q8_0, 10, 8224).logits_topk(torch.zeros((1, 8224), device="cuda"), 3, path=Q8)


def test_gemma_embed_table_logits_full_size():
    # the EmbeddingGemma-shaped Q8_0 table (262,144 x 768) as an lm_head, B = 1 and 2
    cfg = synth.CONFIGS["gemma_embed"]
    host = cfg.table()
    t = table(host, Q8_0, cfg.V, cfg.d)
    R = synth.residuals(2, cfg.d, seed=2600)
    for B in (1, 2):
        gids, gsc = run(t, R[:B], 10)
        L, A = oracle.logits(host, Q8_0, cfg.V, cfg.d, R[:B])
        oids, _ = oracle.topk(L, 10)
        fails = accept.check_full(gids, gsc, L, A, oids, accept.tol_coeff(Q8_0))
        assert not fails, fails[:3]
