"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test compares the oracle with something other than itself: values the
pages print (tests/golden), hand-worked values, library routines (numpy's
binary16, torch's bfloat16, numpy float64 matmul and lexsort), closed forms
and special cases.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import accept
from tests.conftest import read_golden

F32, BF16, Q8_0, F16 = oracle.F32, oracle.BF16, oracle.Q8_0, oracle.F16
DT = {"f32": F32, "bf16": BF16, "q8_0": Q8_0, "f16": F16}


# ---------------------------------------------------------------- sizes (pages)
def test_row_and_table_sizes_match_pages():
    for name, dt, V, d, qty, expected, unit, src in read_golden("sizes.txt"):
        rb = oracle.row_bytes(DT[dt], int(d))
        n = rb * int(V)
        if unit == "B":
            got = n
            assert got == int(expected), (name, got, expected, src)
            continue
        div, nd = {"KiB1": (1024, 1), "kB1": (1000, 1), "MiB2": (1024 ** 2, 2), "GB2": (1e9, 2)}[unit]
        assert round(n / div, nd) == float(expected), (name, n / div, expected, src)


def test_row_bytes_rejects_bad_shapes():
    assert oracle.row_bytes(Q8_0, 48) == -1      # not a whole number of 32-value blocks
    assert oracle.row_bytes(BF16, 0) == -1
    assert oracle.row_bytes(7, 64) == -1
    assert oracle.row_bytes(Q8_0, 768) == 816


# ---------------------------------------------------------------- decoders
def test_f16_decoder_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _q8_row(blocks):
    """blocks: list of (scale_bits, [32 ints]) -> bytes of one Q8_0 row."""
    raw = b""
    for sbits, qs in blocks:
        raw += struct.pack("<H", sbits) + struct.pack("<32b", *qs)
    return np.frombuffer(raw, np.uint8)


def test_q8_0_hand_built_blocks():
    rows = read_golden("q8_0_blocks.txt")
    for sbits_s, q_s, expected, note in rows:
        sbits, q = int(sbits_s, 16), int(q_s)
        qs = [0] * 32
        qs[5] = q
        qs[31] = q
        row = _q8_row([(0x3C00, list(range(-16, 16))), (sbits, qs)])
        x = oracle.dequant_row(row, Q8_0, 64)
        want = float(Fraction(expected))
        assert x[32 + 5] == want and x[32 + 31] == want, (note, x[37], want)
        # the first block (scale 1.0) decodes to its integers
        assert np.array_equal(x[:32], np.arange(-16, 16, dtype=np.float64))
        # values are exact in float32
        assert float(np.float32(x[37])) == x[37]


def test_q8_0_block_order_and_signed_bytes():
    # value c of the row lives in block c // 32 at byte 2 + c % 32; bytes are signed
    qs0 = [(-128 + 7 * j) for j in range(32)]
    qs1 = [(127 - 3 * j) for j in range(32)]
    row = _q8_row([(0x4000, qs0), (0x3800, qs1)])      # scales 2.0 and 0.5
    x = oracle.dequant_row(row, Q8_0, 64)
    assert np.array_equal(x[:32], 2.0 * np.array(qs0, np.float64))
    assert np.array_equal(x[32:], 0.5 * np.array(qs1, np.float64))


# ---------------------------------------------------------------- embedding scale
def test_sqrt_d_is_nearest_f32_to_sqrt_768():
    (hidden, hexbits, dec), = read_golden("embed_scale.txt")
    got = oracle.sqrt_d(int(hidden))
    bits = struct.unpack("<I", struct.pack("<f", float(got)))[0]
    assert bits == int(hexbits, 16)
    assert float(got) == float(dec)
    # independent check with exact rationals: no other f32 lies closer to sqrt(768)
    f = Fraction(float(got))
    up = Fraction(float(np.nextafter(np.float32(got), np.float32(np.inf))))
    dn = Fraction(float(np.nextafter(np.float32(got), np.float32(-np.inf))))
    # compare squared distances |f - s| with s^2 = 768 via midpoints: s lies between the midpoints
    assert ((f + dn) / 2) ** 2 < 768 < ((f + up) / 2) ** 2


@pytest.mark.parametrize("d", [1, 2, 3, 256, 768, 896, 5120, 5376, 12345])
def test_sqrt_d_matches_midpoint_bracket(d):
    got = np.float32(oracle.sqrt_d(d))
    f = Fraction(float(got))
    up = Fraction(float(np.nextafter(got, np.float32(np.inf))))
    dn = Fraction(float(np.nextafter(got, np.float32(-np.inf))))
    assert ((f + dn) / 2) ** 2 <= d <= ((f + up) / 2) ** 2


# ---------------------------------------------------------------- gather
def _table(dtype, V, d, seed=0):
    g = np.random.default_rng(seed)
    if dtype == F32:
        return (g.standard_normal((V, d)) * 0.02).astype(np.float32)
    if dtype == BF16:
        x = torch.from_numpy((g.standard_normal((V, d)) * 0.02).astype(np.float32))
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == F16:
        # N(0, 0.02) plus subnormal and extreme binary16 patterns
        h = (g.standard_normal((V, d)) * 0.02).astype(np.float16).view(np.uint16)
        h.reshape(-1)[:6] = [0x0001, 0x03ff, 0x8001, 0x7bff, 0xfbff, 0x8000]
        return h
    nb = d // 32
    out = np.empty((V, nb, 34), np.uint8)
    sc = np.abs(g.standard_normal((V, nb)) * 0.01).astype(np.float16)
    out[:, :, :2] = sc.view(np.uint8).reshape(V, nb, 2)
    out[:, :, 2:] = g.integers(-128, 128, (V, nb, 32)).astype(np.int8).view(np.uint8)
    return out.reshape(V, nb * 34)


def _library_dequant(table, dtype, V, d):
    """Dequantize with library routines only (numpy binary16, torch bfloat16)."""
    if dtype == F32:
        return table.astype(np.float64)
    if dtype == BF16:
        return torch.from_numpy(table.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == F16:
        return table.view(np.float16).astype(np.float64)
    blk = table.reshape(V, d // 32, 34)
    s = blk[:, :, :2].copy().view("<f2").astype(np.float64)          # [V, nb, 1]
    q = blk[:, :, 2:].view(np.int8).astype(np.float64)                # [V, nb, 32]
    return (q * s).reshape(V, d)


@pytest.mark.parametrize("dtype", [F32, BF16, Q8_0, F16])
def test_gather_equals_library_dequant_rows(dtype):
    V, d = 300, 96
    t = _table(dtype, V, d, seed=dtype)
    ids = np.array([0, 299, 5, 5, 17, 299, 0], np.int32)
    out, bad = oracle.embed_gather(t, dtype, V, d, ids)
    ref = _library_dequant(t, dtype, V, d)[ids].astype(np.float32)
    assert bad == 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype", [F32, BF16, Q8_0, F16])
def test_gather_scale_is_one_f32_rounding(dtype):
    V, d = 64, 768
    t = _table(dtype, V, d, seed=10 + dtype)
    ids = np.arange(V, dtype=np.int32)[::-1].copy()
    s = np.float32(math.sqrt(d))
    out, _ = oracle.embed_gather(t, dtype, V, d, ids, scale=s)
    x = _library_dequant(t, dtype, V, d)[ids].astype(np.float32)
    ref = x * s                      # numpy float32 multiply: one IEEE round-to-nearest-even
    assert ref.dtype == np.float32
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    # and it is not the same as multiplying by the scale in a different order for Q8_0
    if dtype == Q8_0:
        blk = t.reshape(V, d // 32, 34)
        sc = blk[:, :, :2].copy().view("<f2").astype(np.float32)
        q = blk[:, :, 2:].view(np.int8).astype(np.float32)
        other = (q * (sc * s)).reshape(V, d)[ids]
        assert not np.array_equal(other.view(np.uint32), out.view(np.uint32))


def test_gather_address_pin_rows_encode_their_id():
    V, d = 4097, 8
    t = np.zeros((V, d), np.float32)
    t[:, :] = np.arange(V, dtype=np.float32)[:, None] * 16 + np.arange(d, dtype=np.float32)
    ids = np.array([4096, 0, 1, 4095, 2048, 1], np.int32)
    out, bad = oracle.embed_gather(t, F32, V, d, ids)
    assert bad == 0
    assert np.array_equal(out, ids[:, None].astype(np.float32) * 16 + np.arange(d, dtype=np.float32))


def test_gather_64bit_offsets_past_2_and_4_gib():
    # 31B-shaped rows (hidden 5376, bf16 -> 10,752 B): id 199,729 starts past 2^31 bytes
    # and id 399,458 past 2^32 bytes.
    d = 5376
    V = 399_460
    rb = 2 * d
    assert 199_729 * rb > 2 ** 31 > 199_728 * rb
    assert 399_458 * rb > 2 ** 32 > 399_457 * rb
    t = np.zeros((V, d), np.uint16)          # calloc'd: only touched rows are backed
    rows = (0, 1, 199_728, 199_729, 199_730, 399_457, 399_458, 399_459)
    for i in rows:
        t[i, :] = 0x3F80 + (i % 64)          # bf16 1 + (i % 64) / 128
    ids = np.array([199_729, 0, 399_458, 199_730, 399_459, 199_728, 1, 399_457], np.int32)
    out, bad = oracle.embed_gather(t, BF16, V, d, ids)
    assert bad == 0
    want = 1.0 + (ids % 64) / 128.0
    assert np.array_equal(out, np.repeat(want[:, None], d, axis=1).astype(np.float32))


def test_gather_bad_ids_zero_rows_and_count():
    V, d = 100, 32
    t = _table(BF16, V, d)
    ids = np.array([3, -1, 100, 2 ** 31 - 1, 99, -(2 ** 31)], np.int32)
    out, bad = oracle.embed_gather(t, BF16, V, d, ids, scale=np.float32(2.0))
    assert bad == 4
    for j in (1, 2, 3, 5):
        assert np.array_equal(out[j].view(np.uint32), np.zeros(d, np.uint32))
    ref = _library_dequant(t, BF16, V, d)
    assert np.array_equal(out[0], (ref[3] * 2).astype(np.float32))
    assert np.array_equal(out[4], (ref[99] * 2).astype(np.float32))


def test_gather_empty():
    t = _table(F32, 10, 8)
    out, bad = oracle.embed_gather(t, F32, 10, 8, np.zeros(0, np.int32))
    assert out.shape == (0, 8) and bad == 0


# ---------------------------------------------------------------- logits
@pytest.mark.parametrize("dtype", [F32, BF16, Q8_0, F16])
def test_logits_match_numpy_float64(dtype):
    V, d, B = 517, 256, 3
    t = _table(dtype, V, d, seed=20 + dtype)
    R = np.random.default_rng(5).standard_normal((B, d)).astype(np.float32)
    L, A = oracle.logits(t, dtype, V, d, R)
    E = _library_dequant(t, dtype, V, d)
    Lref = R.astype(np.float64) @ E.T
    Aref = np.abs(R.astype(np.float64)) @ np.abs(E).T
    assert np.all(np.abs(L - Lref) <= 1e-12 * Aref)
    assert np.allclose(A, Aref, rtol=1e-13, atol=0)


def test_logits_one_hot_residual_selects_a_column_exactly():
    V, d = 300, 64
    t = _table(BF16, V, d, seed=3)
    E = _library_dequant(t, BF16, V, d)
    for j in (0, 17, 63):
        r = np.zeros((1, d), np.float32)
        r[0, j] = 1.0
        L, _ = oracle.logits(t, BF16, V, d, r)
        assert np.array_equal(L[0], E[:, j])


def test_logits_are_not_transposed_or_shifted():
    # a table whose row v is v * e_0 and residual e_0: logits are exactly 0, 1, 2, ...
    V, d = 50, 32
    t = np.zeros((V, d), np.float32)
    t[:, 0] = np.arange(V)
    t[:, 1] = 1000.0            # ignored by the residual below
    r = np.zeros((2, d), np.float32)
    r[0, 0] = 1.0
    r[1, 0] = -2.0
    L, A = oracle.logits(t, F32, V, d, r)
    assert np.array_equal(L[0], np.arange(V, dtype=np.float64))
    assert np.array_equal(L[1], -2.0 * np.arange(V))
    assert np.array_equal(A[1], 2.0 * np.arange(V))


def test_logits_at_matches_full_logits():
    V, d, B = 200, 96, 4
    t = _table(Q8_0, V, d, seed=7)
    R = np.random.default_rng(9).standard_normal((B, d)).astype(np.float32)
    L, A = oracle.logits(t, Q8_0, V, d, R)
    bs = np.array([0, 3, 3, 1])
    vs = np.array([199, 0, 57, 57], np.int32)
    l2, a2 = oracle.logits_at(t, Q8_0, V, d, R, bs, vs)
    assert np.array_equal(l2, L[bs, vs]) and np.array_equal(a2, A[bs, vs])


# ---------------------------------------------------------------- top-k
def test_topk_matches_lexsort_on_random_logits():
    g = np.random.default_rng(11)
    L = g.standard_normal((6, 1000))
    L[2, 10:20] = L[2, 5]                    # ties resolved by the smaller id
    for k in (1, 5, 64):
        ids, sc = oracle.topk(L, k)
        for b in range(L.shape[0]):
            order = np.lexsort((np.arange(L.shape[1]), -L[b]))
            assert np.array_equal(ids[b], order[:k])
            assert np.array_equal(sc[b], L[b, order[:k]].astype(np.float32))


def test_topk_k1_is_argmax():
    g = np.random.default_rng(12)
    L = np.round(g.standard_normal((5, 300)), 1)       # many exact ties
    ids, _ = oracle.topk(L, 1)
    assert np.array_equal(ids[:, 0], np.argmax(L, axis=1))


def test_zero_residual_gives_first_k_ids():
    V, d = 40, 32
    t = _table(BF16, V, d, seed=1)
    L, _ = oracle.logits(t, BF16, V, d, np.zeros((1, d), np.float32))
    ids, sc = oracle.topk(L, 7)
    assert np.array_equal(ids[0], np.arange(7))
    assert np.all(sc == 0)


def test_negative_zero_ties_with_positive_zero():
    L = np.array([[-0.0, 0.0, -1.0, -0.0, 0.0]])
    ids, _ = oracle.topk(L, 4)
    assert np.array_equal(ids[0], [0, 1, 3, 4])


def test_duplicate_rows_rank_by_id():
    V, d = 64, 32
    t = _table(F32, V, d, seed=4) * 0.01
    r = np.random.default_rng(6).standard_normal((1, d)).astype(np.float32)
    best = (r[0] / np.linalg.norm(r[0])).astype(np.float32)
    for v in (41, 3, 17):
        t[v] = best
    L, _ = oracle.logits(t, F32, V, d, r)
    ids, _ = oracle.topk(L, 3)
    assert np.array_equal(ids[0], [3, 17, 41])


def test_planted_winners_come_out_in_order():
    V, d = 2000, 128
    t = _table(F32, V, d, seed=8)
    r = np.random.default_rng(13).standard_normal((1, d)).astype(np.float32)
    u = r[0] / np.linalg.norm(r[0])
    planted = [1234, 7, 1999, 512]
    for j, v in enumerate(planted):
        t[v] = (u * (10.0 - j)).astype(np.float32)
    L, _ = oracle.logits(t, F32, V, d, r)
    ids, _ = oracle.topk(L, 4)
    assert list(ids[0]) == planted


def test_permuting_rows_permutes_ids():
    V, d = 500, 64
    t = _table(BF16, V, d, seed=14)
    R = np.random.default_rng(15).standard_normal((2, d)).astype(np.float32)
    perm = np.random.default_rng(16).permutation(V)
    L1, _ = oracle.logits(t, BF16, V, d, R)
    L2, _ = oracle.logits(t[perm], BF16, V, d, R)
    assert np.array_equal(L2, L1[:, perm])
    i1, _ = oracle.topk(L1, 10)
    i2, _ = oracle.topk(L2, 10)
    inv = np.argsort(perm)
    assert np.array_equal(inv[i1], i2)


# ---------------------------------------------------------------- probabilities
def test_uniform_logits_give_one_over_v():
    for V in (1, 7, 262144):
        L = np.zeros((1, V))
        assert oracle.log_partition(L, 1.0)[0] == pytest.approx(math.log(V), rel=0, abs=1e-12)
        p = oracle.probs_at(L, [[0]], 0.37)
        assert p[0, 0] == pytest.approx(1.0 / V, rel=1e-12)


def test_two_token_probabilities_are_logistic():
    # p(v0) = 1 / (1 + exp((L1 - L0) / T)); a temperature that multiplied instead
    # of dividing, or a dropped shift, would miss it
    for l0, l1, T in ((0.3, -1.2, 1.0), (2.0, 5.0, 2.5), (-7.0, -7.5, 0.25), (1000.0, 999.0, 1.0)):
        L = np.array([[l0, l1]])
        p = oracle.probs_at(L, [[0, 1]], T)
        want0 = 1.0 / (1.0 + math.exp((l1 - l0) / T))
        assert p[0, 0] == pytest.approx(want0, rel=1e-13)
        assert p[0, 1] == pytest.approx(1.0 - want0, rel=1e-12)


def test_probabilities_of_log_weights_are_the_weights():
    w = np.array([1.0, 2.0, 3.0, 4.0, 10.0])
    L = np.log(w)[None, :]
    p = oracle.probs_at(L, [[4, 3, 2, 1, 0]], 1.0)
    assert np.allclose(p[0], w[::-1] / w.sum(), rtol=1e-13, atol=0)
    # at T = 1/2 the weights are squared
    p2 = oracle.probs_at(L, [[4, 0]], 0.5)
    assert np.allclose(p2[0], np.array([100.0, 1.0]) / (w ** 2).sum(), rtol=1e-13, atol=0)


def test_log_partition_matches_scipy_and_probabilities_sum_to_one():
    from scipy.special import logsumexp
    g = np.random.default_rng(31)
    L = g.standard_normal((3, 5000)) * 4.0 + 50.0          # shifted: a naive sum would still fit,
    for T in (0.3, 1.0, 7.0):                               # the shift must cancel exactly
        lse = oracle.log_partition(L, T)
        assert np.allclose(lse, logsumexp(L / T, axis=1), rtol=1e-13, atol=0)
        p = oracle.probs_at(L, np.tile(np.arange(5000, dtype=np.int32), (3, 1)), T)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_large_logits_do_not_overflow():
    L = np.array([[800.0, 799.0, -800.0]])
    p = oracle.probs_at(L, [[0, 1, 2]], 1.0)
    e = math.exp(-1.0)
    assert p[0, 0] == pytest.approx(1.0 / (1.0 + e), rel=1e-13)
    assert p[0, 1] == pytest.approx(e / (1.0 + e), rel=1e-12)
    assert 0.0 <= p[0, 2] < 1e-300


def test_probability_check_accepts_oracle_and_rejects_shifted():
    V, d = 300, 64
    t = _table(BF16, V, d, seed=19)
    R = np.random.default_rng(20).standard_normal((2, d)).astype(np.float32)
    L, A = oracle.logits(t, BF16, V, d, R)
    ids, _ = oracle.topk(L, 5)
    for T in (0.5, 1.0):
        p = oracle.probs_at(L, ids, T)
        assert accept.check_probs(ids, p, T, 2e-3, L, A) == []
        # beyond the logit tolerance: a probability off by a factor e^(3 max tol / T)
        off = p * np.exp(3.0 * 2e-3 * A.max() / T)
        assert accept.check_probs(ids, off, T, 2e-3, L, A)


# ---------------------------------------------------------------- wire codecs
def _f16_edge_values():
    g = np.random.default_rng(33)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** g.integers(-9, 5, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.0, 65520.0, 1e30, -1e30, 6.1035156e-05,
                  5.9604645e-08, 2.9802322e-08, 2.9802326e-08, 8.940697e-08, 1e-45, 3.4028235e38,
                  1.0009766, 1.0004883, 1.0014648, -2048.5, 2049.0, 4097.0], np.float32)])
    # exact halfway points between neighbouring binary16 values (ties to even)
    h = np.arange(0x0000, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    return np.concatenate([x, mid, -mid])


def test_f16_encoder_matches_numpy_with_saturation():
    x = _f16_edge_values()
    got = np.array([oracle.f32_to_f16_sat(v) for v in x], np.uint16)
    want = np.clip(x, -65504, 65504).astype(np.float16).view(np.uint16)   # numpy: round to nearest even
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_f16_wire_round_trip():
    x = _f16_edge_values()[None, :5000]
    enc = oracle.wire_encode(x, oracle.WIRE_F16)
    assert enc.shape == (1, 2 * 5000)
    assert np.array_equal(enc.view(np.uint16)[0], np.clip(x[0], -65504, 65504).astype(np.float16).view(np.uint16))
    dec = oracle.wire_decode(enc, 5000, oracle.WIRE_F16)
    assert np.array_equal(dec, np.clip(x, -65504, 65504).astype(np.float16).astype(np.float32))


def test_i8_wire_hand_worked_row():
    # max |x| = 127 -> scale 1; codes round half to even: -63.5 -> -64, 0.5 -> 0, 2.5 -> 2
    x = np.array([[127, -63.5, 0.5, 2.5, -0.49, 0, 126.5, -127]], np.float32)
    enc = oracle.wire_encode(x, oracle.WIRE_I8)
    assert enc.shape == (1, 8 + 8)
    assert enc[0, :4].view(np.float32)[0] == 1.0 and enc[0, 4:8].view(np.float32)[0] == 0.0
    assert enc[0, 8:].view(np.int8).tolist() == [127, -64, 0, 2, 0, 0, 126, -127]
    # max 254 -> scale 2
    enc = oracle.wire_encode(np.array([[254.0, 1.0, -3.0, 5.0]], np.float32), oracle.WIRE_I8)
    assert enc[0, :4].view(np.float32)[0] == 2.0
    assert enc[0, 8:].view(np.int8).tolist() == [127, 0, -2, 2]
    dec = oracle.wire_decode(enc, 4, oracle.WIRE_I8)
    assert dec.tolist() == [[254.0, 0.0, -4.0, 4.0]]


def test_i8_wire_zero_row_and_scale_in_f32():
    enc = oracle.wire_encode(np.zeros((2, 16), np.float32), oracle.WIRE_I8)
    assert np.all(enc == 0)
    g = np.random.default_rng(34)
    x = g.standard_normal((5, 333)).astype(np.float32) * np.float32([[1e-3], [1.0], [7.0], [1e4], [3e-30]])
    enc = oracle.wire_encode(x, oracle.WIRE_I8)
    for r in range(5):
        m = np.max(np.abs(x[r]))
        scale = np.float32(m) / np.float32(127.0)                 # numpy f32 division
        assert enc[r, :4].view(np.float32)[0] == scale
        q = np.clip(np.rint(x[r] / scale), -127, 127)             # numpy f32 division, round half even
        assert np.array_equal(enc[r, 8:].view(np.int8), q.astype(np.int8))
        dec = oracle.wire_decode(enc[r:r + 1], 333, oracle.WIRE_I8)[0]
        assert np.array_equal(dec, q.astype(np.float32) * scale)
        assert np.all(np.abs(dec.astype(np.float64) - x[r]) <= 0.5 * scale * (1 + 1e-6) + 1e-45)


# ---------------------------------------------------------------- acceptance rule
def test_acceptance_rule_accepts_exact_and_rejects_wrong():
    V, d = 300, 64
    t = _table(BF16, V, d, seed=17)
    R = np.random.default_rng(18).standard_normal((2, d)).astype(np.float32)
    L, A = oracle.logits(t, BF16, V, d, R)
    ids, sc = oracle.topk(L, 5)
    assert accept.check_full(ids, sc, L, A, ids, 2e-3) == []
    bad = ids.copy()
    bad[0, 0] = np.argmin(L[0])                        # a clearly wrong id
    assert accept.check_full(bad, sc, L, A, ids, 2e-3)
    dup = ids.copy()
    dup[1, 1] = dup[1, 0]
    assert accept.check_full(dup, sc, L, A, ids, 2e-3)
    inc = sc.copy()
    inc[0] = inc[0][::-1]
    assert accept.check_full(ids, inc, L, A, ids, 2e-3)
