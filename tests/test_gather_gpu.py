"""embed_gather on the GPU against the CPU oracle: bit-exact, every dtype and edge case."""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from tests.gpu_util import bits, ids_dev, note, table

pytestmark = pytest.mark.gpu

F32, BF16, Q8_0, F16 = etg.F32, etg.BF16, etg.Q8_0, etg.F16


def _gather_both(host, dtype, V, d, ids, scaled):
    t = table(host, dtype, V, d)
    note(f"gather dtype={dtype} V={V} d={d} n={ids.size} scaled={scaled}")
    out = t.embed_gather(ids_dev(ids), scale="sqrt_d" if scaled else None, check=False)
    torch.cuda.synchronize()
    ref, nbad = oracle.embed_gather(host, dtype, V, d, ids, scale=oracle.sqrt_d(d) if scaled else None)
    return out, ref, nbad


@pytest.mark.parametrize("name", ["tiny", "qwen05b", "gemma_embed"])
@pytest.mark.parametrize("scaled", [False, True])
def test_gather_configs_bit_exact(name, scaled):
    cfg = synth.CONFIGS[name]
    host = cfg.table()
    ids = cfg.ids()
    out, ref, nbad = _gather_both(host, cfg.dtype, cfg.V, cfg.d, ids, scaled)
    assert nbad == 0
    assert out.shape == (ids.size, cfg.d)
    assert np.array_equal(bits(out), bits(ref))


def test_scale_constants_agree():
    for d in (256, 768, 896, 5120, 5376, 3):
        assert np.float32(etg.sqrt_d(d)) == oracle.sqrt_d(d)


@pytest.mark.parametrize("dtype,d", [(F32, 4), (F32, 100), (BF16, 8), (BF16, 200), (BF16, 896),
                                     (Q8_0, 32), (Q8_0, 96), (Q8_0, 768), (Q8_0, 896), (Q8_0, 4096),
                                     (F16, 8), (F16, 200), (F16, 2560)])
@pytest.mark.parametrize("n", [1, 65, 1000])
def test_gather_shapes_bit_exact(dtype, d, n):
    V = 3001
    host = synth.make_table(dtype, V, d, seed=50 + d)
    ids = synth.uniform_ids(n, V, seed=60 + n)
    ids[0] = V - 1
    if n > 2:
        ids[1] = 0
    for scaled in (False, True):
        out, ref, nbad = _gather_both(host, dtype, V, d, ids, scaled)
        assert nbad == 0
        assert np.array_equal(bits(out), bits(ref))


# Q8_0 rows that are not whole 16-byte chunks are staged through LDS in pieces of
# 64 blocks: a row of 257 blocks (the last piece has one block), 513 and 2,047
# blocks (the widest row, 69,598 bytes); odd block counts put every other row
# start 2 bytes past a dword boundary
@pytest.mark.parametrize("d", [8224, 16416, 65504])
def test_gather_long_q8_rows_bit_exact(d):
    V = 67
    host = synth.make_table(Q8_0, V, d, seed=70 + d)
    ids = np.array([0, 66, 1, 65, 33, 2, 3, 34, 66, -1, 5], np.int32)
    for scaled in (False, True):
        out, ref, nbad = _gather_both(host, Q8_0, V, d, ids, scaled)
        assert nbad == 1
        assert np.array_equal(bits(out), bits(ref))


def test_gather_more_rows_than_one_launch():
    # 2^24 + 5 ids: the gather is split into two launches (at most 2^24 rows each);
    # rows on both sides of the split, and the bad-id count over both
    V, d = 1000, 4
    n = (1 << 24) + 5
    host = synth.make_table(F32, V, d, seed=71)
    ids = synth.uniform_ids(n, V, seed=72)
    ids[(1 << 24) - 1] = -7
    ids[1 << 24] = V
    t = table(host, F32, V, d)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"gather n={n} in two launches")
    out = t.embed_gather(ids_dev(ids), scale="sqrt_d", bad_count=cnt, check=False)
    torch.cuda.synchronize()
    ref, nbad = oracle.embed_gather(host, F32, V, d, ids, scale=oracle.sqrt_d(d))
    assert int(cnt.item()) == nbad == 2
    assert np.array_equal(bits(out), bits(ref))
    del out
    torch.cuda.empty_cache()


def test_gather_special_values_bit_exact():
    # subnormal, huge and signed-zero inputs through every dtype
    V, d = 8, 64
    f = np.zeros((V, d), np.float32)
    f[0, :4] = [1e-45, -1e-45, 1.1754942e-38, -0.0]
    f[1, :4] = [3.4028235e38, -3.4028235e38, 1.0, -1.0]
    f[2] = np.linspace(-5, 5, d, dtype=np.float32)
    b = synth.f32_to_bf16_bits(f)
    b[3, :4] = [0x0001, 0x8001, 0x7F7F, 0x8000]          # bf16 subnormals, max finite, -0
    q = synth.q8_0_table(V, d, seed=3)
    blk = q.reshape(V, 2, 34)
    blk[0, 0, :2] = [0x01, 0x00]                          # scale = smallest f16 subnormal
    blk[0, 1, :2] = [0xFF, 0x7B]                          # scale = 65504
    blk[0, 0, 2:4] = np.array([-128, 127], np.int8).view(np.uint8)
    blk[0, 1, 2:4] = np.array([-128, 127], np.int8).view(np.uint8)
    blk[1, 0, :2] = [0x00, 0x80]                          # scale = -0
    h = np.clip(f, -60000, 60000).astype(np.float16).view(np.uint16)
    h[0, :6] = [0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x8000]  # subnormals, max finite, -0
    h[1, :2] = [0x0400, 0x3C00]                           # smallest normal, 1.0
    h[2] = np.linspace(-5, 5, d, dtype=np.float32).astype(np.float16).view(np.uint16)
    ids = np.arange(V, dtype=np.int32)
    for host, dt in ((f, F32), (b, BF16), (q, Q8_0), (h, F16)):
        for scaled in (False, True):
            out, ref, _ = _gather_both(host, dt, V, d, ids, scaled)
            assert np.array_equal(bits(out), bits(ref)), (dt, scaled)


# d = 96: 102-byte rows (2-byte aligned path); d = 256: 272-byte rows (16-byte
# aligned path, two rows per wave, 7 ids so the last wave has one)
@pytest.mark.parametrize("d", [96, 256])
def test_gather_bad_ids_zero_and_count(d):
    V = 500
    host = synth.make_table(Q8_0, V, d, seed=7)
    ids = np.array([3, -1, 500, 2 ** 31 - 1, 499, -(2 ** 31), 0], np.int32)
    t = table(host, Q8_0, V, d)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    note("gather bad ids")
    out = t.embed_gather(ids_dev(ids), scale="sqrt_d", bad_count=cnt, check=False)
    torch.cuda.synchronize()
    ref, nbad = oracle.embed_gather(host, Q8_0, V, d, ids, scale=oracle.sqrt_d(d))
    assert int(cnt.item()) == nbad == 4
    assert np.array_equal(bits(out), bits(ref))
    with pytest.raises(ValueError, match="bad token id"):
        t.embed_gather(ids_dev(ids))


def test_gather_empty():
    host = synth.make_table(BF16, 10, 64, seed=1)
    t = table(host, BF16, 10, 64)
    out = t.embed_gather(torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 64)


def test_gather_offsets_past_2_and_4_gib():
    # 31B-shaped rows (10,752 bytes): rows past 2^31 and 2^32 bytes, on a zeroed table.
    d, V = 5376, 399_460
    rows = (0, 1, 199_728, 199_729, 199_730, 399_457, 399_458, 399_459)
    note("gather 64-bit offsets, 4.3 GB table")
    dev = torch.zeros((V, d), dtype=torch.int16, device="cuda")
    host = np.zeros((V, d), np.uint16)
    for i in rows:
        val = 0x3F80 + (i % 64) + 16 * (i % 3)
        host[i, :] = val
        dev[i, :] = val
    t = etg.Table(dev, BF16, V, d)
    ids = np.array([199_729, 0, 399_458, 199_730, 399_459, 199_728, 1, 399_457], np.int32)
    out = t.embed_gather(ids_dev(ids), check=False)
    torch.cuda.synchronize()
    ref, _ = oracle.embed_gather(host, BF16, V, d, ids)
    assert np.array_equal(bits(out), bits(ref))
    del t, dev
    torch.cuda.empty_cache()


def test_gather_repeatable():
    cfg = synth.CONFIGS["gemma_embed"]
    host = cfg.table()
    ids = ids_dev(cfg.ids())
    t = table(host, cfg.dtype, cfg.V, cfg.d)
    note("gather repeat x10")
    first = t.embed_gather(ids, scale="sqrt_d", check=False).clone()
    for _ in range(10):
        again = t.embed_gather(ids, scale="sqrt_d", check=False)
        assert torch.equal(first.view(torch.int32), again.view(torch.int32))


def _random_gathers(n, seed):
    rng = np.random.default_rng(seed)
    step = {F32: 4, BF16: 8, F16: 8, Q8_0: 32}
    out = []
    for i in range(n):
        dt = [F32, BF16, F16, Q8_0][int(rng.integers(4))]
        d = int(rng.integers(1, 2048 // step[dt] + 1)) * step[dt]
        V = int(rng.choice([1, 2, 17, int(rng.integers(3, 5000))]))
        cnt = int(rng.choice([1, 63, 64, 65, int(rng.integers(2, 3000))]))
        out.append((i, dt, V, d, cnt, int(rng.integers(3))))
    return out


@pytest.mark.parametrize("i,dtype,V,d,n,scale_kind", _random_gathers(30, 41))
def test_gather_random_shapes_bit_exact(i, dtype, V, d, n, scale_kind):
    # seeded random tables, widths and id lists with some ids out of range: rows and
    # the bad-id count bit-exact against the oracle, with no scale, x sqrt(d), or an
    # arbitrary f32 scale
    rng = np.random.default_rng(4000 + i)
    host = synth.make_table(dtype, V, d, seed=4100 + i)
    ids = rng.integers(-2, V + 2, size=n).astype(np.int32)
    scale = [None, "sqrt_d", float(np.float32(rng.uniform(-3, 3)))][scale_kind]
    oscale = None if scale is None else oracle.sqrt_d(d) if scale == "sqrt_d" else np.float32(scale)
    t = table(host, dtype, V, d)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"gather random i={i} dtype={dtype} V={V} d={d} n={n} scale={scale}")
    out = t.embed_gather(ids_dev(ids), scale=scale, bad_count=cnt, check=False)
    torch.cuda.synchronize()
    ref, nbad = oracle.embed_gather(host, dtype, V, d, ids, scale=oscale)
    assert int(cnt.item()) == nbad
    assert np.array_equal(bits(out), bits(ref))
