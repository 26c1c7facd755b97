"""The seeded input generators: determinism and the workload shapes they promise."""
import numpy as np
import torch

import synth


def test_bf16_encoding_matches_torch_round_to_nearest_even():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100_000).astype(np.float32) * 0.02,
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], np.float32)])
    got = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_tables_are_deterministic_and_chunk_independent():
    a = synth.normal_bf16_table(9000, 64, 0.02, 7)
    b = synth.normal_bf16_table(9000, 64, 0.02, 7)
    assert np.array_equal(a, b)
    c = synth.normal_bf16_table(9000, 64, 0.02, 8)
    assert not np.array_equal(a, c)


def test_q8_0_layout_and_ranges():
    t = synth.q8_0_table(5000, 96, 3)
    assert t.shape == (5000, 3 * 34) and t.dtype == np.uint8
    blk = t.reshape(5000, 3, 34)
    s = blk[:, :, :2].copy().view("<f2").astype(np.float64)
    q = blk[:, :, 2:].view(np.int8)
    assert np.all(s >= 0) and 0.005 < s.mean() < 0.011      # |N(0, 0.01)| has mean 0.008
    assert q.min() == -127 and q.max() == 127


def test_qwen_stream_has_exactly_109_distinct_ids():
    cfg = synth.CONFIGS["qwen05b"]
    ids = cfg.ids()
    assert ids.shape == (628,) and ids.dtype == np.int32
    assert np.unique(ids).size == 109
    assert ids.min() >= 0 and ids.max() < cfg.V
    # Zipf: the most frequent id takes a large share
    _, counts = np.unique(ids, return_counts=True)
    assert counts.max() > 60


def test_gemma_stream_is_zipf_over_the_whole_vocab():
    cfg = synth.CONFIGS["gemma_embed"]
    ids = cfg.ids()
    assert ids.shape == (16384,)
    u = np.unique(ids).size
    assert 4000 < u < 6500            # about 5,000 distinct ids for 16,384 Zipf(1.1) draws
    assert ids.min() >= 0 and ids.max() < cfg.V
    assert np.array_equal(ids, cfg.ids())


def test_config_sizes():
    c = synth.CONFIGS
    assert c["lm31b"].table_bytes == 2_818_572_288
    assert c["prefill"].table_bytes == 2_684_354_560
    assert c["qwen05b"].table_bytes == 272_269_312
    assert c["gemma_embed"].row_bytes == 816
    assert c["tiny"].table_bytes == 4 * 1024 * 1024
