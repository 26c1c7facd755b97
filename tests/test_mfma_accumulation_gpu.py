"""The matrix cores' f32 accumulation against the bound the rank path assumes.

The rank path's certificate assumes that accumulating the exact products of
bf16 operands in f32 on the matrix cores stays within kpad * 2^-22 *
sum_i |r_i e_i| of the exact sum (four unit roundoffs per term).  These tests
feed residual rows that are exactly bf16 (so the lo half of the split is zero
and every difference from the oracle's f64 logits is accumulation error)
through the raw logits of the three MFMA kernels.  The table rows are built to
hurt an accumulator: long runs of same-sign products that cancel (partial sums
far above the result), one large product among tiny ones in every group of 16
(alignment of the small ones to the large one), and random rows.  The observed
errors are reported as multiples of d * 2^-24 * sum|r e|; the assertion is the
assumed bound.
"""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from tests.gpu_util import note, table, to_dev

pytestmark = pytest.mark.gpu


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _adversarial_table(V, d, seed):
    g = np.random.default_rng(seed)
    E = np.empty((V, d), np.float32)
    n = V // 4
    # runs of equal sign: partial sums climb to ~d/2 then return towards 0
    for v in range(n):
        run = 1 << (4 + v % 8)
        sign = np.where((np.arange(d) // run) % 2 == 0, 1.0, -1.0)
        E[v] = sign * (1.0 + g.random(d).astype(np.float32))
    # one large value per group of 16 (K step of the matrix cores), the rest tiny
    for v in range(n, 2 * n):
        x = g.standard_normal(d).astype(np.float32) * np.float32(2.0 ** -12)
        x[(v % 16)::16] = g.standard_normal(d // 16).astype(np.float32) * np.float32(2.0 ** 10)
        E[v] = x
    # wide exponent range across the row
    for v in range(2 * n, 3 * n):
        E[v] = g.standard_normal(d).astype(np.float32) * np.exp2(g.integers(-20, 20, d)).astype(np.float32)
    E[3 * n:] = g.standard_normal((V - 3 * n, d)).astype(np.float32) * np.float32(0.02)
    return _bf16(E)


@pytest.mark.parametrize("path,B", [(etg.PATH_GEMM, 70), (etg.PATH_WIDE, 17), (etg.PATH_STREAM, 8)])
@pytest.mark.parametrize("d", [512, 5120])
def test_matrix_core_accumulation_within_the_assumed_bound(path, B, d):
    V = 1024
    host = _adversarial_table(V, d, seed=3000 + d)
    g = np.random.default_rng(4000 + d)
    R = _f(_bf16(np.where(g.random((B, d)) < 0.5, 1.0, -1.0) * (1.0 + g.random((B, d)))))
    R[0] = 1.0                                          # every product of row 0 is its table value
    R[1] = _f(_bf16(np.abs(_f(host[0]))))               # aligned with the run-of-signs row 0
    t = table(host, etg.BF16, V, d)
    note(f"mfma accumulation path={path} B={B} d={d}")
    raw = t.logits_raw(to_dev(R), path=path)
    torch.cuda.synchronize()
    raw = raw.cpu().numpy().astype(np.float64)
    L, A = oracle.logits(host, etg.BF16, V, d, R)
    kpad = -(-d // 64) * 64
    err = np.abs(raw - L)
    bound = kpad * 2.0 ** -22 * A + 2.0 ** -100
    worst = float(np.max(err / (d * 2.0 ** -24 * A + 1e-300)))
    print(f"path {path} d {d}: worst error = {worst:.3f} x d 2^-24 sum|r e| (assumed at most 4)")
    assert np.all(err <= bound), f"accumulation error {worst:.2f} x d u exceeds the assumed 4 x d u"
