"""Seeded synthetic inputs for the static embedding / tied lm_head path.

This module only *makes* inputs: tables in their storage encodings, token-id
streams and residuals.  It holds none of the method's arithmetic (no dequant,
no gather, no dot products, no selection), so both the CPU oracle and the HIP
library can be fed from it without sharing any of the computation.

Workload shapes follow the pages:

* the row-addressed table (``row i`` at byte offset ``i * row_bytes``) of the
  HELIX Columnar Embedding proposal, section 3 "Wire format" / "Index";
* the sparse access of that proposal's section 2 "Insight" (628 tokens of a
  long-context prompt touch 109 distinct vocabulary ids);
* the EmbeddingGemma Q8_0 ``token_embd [768, 262144]`` table of the
  embeddinggemma.c port specification ("Tensor inventory"), with 32-value
  blocks of int8 and one f16 scale;
* the 262,144 x 5,376 tied lm_head of ADR-0008 ("POST /v1/logits").

Real weights, tokenizers and evaluation text are not available; every array
here is drawn from a seeded numpy PCG64 generator.  Large tables are drawn in
fixed row chunks, each with its own child seed, so the bytes do not depend on
the number of worker threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Storage dtype codes (the same small integers are used by both sides'
# public interfaces; each side defines them on its own).
F32, BF16, Q8_0, F16 = 0, 1, 2, 3
DTYPE_NAMES = {F32: "f32", BF16: "bf16", Q8_0: "q8_0", F16: "f16"}

Q8_BLOCK = 32          # values per Q8_0 block
Q8_BLOCK_BYTES = 34    # 2-byte f16 scale + 32 int8 values

_CHUNK_ROWS = 4096     # rows per independently seeded chunk


def storage_row_bytes(dtype: int, d: int) -> int:
    """Bytes of one stored row (used only to size buffers)."""
    if dtype == F32:
        return 4 * d
    if dtype in (BF16, F16):
        return 2 * d
    if dtype == Q8_0:
        return Q8_BLOCK_BYTES * (d // Q8_BLOCK)
    raise ValueError(f"unknown dtype {dtype}")


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite float32 values as bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _chunked(V: int, fill, out: np.ndarray, seed: int) -> np.ndarray:
    nchunks = (V + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    seeds = np.random.SeedSequence(seed).spawn(max(nchunks, 1))

    def job(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(V, r0 + _CHUNK_ROWS)
        fill(np.random.Generator(np.random.PCG64(seeds[c])), out[r0:r1])

    if nchunks <= 1:
        for c in range(nchunks):
            job(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, range(nchunks)))
    return out


def normal_f32_table(V: int, d: int, std: float, seed: int) -> np.ndarray:
    """float32 [V, d] with entries N(0, std^2)."""
    out = np.empty((V, d), np.float32)

    def fill(g, blk):
        g.standard_normal(out=blk, dtype=np.float32)
        blk *= np.float32(std)

    return _chunked(V, fill, out, seed)


def normal_bf16_table(V: int, d: int, std: float, seed: int) -> np.ndarray:
    """bfloat16 bit patterns (uint16 [V, d]) of N(0, std^2) float32 draws."""
    out = np.empty((V, d), np.uint16)

    def fill(g, blk):
        tmp = g.standard_normal(size=blk.shape, dtype=np.float32)
        tmp *= np.float32(std)
        blk[...] = f32_to_bf16_bits(tmp)

    return _chunked(V, fill, out, seed)


def normal_f16_table(V: int, d: int, std: float, seed: int) -> np.ndarray:
    """binary16 bit patterns (uint16 [V, d]) of N(0, std^2) float32 draws (numpy's
    round-to-nearest-even conversion)."""
    out = np.empty((V, d), np.uint16)

    def fill(g, blk):
        tmp = g.standard_normal(size=blk.shape, dtype=np.float32)
        tmp *= np.float32(std)
        blk[...] = tmp.astype(np.float16).view(np.uint16)

    return _chunked(V, fill, out, seed)


def q8_0_table(V: int, d: int, seed: int, scale_std: float = 0.01,
               qlo: int = -127, qhi: int = 127) -> np.ndarray:
    """Q8_0 rows (uint8 [V, 34*d/32]).

    Each 32-value block is stored as a little-endian f16 scale followed by 32
    int8 values; blocks follow each other along the row and rows are
    contiguous.  Values are uniform integers in [qlo, qhi]; scales are the f16
    rounding of |N(0, scale_std^2)|.
    """
    if d % Q8_BLOCK:
        raise ValueError("Q8_0 rows need d to be a multiple of 32")
    nb = d // Q8_BLOCK
    out = np.empty((V, nb, Q8_BLOCK_BYTES), np.uint8)

    def fill(g, blk):
        n = blk.shape[0]
        sc = np.abs(g.standard_normal(size=(n, nb)) * scale_std).astype(np.float16)
        q = g.integers(qlo, qhi + 1, size=(n, nb, Q8_BLOCK), dtype=np.int16).astype(np.int8)
        blk[:, :, 0:2] = sc.astype("<f2").view(np.uint8).reshape(n, nb, 2)
        blk[:, :, 2:] = q.view(np.uint8)

    _chunked(V, fill, out, seed)
    return out.reshape(V, nb * Q8_BLOCK_BYTES)


def make_table(dtype: int, V: int, d: int, seed: int, std: float = 0.02) -> np.ndarray:
    if dtype == F32:
        return normal_f32_table(V, d, std, seed)
    if dtype == BF16:
        return normal_bf16_table(V, d, std, seed)
    if dtype == Q8_0:
        return q8_0_table(V, d, seed)
    if dtype == F16:
        return normal_f16_table(V, d, std, seed)
    raise ValueError(f"unknown dtype {dtype}")


def uniform_ids(n: int, V: int, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    return g.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def _zipf_ranks(g: np.random.Generator, n: int, S: int, s: float) -> np.ndarray:
    """0-based ranks from a Zipf law truncated to S ranks: P(r) proportional to (r+1)^-s."""
    w = np.arange(1, S + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, g.random(n), side="right"), S - 1)


def zipf_ids(n: int, V: int, seed: int, s: float = 1.1, support: int | None = None,
             cover_support: bool = False) -> np.ndarray:
    """Token ids with a Zipf(s) rank law, ranks mapped to ids by a seeded permutation of [0, V).

    ``support`` truncates the law to that many ranks (default: all V ids).
    With ``cover_support`` every rank of the support appears at least once
    (each once, then n - support Zipf draws, shuffled), so the stream has
    exactly ``support`` distinct ids.
    """
    g = np.random.default_rng(seed)
    S = V if support is None else support
    perm = g.permutation(V)
    if cover_support:
        if n < S:
            raise ValueError("cover_support needs n >= support")
        ranks = np.concatenate([np.arange(S), _zipf_ranks(g, n - S, S, s)])
        g.shuffle(ranks)
    else:
        ranks = _zipf_ranks(g, n, S, s)
    return perm[ranks].astype(np.int32)


def residuals(B: int, d: int, seed: int) -> np.ndarray:
    """float32 [B, d] residual rows, N(0, 1)."""
    g = np.random.default_rng(seed)
    return g.standard_normal(size=(B, d), dtype=np.float32)


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    dtype: int
    V: int
    d: int
    gather_n: int = 0              # 0: no gather in this workload
    gather_ids: str = "uniform"    # "uniform" | "zipf" | "zipf_cover"
    zipf_support: int | None = None
    gather_scale: bool = False     # multiply by f32(sqrt(d))
    batches: tuple = field(default_factory=tuple)
    k: int = 0

    @property
    def table_seed(self) -> int:
        return 1000 + self.index

    @property
    def ids_seed(self) -> int:
        return 2000 + self.index

    def residual_seed(self, B: int) -> int:
        return 3000 + self.index + 7919 * B

    @property
    def row_bytes(self) -> int:
        return storage_row_bytes(self.dtype, self.d)

    @property
    def table_bytes(self) -> int:
        return self.V * self.row_bytes

    def table(self) -> np.ndarray:
        return make_table(self.dtype, self.V, self.d, self.table_seed)

    def ids(self) -> np.ndarray:
        if self.gather_ids == "uniform":
            return uniform_ids(self.gather_n, self.V, self.ids_seed)
        if self.gather_ids == "zipf":
            return zipf_ids(self.gather_n, self.V, self.ids_seed, 1.1, self.zipf_support)
        if self.gather_ids == "zipf_cover":
            return zipf_ids(self.gather_n, self.V, self.ids_seed, 1.1, self.zipf_support, True)
        raise ValueError(self.gather_ids)

    def residuals(self, B: int) -> np.ndarray:
        return residuals(B, self.d, self.residual_seed(B))


CONFIGS = {
    # f32 table V=4096 d=256 N(0,0.02); gather 64 uniform ids; logits + top-5 for 4 residuals
    "tiny": Config(1, "tiny", F32, 4096, 256, gather_n=64, gather_ids="uniform",
                   batches=(4,), k=5),
    # bf16 table 151,936 x 896 (Qwen2.5-0.5B shape); 628 Zipf(1.1) ids over exactly 109
    # distinct rows; logits + top-10 for one residual
    "qwen05b": Config(2, "qwen05b", BF16, 151936, 896, gather_n=628, gather_ids="zipf_cover",
                      zipf_support=109, batches=(1,), k=10),
    # Q8_0 table 262,144 x 768 (EmbeddingGemma shape); 32 x 512 Zipf(1.1) ids, x sqrt(768)
    "gemma_embed": Config(3, "gemma_embed", Q8_0, 262144, 768, gather_n=32 * 512,
                          gather_ids="zipf", gather_scale=True),
    # bf16 tied lm_head 262,144 x 5,376; logits + top-10 for batches of 1, 8, 64
    "lm31b": Config(4, "lm31b", BF16, 262144, 5376, batches=(1, 8, 64), k=10),
    # bf16 262,144 x 5,120; logits + top-40 for 1,024 residuals (dense contraction)
    "prefill": Config(5, "prefill", BF16, 262144, 5120, batches=(1024,), k=40),
    # the 31B-shaped lm_head stored as Q8_0 (1.50 GB; a timed Q8_0 lm_head): int8 uniform
    # [-127, 127], f16(|N(0, 0.01)|) scales as for gemma_embed; logits + top-10, B = 1, 2, 8
    "lm31b_q8": Config(6, "lm31b_q8", Q8_0, 262144, 5376, batches=(1, 2, 8), k=10),
}

