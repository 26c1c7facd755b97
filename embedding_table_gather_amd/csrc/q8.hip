// Q8_0 stream path of the lm_head projection: ADR-0008 "POST /v1/logits",
// logits = residual @ lm_head.T over every vocabulary row, for a table stored in
// Q8_0 blocks (32 int8 values after a binary16 scale, 34 bytes; the
// embeddinggemma.c port specification, "Tensor inventory"), fused with a
// per-block top-k.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// One HBM pass over the table per pass of up to 2 residual rows.
//
// A workgroup owns a contiguous run of table rows and each wave a contiguous part
// of it.  The lanes split a row's nb blocks: LPR = min(64, next power of two >= nb)
// lanes per row, 64 / LPR rows per wave step, and lane l takes blocks
// j = l % LPR + LPR t (t < T).  Per block the lane computes
//   partial = scale * sum_p int8[p] * r[32 j + p]        (f32 FMAs, p in order)
// sums its partials in t order, and the LPR lanes of a row add theirs by a
// butterfly, so every logit has one fixed summation order.
//
// Blocks start at even byte offsets only, so a lane loads the 32 bytes from the
// dword-aligned address at or below the block start (two dwordx4) and one dword
// at block bytes 30..33 (2-byte aligned, which gfx9 global memory accepts), all
// inside the block's own dwords or the block; a funnel shift by 0 or 16 bits
// lines the 34 bytes up.
//
// The residual rows sit in LDS as f32, block j at float offset 36 j (a 144-byte
// stride: the 16-byte reads of 16 consecutive blocks cover all 64 banks once).
// ---------------------------------------------------------------------------
// waves per workgroup: 8 for one residual row (two workgroups per CU), 16 for two
// (one workgroup per CU: its two residual copies and 16 wave buffers fit 160 KiB)
template <int RB>
struct Q8Waves {
  static constexpr int value = RB == 2 ? 16 : 8;
};
static constexpr int kQ8Stride = 36;    // floats per block in the LDS residual
static constexpr int kQ8MaxT = 4;       // blocks per lane per row: hidden <= 64 * 4 * 32
static constexpr int kQ8MaxChunks = 9;  // 16-byte chunks per lane per staged step (<= 9 KiB)

__host__ __device__ constexpr int align4(int n) { return (n + 3) & ~3; }

// The 34 bytes of a block as 9 dwords (s[0] = scale | q0 q1 << 16, s[8] low half = q30 q31).
struct Q8Block {
  uint32_t s[9];
};

__device__ __forceinline__ void q8_load(const uint8_t* blk, u32x4& a, u32x4& b, uint32_t& tail) {
  typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
  typedef uint32_t u32a2 __attribute__((aligned(2)));
  // pointer arithmetic, not an integer cast, so the loads stay global (not flat)
  const uint8_t* a0 = blk - ((uintptr_t)blk & 3);
  const u32x4a x = __builtin_nontemporal_load((const u32x4a*)a0);
  const u32x4a y = __builtin_nontemporal_load((const u32x4a*)(a0 + 16));
  a = u32x4{x[0], x[1], x[2], x[3]};
  b = u32x4{y[0], y[1], y[2], y[3]};
  tail = *(const u32a2*)(blk + 30);  // block bytes 30..33, kept whole until the arithmetic
}

__device__ __forceinline__ Q8Block q8_align(const u32x4& a, const u32x4& b, uint32_t tail, uint32_t sh) {
  const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  Q8Block o;
#pragma unroll
  for (int i = 0; i < 7; i++) o.s[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
  o.s[7] = __builtin_amdgcn_alignbit(tail, w[7], sh);  // bytes 28..31 (bytes 30, 31 from the tail when sh = 16)
  o.s[8] = tail >> 16;                                 // bytes 32, 33
  return o;
}

// The block from 9 dwords read at the dword-aligned offset at or below its start.
__device__ __forceinline__ Q8Block q8_align_words(const uint32_t (&w)[9], uint32_t sh) {
  Q8Block o;
#pragma unroll
  for (int i = 0; i < 8; i++) o.s[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
  o.s[8] = w[8] >> sh;
  return o;
}

// int8 value p (0..31) of the block: byte p + 2 of the 34.
__device__ __forceinline__ float q8_value(const Q8Block& blk, int p) {
  const int n = p + 2;
  return (float)(int8_t)(uint8_t)(blk.s[n >> 2] >> (8 * (n & 3)));
}

// logits    nullable [B][V] raw logits
// lse       nullable [B][gridDim.x] log-partition partials at lse_c = log2(e) / T
// U > 0: staged loads of U 16-byte chunks per lane per step; U = 0: per-lane block loads.
template <int RB, int T, int U>
__global__ void __launch_bounds__(64 * Q8Waves<RB>::value) q8_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden, const void* __restrict__ R,
    int wire, int64_t B, int k, uint64_t* __restrict__ cand, int lpr_log2, int rows_per_blk,
    float* __restrict__ logits, float2* __restrict__ lse, float lse_c) {
  extern __shared__ __attribute__((aligned(16))) float q8smem[];
  const int nb = hidden >> 5;
  float* sres = q8smem;                             // [RB][nb][kQ8Stride]
  float* vlog = q8smem + (size_t)RB * nb * kQ8Stride;  // [rows of this block][RB]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t nblk = gridDim.x;
  const int64_t r_begin = (int64_t)blockIdx.x * V / nblk;
  const int nrows = (int)(((int64_t)blockIdx.x + 1) * V / nblk - r_begin);
  const int64_t b0 = (int64_t)blockIdx.y * RB;
  const int nbr = (int)min((int64_t)RB, B - b0);

  for (int i = tid; i < RB * nb * 32; i += blockDim.x) {
    const int b = i / hidden, c = i - b * hidden;
    sres[(b * nb + (c >> 5)) * kQ8Stride + (c & 31)] = b < nbr ? residual_value(R, wire, b0 + b, hidden, c) : 0.f;
  }
  __syncthreads();

  const int LPR = 1 << lpr_log2, G = 64 >> lpr_log2;
  const int seg = lane >> lpr_log2, sl = lane & (LPR - 1);
  // this wave's rows [w0, w1) of the block
  constexpr int kQ8Waves = Q8Waves<RB>::value;
  const int w0 = (int)((int64_t)wv * nrows / kQ8Waves), w1 = (int)((int64_t)(wv + 1) * nrows / kQ8Waves);
  // Rows are software-pipelined: the loads of the wave's next step are issued
  // before the current step's arithmetic.
  //  staged:   the step's G rows (contiguous, 16-byte aligned) are read as 16-byte
  //            chunks, 64 lanes per instruction, into registers, then written to the
  //            wave's LDS buffer, from which each lane reads its blocks' words;
  //  unstaged: each lane reads its blocks straight from global memory.
  auto row_ptr = [&](int i0) {
    const int rl = i0 + seg;
    return table + (uint64_t)(r_begin + (rl < w1 ? rl : w0)) * (uint64_t)row_bytes;
  };
  constexpr bool STAGED = U > 0;
  constexpr int TS = STAGED ? 1 : T;
  u32x4 na[TS], nb2[TS];
  uint32_t ntail[TS];
  u32x4 stg[STAGED ? U : 1];
  // wave buffer: U KiB (>= one step's rows); chunks past the step's rows repeat its
  // last chunk, so every load and store is unconditional and in bounds
  unsigned char* wbuf = (unsigned char*)(vlog + align4(rows_per_blk * RB)) + (size_t)wv * (STAGED ? U * 1024 : 0);
  auto issue = [&](int i0) {
    if constexpr (STAGED) {
      const uint8_t* src = table + (uint64_t)(r_begin + i0) * (uint64_t)row_bytes;
      const int nch = min(64 >> lpr_log2, w1 - i0) * (int)(row_bytes >> 4);
#pragma unroll
      for (int u = 0; u < U; u++)
        stg[u] = __builtin_nontemporal_load((const u32x4*)(src + 16 * min(lane + 64 * u, nch - 1)));
    } else {
      const uint8_t* rowp = row_ptr(i0);
#pragma unroll
      for (int t = 0; t < T; t++) {
        const int j = sl + (t << lpr_log2);
        // lanes past the row's blocks read block 0 and contribute nothing
        q8_load(rowp + 34 * (j < nb ? j : 0), na[t], nb2[t], ntail[t]);
      }
    }
  };
  if (w0 < w1) issue(w0);
  for (int i0 = w0; i0 < w1; i0 += G) {
    const int rl = i0 + seg;
    const bool row_ok = rl < w1;
    const uint8_t* rowp = row_ptr(i0);
    u32x4 ra[TS], rb[TS];
    uint32_t tail[TS];
    if constexpr (STAGED) {
#pragma unroll
      for (int u = 0; u < U; u++) *(u32x4*)(wbuf + 16 * (lane + 64 * u)) = stg[u];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
#pragma unroll
      for (int t = 0; t < T; t++) ra[t] = na[t], rb[t] = nb2[t], tail[t] = ntail[t];
    }
    if (i0 + G < w1) issue(i0 + G);
    float sum[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) sum[b] = 0.f;
#pragma unroll
    for (int t = 0; t < T; t++) {
      const int j = sl + (t << lpr_log2);
      if (j < nb) {
        const uint32_t sh = (((uintptr_t)rowp + 34u * (uint32_t)j) & 2u) ? 16u : 0u;
        Q8Block blk;
        if constexpr (STAGED) {
          // the row sits at seg * row_bytes in the buffer (16-byte aligned)
          const uint32_t* bw = (const uint32_t*)(wbuf + ((seg * (int)row_bytes + 34 * j) & ~3));
          uint32_t w[9];
#pragma unroll
          for (int i = 0; i < 9; i++) w[i] = bw[i];
          blk = q8_align_words(w, sh);
        } else {
          blk = q8_align(ra[t], rb[t], tail[t], sh);
        }
        const float scale = f16_bits_to_f32(blk.s[0] & 0xffffu);
#pragma unroll
        for (int b = 0; b < RB; b++) {
          const f32x4* rr = (const f32x4*)(sres + (b * nb + j) * kQ8Stride);
          float dot = 0.f;
#pragma unroll
          for (int p4 = 0; p4 < 8; p4++) {
            const f32x4 r4 = rr[p4];
#pragma unroll
            for (int e = 0; e < 4; e++) dot = __builtin_fmaf(q8_value(blk, 4 * p4 + e), r4[e], dot);
          }
          sum[b] += dot * scale;
        }
      }
    }
    // the LPR lanes of a row: butterfly (every lane gets the same value)
#pragma unroll
    for (int b = 0; b < RB; b++)
      for (int off = LPR >> 1; off > 0; off >>= 1) sum[b] += __shfl_xor(sum[b], off, 64);
    if (row_ok && sl == 0) {
#pragma unroll
      for (int b = 0; b < RB; b++) vlog[rl * RB + b] = sum[b];
    }
    if constexpr (STAGED) {
      // every lane is done with the buffer before the next step overwrites it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();

  for (int b = wv; b < nbr; b += kQ8Waves) {
    if (logits != nullptr)
      for (int i = lane; i < nrows; i += 64) logits[(b0 + b) * V + r_begin + i] = vlog[i * RB + b];
    if (lse != nullptr) {
      float m = -__builtin_inff();
      for (int i = lane; i < nrows; i += 64) m = fmaxf(m, vlog[i * RB + b]);
      m = wave_max_f32(m);
      float s = 0.f;
      if (m > -__builtin_inff())
        for (int i = lane; i < nrows; i += 64) s += exp2f((vlog[i * RB + b] - m) * lse_c);
      s = wave_sum(s);
      if (lane == 0) lse[(b0 + b) * nblk + blockIdx.x] = make_float2(m, s);
    }
    uint64_t* out = cand + ((b0 + b) * nblk + blockIdx.x) * (int64_t)k;
    uint64_t prev = ~0ull;
    for (int t = 0; t < k; t++) {
      uint64_t best = 0;
      for (int i = lane; i < nrows; i += 64) {
        const uint64_t key = make_key(vlog[i * RB + b], (uint32_t)(r_begin + i));
        if (key < prev && key > best) best = key;
      }
      best = wave_max_u64(best);
      if (lane == 0) out[t] = best;
      prev = best;
    }
  }
}

template <int RB, int T, int U>
static hipError_t launch_q8_cfg(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_dynamic_lds((const void*)q8_logits_kernel<RB, T, U>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((q8_logits_kernel<RB, T, U>), dim3((unsigned)p.nblk, (unsigned)p.npass),
                     dim3(64 * Q8Waves<RB>::value),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, R, (int)x.wire, p.batch, p.k,
                     cand, p.lpr_log2, (int)p.rows_per_blk, x.logits, x.lse, x.lse_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

template <int RB>
static hipError_t launch_q8_rb(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                               const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
#define ETG_Q8_CASE(TV, UV) \
  if (p.q8_t == TV && p.q8_chunks == UV) return launch_q8_cfg<RB, TV, UV>(t, p, R, cand, x, stream, ev0, ev1);
  // unstaged, then the staged (T, U) pairs the planner can produce
  ETG_Q8_CASE(1, 0) ETG_Q8_CASE(2, 0) ETG_Q8_CASE(3, 0) ETG_Q8_CASE(4, 0)
  ETG_Q8_CASE(1, 1) ETG_Q8_CASE(1, 2) ETG_Q8_CASE(1, 3)
  ETG_Q8_CASE(2, 3) ETG_Q8_CASE(2, 4) ETG_Q8_CASE(2, 5)
  ETG_Q8_CASE(3, 5) ETG_Q8_CASE(3, 6) ETG_Q8_CASE(3, 7)
  ETG_Q8_CASE(4, 7) ETG_Q8_CASE(4, 8) ETG_Q8_CASE(4, 9)
#undef ETG_Q8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_q8(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand, const LogitsExtras& x,
                     hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.q8_mfma) return launch_stream_q8(t, p, R, cand, x, stream, ev0, ev1);
  return p.rb == 2 ? launch_q8_rb<2>(t, p, R, cand, x, stream, ev0, ev1)
                   : launch_q8_rb<1>(t, p, R, cand, x, stream, ev0, ev1);
}

int32_t plan_q8(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  // hidden a multiple of 256 and two or more residual rows: the matrix-core kernel
  // (8 residual rows per table pass); one row streams faster through this one
  if (t.hidden % 256 == 0 && batch >= 2) {
    const char* w = "";
    if (plan_stream_q8(t, batch, k, p, &w) == 0) return 0;
  }
  const int64_t nb = t.hidden / 32;
  int lg = 0;
  while ((1 << lg) < nb && lg < 6) lg++;
  p->lpr_log2 = lg;
  p->q8_t = (int32_t)cdiv(nb, (int64_t)1 << lg);
  if (p->q8_t > kQ8MaxT) {
    *why = "hidden too large for the q8 path (at most 8192)";
    return -5;
  }
  p->rb = batch >= 2 ? 2 : 1;
  p->npass = (int32_t)cdiv(batch, p->rb);
  const int waves = p->rb == 2 ? Q8Waves<2>::value : Q8Waves<1>::value;
  // two 8-wave workgroups or one 16-wave workgroup per CU, at most 4096 rows each
  int64_t nblk = std::min<int64_t>((p->rb == 2 ? 1 : 2) * kTargetBlocks, std::max<int64_t>(1, cdiv(t.V, 64)));
  nblk = std::max<int64_t>(nblk, cdiv(t.V, 4096));
  p->nblk = (int32_t)nblk;
  p->rows_per_blk = cdiv(t.V, nblk);
  p->lds_bytes = ((size_t)p->rb * nb * kQ8Stride + align4((int)(p->rows_per_blk * p->rb))) * 4;
  if (p->lds_bytes > kMaxLds) {
    *why = "q8 path LDS";
    return -5;
  }
  // staged loads when rows are whole 16-byte chunks and the wave buffers fit:
  // U = KiB per step (one 16-byte chunk per lane per KiB)
  const int64_t step_bytes = ((int64_t)64 >> lg) * t.row_bytes;
  const int64_t u = cdiv(step_bytes, 1024);
  const size_t staged = p->lds_bytes + (size_t)waves * u * 1024;
  p->q8_chunks = 0;
  // (the launcher instantiates U in [2T - 1, 2T + 1], which covers every staged shape)
  if (t.row_bytes % 16 == 0 && u <= kQ8MaxChunks && u >= 2 * p->q8_t - 1 && u <= 2 * p->q8_t + 1 &&
      staged <= kMaxLds) {
    p->q8_chunks = (int32_t)u;
    p->lds_bytes = staged;
  }
  p->img_bytes = 0;
  p->ncand = p->nblk * k;
  return 0;
}

}  // namespace etg
