// Stream path of the tied lm_head projection (bf16 tables, up to 8 residual rows
// per table pass): ADR-0008 "POST /v1/logits", logits = residual @ lm_head.T over
// every vocabulary row, fused with a per-block top-k.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// Stream path layout.
//
// The table is cut into 8-row groups.  One MFMA step covers 8 rows x 64 values
// (128 contiguous bytes per row) of the table.  Lane l loads row (l % 8), bytes
// [128 s + 16 (l / 8), +16): one load instruction reads 8 full 128-byte lines.
//
// In the 16x16x32 MFMA, lane l supplies A row m = l % 16 with K-group g = l / 16.
// So A row m is table row m % 8, and its K slice is the half h = m / 8 of the
// lane's 32-value window: value index 64 s + 16 g + 8 h + e (e = 0..7).  A dot
// product does not depend on the order of its terms, so any bijection of value
// indices works as long as the residual operand uses the same one.
//
// B column n (lane l supplies column n = l % 16, group g = l / 16) carries a
// residual row at the same value indices for half h = n / 8.  Rows with h = 0
// meet columns with h = 0 and likewise for h = 1; the cross terms D[r][8 + ...]
// and D[r + 8][...] are unused.
//
// The residual is carried as a pair of bf16 values, hi = bf16(x) and
// lo = bf16(x - hi), so the operand error is at most 2^-16 |x| (one bf16
// rounding alone can be 2^-8 |x|).  Two layouts:
//   packed (batch <= 4): one operand image, column n % 8 = b + 4 * part
//                        (part 0 = hi, 1 = lo); one MFMA per step;
//   dual   (batch <= 8): image 0 holds hi, image 1 holds lo, column n % 8 = b;
//                        two MFMAs per step into the same accumulator.
// Then logit[row r][b] = sum over h (and part) of D[r + 8h][8h + ...].
// D layout: lane L holds D[4 (L / 16) + i][L % 16], i = 0..3.  For L < 32 with
// b = L % 16 < nbc, the terms sit in lanes L, L + 40 (+ 4, + 44 when packed).
//
// Each block builds the operand image [step][image][64 lanes] x 16 bytes in LDS
// from the fp32 residual, `chunk` steps at a time (all of it when it fits).
// ---------------------------------------------------------------------------

static constexpr int kStreamWaves = 16;
static constexpr int kStreamUnroll = 6;  // K steps per load group (half of it with two images)
static constexpr int kStreamMaxPairs = 4;  // a wave handles at most 8 groups (64 rows)

// Fill LDS with steps [c0, c0 + n) of the bf16 hi/lo operand image, converted from
// the residual rows of this pass (f32, or decoded from their wire format).  Image slot (s, im, lane) holds the 8
// values of B column n = lane % 16, K-group g = lane / 16 (layout above).
// WIRE is the residual rows' wire format, fixed per kernel instance so that no
// value is read behind a branch on the format (such branches serialise the loads).
template <int NIMG, int WIRE>
__device__ __forceinline__ void stream_stage_image(u32x4* simg, const void* __restrict__ R, int64_t B, int hidden,
                                                   int64_t b0, int c0, int n) {
  constexpr int NBC = NIMG == 1 ? 4 : 8;
  // slots per thread per round, their loads all issued before any conversion (fewer in
  // the one-image kernel, whose K loop sits at the 128-register line of its workgroup)
  constexpr int SU = NIMG == 1 ? 2 : 4;
  const int total = n * NIMG * 64;
  for (int i0 = threadIdx.x; i0 < total; i0 += SU * blockDim.x) {
    float x[SU][8];
    int part[SU];
#pragma unroll
    for (int u = 0; u < SU; u++) {
      const int i = i0 + u * blockDim.x;
      const int lane = i & 63;
      const int q = i >> 6;
      const int im = q % NIMG;
      const int s = c0 + q / NIMG;
      const int nn = lane & 15, g = lane >> 4;
      const int h = nn >> 3, j8 = nn & 7;
      part[u] = NIMG == 1 ? j8 / NBC : im;
      const int64_t b = b0 + j8 % NBC;
      const int cbase = 64 * s + 16 * g + 8 * h;
      const bool live = i < total && b < B;
      if constexpr (NIMG == 2) {
        residual_values8(R, WIRE, live ? B : 0, b, hidden, cbase, x[u]);
      } else {  // value by value: vector loads cost the one-image kernel a register spill
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int c = cbase + e;
          x[u][e] = (live && c < hidden) ? residual_value(R, WIRE, b, hidden, c) : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SU; u++) {
      const int i = i0 + u * blockDim.x;
      if (i >= total) break;
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const uint32_t hi = bf16_rne(x[u][e]);
        // part 1 carries the remainder x - hi (exact in f32), rounded to bf16
        v[e] = part[u] == 1 ? bf16_rne(x[u][e] - __uint_as_float(hi << 16)) : hi;
      }
      simg[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    }
  }
}

// Lanes 0..31 receive lane L + 32's value (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float lane_plus32(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}

// Lane L receives lane L + N's value within its row of 16 lanes (DPP row_shl:N; 0 past
// the row's end).
template <int N>
__device__ __forceinline__ float row_shl(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x100 + N, 0xf, 0xf, false));
}

template <int NBC>
__device__ __forceinline__ void stream_store_group(f32x4 acc, float* dst, int lane) {
  // y = D[r][b] + D[r + 8][8 + b] (lanes L and L + 40), then + the lo columns' sum
  // from lane L + 4 when packed; cross-lane moves by permlane and DPP, not LDS
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; i++) y[i] = acc[i] + row_shl<8>(lane_plus32(acc[i]));
  if (NBC == 4) {
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = y[i] + row_shl<4>(y[i]);
  }
  if (lane < 32 && (lane & 15) < NBC) {
    const int b = lane & 15, r0 = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; i++) dst[(r0 + i) * NBC + b] = y[i];
  }
}

// The k best (logit, row) of this block for residual column b, as descending keys.
// slog is [wave][group * 8 + r][NBC]; wave w owns groups [sg0[w], sg0[w] + sng[w]).
// Each lane holds one row per wave in registers; round t takes the largest key
// below the key of round t - 1 (keys are unique).
template <int NBC>
__device__ void stream_block_topk(const float* slog, const int64_t* sg0, const int* sng, int b, int lane,
                                  int max_groups, int64_t V, int k, uint64_t* out) {
  const int per_wave = max_groups * 8;  // <= 64
  uint64_t key[kStreamWaves];
#pragma unroll
  for (int w = 0; w < kStreamWaves; w++) {
    const int64_t row = sg0[w] * 8 + lane;
    key[w] = (lane < sng[w] * 8 && row < V) ? make_key(slog[(w * per_wave + lane) * NBC + b], (uint32_t)row) : 0;
  }
  uint64_t prev = ~0ull;
  for (int t = 0; t < k; t++) {
    uint64_t best = 0;
#pragma unroll
    for (int w = 0; w < kStreamWaves; w++) best = (key[w] < prev && key[w] > best) ? key[w] : best;
    best = wave_max_u64(best);
    if (lane == 0) out[t] = best;
    prev = best;
  }
}

// The k best keys of this block for each of its nb residual columns, for k up to
// kStreamWaves, by threshold: each wave takes the largest logit of its rows per
// column; T, the k-th largest of those wave maxima, is a lower bound on the
// column's k-th largest logit (the k waves reaching T each hold a row of their
// own at or above it).  Only the logits >= T (k to a few k of them) are keyed into
// an LDS list, and each listed key is written to the slot of its rank among them
// (keys are unique).  Returns false, having written nothing, when a list would
// hold more than kStreamThrCap keys (ties, or blocks with fewer than k waves of
// rows); the caller then selects by rounds.  Called by every thread of the block.
static constexpr int kStreamThrCap = 32;

template <int NBC>
__device__ bool stream_block_topk_thr(const float* slog, const int64_t* sg0, const int* sng, int nb, int max_groups,
                                      int64_t V, int k, int64_t b0, uint64_t* __restrict__ cand) {
  __shared__ uint32_t smax[NBC][kStreamWaves];
  __shared__ uint32_t sthr[NBC];
  __shared__ uint32_t scnt[NBC];
  __shared__ uint64_t slist[NBC][kStreamThrCap];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per_wave = max_groups * 8;
  const int64_t row = sg0[wv] * 8 + lane;
  const bool ok = lane < sng[wv] * 8 && row < V;
  uint32_t o[NBC], m[NBC];
#pragma unroll
  for (int b = 0; b < NBC; b++) {
    o[b] = (ok && b < nb) ? score_ord(slog[(wv * per_wave + lane) * NBC + b]) : 0u;
    m[b] = o[b];
  }
  wave_minmax_u32_multi<true>(m);
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < NBC; b++) smax[b][wv] = m[b];
  }
  if (tid < NBC) scnt[tid] = 0;
  __syncthreads();
  if (tid < nb) {
    // the k-th largest of the wave maxima: insertion into a descending list
    uint32_t t[kStreamWaves];
#pragma unroll
    for (int j = 0; j < kStreamWaves; j++) t[j] = 0u;
#pragma unroll
    for (int w = 0; w < kStreamWaves; w++) {
      uint32_t x = smax[tid][w];
#pragma unroll
      for (int j = 0; j < kStreamWaves; j++) {
        const uint32_t hi = max(t[j], x);
        x = min(t[j], x);
        t[j] = hi;
      }
    }
    uint32_t thr = t[0];
#pragma unroll
    for (int j = 1; j < kStreamWaves; j++) thr = j == k - 1 ? t[j] : thr;
    sthr[tid] = thr;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NBC; b++) {
    if (b < nb && ok && o[b] >= sthr[b]) {
      const uint32_t slot = atomicAdd(&scnt[b], 1u);
      if (slot < (uint32_t)kStreamThrCap) slist[b][slot] = ((uint64_t)o[b] << 32) | (uint64_t)(~(uint32_t)row);
    }
  }
  __syncthreads();
  bool over = false;
  for (int b = 0; b < nb; b++) over |= scnt[b] > (uint32_t)kStreamThrCap;
  if (over) return false;
  if (wv < nb) {
    const int c = (int)scnt[wv];
    uint64_t* out = cand + ((b0 + wv) * gridDim.x + blockIdx.x) * (int64_t)k;
    if (lane < c) {
      const uint64_t key = slist[wv][lane];
      int rank = 0;
      for (int j = 0; j < c; j++) rank += slist[wv][j] > key ? 1 : 0;
      if (rank < k) out[rank] = key;
    }
    for (int t = c + lane; t < k; t += 64) out[t] = 0;  // fewer than k rows in the block
  }
  return true;
}

// After the K loop: the block's logits are in slog ([wave][row][NBC], the wave's
// rows from group sg0[wave], sng[wave] groups; written and synchronised).  Raw
// logits, the per-block top-k candidates of each residual column and the
// log-partition partials.
template <int NBC>
__device__ __forceinline__ void stream_epilogue(const float* slog, const int64_t* sg0, const int* sng, const float* mylog,
                                                int64_t g_begin, int ng, int max_groups, int64_t V, int64_t B,
                                                int64_t b0, int k, uint64_t* __restrict__ cand,
                                                float* __restrict__ logits, float2* __restrict__ lse, float lse_c) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // raw logits: each wave writes the rows it computed (64 consecutive per store)
  if (logits != nullptr) {
    for (int i = lane; i < ng * 8; i += 64) {
      const int64_t row = g_begin * 8 + i;
      if (row < V) {
#pragma unroll
        for (int b = 0; b < NBC; b++)
          if (b0 + b < B) logits[(b0 + b) * V + row] = mylog[i * NBC + b];
      }
    }
  }
  const int nb = (int)min((int64_t)NBC, B - b0);
  const bool done = k <= kStreamWaves && stream_block_topk_thr<NBC>(slog, sg0, sng, nb, max_groups, V, k, b0, cand);
  if (!done && wv < nb) {
    uint64_t* out = cand + ((b0 + wv) * gridDim.x + blockIdx.x) * (int64_t)k;
    stream_block_topk<NBC>(slog, sg0, sng, wv, lane, max_groups, V, k, out);
  }
  if (lse != nullptr && wv >= NBC && wv < 2 * NBC && b0 + (wv - NBC) < B) {
    // waves NBC .. 2 NBC - 1: log-partition partial of column wv - NBC over the
    // block's rows (lane holds row lane of every wave's run, as in the top-k)
    const int b = wv - NBC, per_wave = max_groups * 8;
    float x[kStreamWaves];
    bool ok[kStreamWaves];
#pragma unroll
    for (int w = 0; w < kStreamWaves; w++) {
      ok[w] = lane < sng[w] * 8 && sg0[w] * 8 + lane < V;
      x[w] = ok[w] ? slog[(w * per_wave + lane) * NBC + b] : 0.f;
    }
    const float2 part = wave_lse_part(x, ok, lse_c);
    if (lane == 0) lse[(b0 + b) * gridDim.x + blockIdx.x] = part;
  }
}

// One pass over the table for NBC residual rows (pass = blockIdx.y).
//  table      bf16 [V][hidden], row_bytes = 2 * hidden
//  R          residual rows [B][hidden] in wire format `wire` (0 = fp32)
//  steps      64-value K steps, ceil(hidden / 64)
//  chunk      K steps staged in LDS at a time (a multiple of the unroll)
//  logits     nullable [B][V]: the block's raw logits
//  lse        nullable [B][gridDim.x]: log-partition partial of the block's rows
//             at lse_c = log2(e) / temperature
// Out-of-range rows and K positions are read from clamped in-range addresses and
// meet zero residual values or are never ranked, so no load is predicated (table
// entries are assumed finite).
template <int NIMG, int WIRE>
__global__ void __launch_bounds__(1024) stream_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden,
    const void* __restrict__ R, int64_t B, int steps, int chunk, int k, uint64_t* __restrict__ cand,
    int64_t ngroups, int max_groups, float* __restrict__ logits, float2* __restrict__ lse, float lse_c) {
  constexpr int NBC = NIMG == 1 ? 4 : 8;
  constexpr int U = NIMG == 1 ? kStreamUnroll : kStreamUnroll / 2;
  const int steps_full = hidden / 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4* simg = (u32x4*)smem;
  float* slog = (float*)(smem + (size_t)chunk * NIMG * 1024);
  __shared__ int64_t sg0[kStreamWaves];
  __shared__ int sng[kStreamWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b0 = (int64_t)blockIdx.y * NBC;

  // Waves own contiguous runs of 8-row groups, as even as the group count allows
  // (on a table of 151,936 rows: 4 or 5 groups per wave; runs of whole 16-row
  // pairs would leave some waves 3 pairs against an average of 2.3).  A run is
  // taken in pairs; an odd run ends with a half pair whose second group reloads
  // the first group's rows (cache hits) and is never stored.
  const int64_t nw = (int64_t)gridDim.x * kStreamWaves;
  const int64_t gw = (int64_t)blockIdx.x * kStreamWaves + wv;
  const int64_t g_begin = gw * ngroups / nw;
  const int ng = (int)((gw + 1) * ngroups / nw - g_begin);
  const int npairs = (ng + 1) >> 1;
  if (lane == 0) {
    sg0[wv] = g_begin;
    sng[wv] = ng;
  }
  const int r = lane & 7, ck = lane >> 3;
  const int64_t last_off = row_bytes - 16;

  f32x4 acc0[kStreamMaxPairs], acc1[kStreamMaxPairs];
#pragma unroll
  for (int p = 0; p < kStreamMaxPairs; p++) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < steps; c0 += chunk) {
    const int c1 = min(steps, c0 + chunk);
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    stream_stage_image<NIMG, WIRE>(simg, R, B, hidden, b0, c0, c1 - c0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kStreamMaxPairs; p++) {
      if (p < npairs) {
        const int64_t row0 = min((g_begin + 2 * p) * 8 + r, V - 1);
        const int64_t row1 = 2 * p + 1 < ng ? min((g_begin + 2 * p) * 8 + 8 + r, V - 1) : row0;
        const uint8_t* p0 = table + (uint64_t)row0 * (uint64_t)row_bytes;
        const uint8_t* p1 = table + (uint64_t)row1 * (uint64_t)row_bytes;
        const u32x4* q0 = (const u32x4*)(p0 + 16 * ck);
        const u32x4* q1 = (const u32x4*)(p1 + 16 * ck);
        // complete steps, U at a time: all loads of the group are issued before the
        // MFMAs that consume them
        const int cf = min(c1, steps_full);
        int s0 = c0;
        for (; s0 + U <= cf; s0 += U) {
          u32x4 a0[U], a1[U];
#pragma unroll
          for (int j = 0; j < U; j++) {
            a0[j] = __builtin_nontemporal_load(q0 + 8 * (s0 + j));
            a1[j] = __builtin_nontemporal_load(q1 + 8 * (s0 + j));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < U; j++) {
            const u32x4* bl = simg + (size_t)(s0 + j - c0) * NIMG * 64 + lane;
#pragma unroll
            for (int im = 0; im < NIMG; im++) {
              const bf16x8 bop = __builtin_bit_cast(bf16x8, bl[im * 64]);
              acc0[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0[j]), bop, acc0[p], 0,
                                                                0, 0);
              acc1[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1[j]), bop, acc1[p], 0,
                                                                0, 0);
            }
          }
        }
        // remaining steps of the chunk, one at a time; a K position at or past
        // `hidden` reads the row's last 16 bytes and meets a zero residual value
        for (; s0 < min(c1, steps); s0++) {
          const int64_t off = min((int64_t)(128 * s0 + 16 * ck), last_off);
          const u32x4 a0 = __builtin_nontemporal_load((const u32x4*)(p0 + off));
          const u32x4 a1 = __builtin_nontemporal_load((const u32x4*)(p1 + off));
          const u32x4* bl = simg + (size_t)(s0 - c0) * NIMG * 64 + lane;
#pragma unroll
          for (int im = 0; im < NIMG; im++) {
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bl[im * 64]);
            acc0[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), bop, acc0[p], 0, 0, 0);
            acc1[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), bop, acc1[p], 0, 0, 0);
          }
        }
      }
    }
  }

  float* mylog = slog + (size_t)wv * max_groups * 8 * NBC;
#pragma unroll
  for (int p = 0; p < kStreamMaxPairs; p++) {
    if (2 * p < ng) stream_store_group<NBC>(acc0[p], mylog + (size_t)(2 * p) * 8 * NBC, lane);
    if (2 * p + 1 < ng) stream_store_group<NBC>(acc1[p], mylog + (size_t)(2 * p + 1) * 8 * NBC, lane);
  }
  __syncthreads();

  stream_epilogue<NBC>(slog, sg0, sng, mylog, g_begin, ng, max_groups, V, B, b0, k, cand, logits, lse, lse_c);
}


template <int NIMG, int WIRE>
static hipError_t launch_stream_nimg(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                     const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_dynamic_lds((const void*)stream_logits_kernel<NIMG, WIRE>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((stream_logits_kernel<NIMG, WIRE>), dim3((unsigned)p.nblk, (unsigned)p.npass),
                     dim3(64 * kStreamWaves), p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, R,
                     p.batch, p.steps, p.chunk, p.k, cand, p.ngroups, p.max_groups, x.logits, x.lse, x.lse_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

template <int NIMG>
static hipError_t launch_stream_wire(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                     const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  switch (x.wire) {
    case WIRE_F16: return launch_stream_nimg<NIMG, WIRE_F16>(t, p, R, cand, x, stream, ev0, ev1);
    case WIRE_I8: return launch_stream_nimg<NIMG, WIRE_I8>(t, p, R, cand, x, stream, ev0, ev1);
    default: return launch_stream_nimg<NIMG, WIRE_F32>(t, p, R, cand, x, stream, ev0, ev1);
  }
}

hipError_t launch_stream(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                         const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  return p.nimg == 1 ? launch_stream_wire<1>(t, p, R, cand, x, stream, ev0, ev1)
                     : launch_stream_wire<2>(t, p, R, cand, x, stream, ev0, ev1);
}

// ---------------------------------------------------------------------------
// Q8_0 tables through the matrix cores (rows of a multiple of 16 bytes: hidden a
// multiple of 256), one table pass per 8 residual rows.
//
// A Q8_0 block (a binary16 scale, then 32 int8 values; the embeddinggemma.c port
// specification, "Tensor inventory") is exactly the K extent of one
// v_mfma_f32_16x16x32_bf16, and int8 values are exact in bf16.  One MFMA per block
// and 16-row table tile gives, exactly multiplied and summed in f32,
//   D[slot][row] = sum_p q[row][p] x[slot][p],
// and the block's scale enters once per result: acc += scale[row] D.  The
// residual image is the A operand (slot m = lane % 16, values 8 (lane / 16) + e
// of the block) and the table the B operand (table row n = lane % 16, the same
// values), so lane L's four results D[4 (L / 16) + i][L % 16] all belong to table
// row L % 16 and take one scale.  Slot b + 8 part carries residual row b as its
// bf16 hi (part 0) or lo (part 1) value; lanes L and L + 32 hold the hi and lo
// sums of residual rows 4 (L / 16) + i.
//
// Table bytes reach the lanes through a per-wave LDS buffer.  A step is 8 blocks
// (272 bytes, 17 16-byte chunks) of each row of a 16-row tile; lane l loads
// chunks l + 64 u of the step, one step ahead of their use.  The row pieces are
// not aligned to 128-byte lines, and this load pattern is what bounds the kernel
// (about 4.6 TB/s with the arithmetic removed), so one residual row keeps the
// lane-split kernel of q8.hip.  The residual image
// is staged per block of the table in chunks of whole steps, as in the bf16 path.
// ---------------------------------------------------------------------------
static constexpr int kQ8mBlocks = 8;                       // Q8_0 blocks per step
static constexpr int kQ8mRowStep = 34 * kQ8mBlocks;        // bytes of a row per step (272)
static constexpr int kQ8mTileChunks = 16 * kQ8mRowStep / 16;  // 16-byte chunks per tile step (272)
static constexpr int kQ8mLoads = (kQ8mTileChunks + 63) / 64;  // per lane (5; the last for 16 lanes)
static constexpr int kQ8mWaveBuf = 16 * kQ8mRowStep;       // bytes of a wave's step buffer
static constexpr int kQ8mMaxPairs = 4;                     // 16-row tiles per wave (accumulator registers)

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Eight int8 values (two dwords) as eight bf16 values (exact).
__device__ __forceinline__ bf16x8 q8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const u32x4 v = {bf16_pair((float)(int8_t)(w0 & 0xffu), (float)(int8_t)((w0 >> 8) & 0xffu)),
                   bf16_pair((float)(int8_t)((w0 >> 16) & 0xffu), (float)(int8_t)(w0 >> 24)),
                   bf16_pair((float)(int8_t)(w1 & 0xffu), (float)(int8_t)((w1 >> 8) & 0xffu)),
                   bf16_pair((float)(int8_t)((w1 >> 16) & 0xffu), (float)(int8_t)(w1 >> 24))};
  return __builtin_bit_cast(bf16x8, v);
}

// Image slots of table blocks [j0, j0 + n): slot (j, lane) holds the 8 values
// 32 (j0 + j) + 8 (lane / 16) + e of slot lane % 16 (residual row b0 + slot % 8,
// part slot / 8) as bf16.
__device__ __forceinline__ void stream_q8_stage_image(u32x4* simg, const void* __restrict__ R, int wire, int64_t B,
                                                      int hidden, int64_t b0, int j0, int n) {
  for (int i = threadIdx.x; i < n * 64; i += blockDim.x) {
    const int lane = i & 63, j = j0 + (i >> 6);
    const int m = lane & 15, g = lane >> 4;
    const int64_t b = b0 + (m & 7);
    const int cbase = 32 * j + 8 * g;
    float x[8];
    residual_values8(R, wire, B, b, hidden, cbase, x);
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t hi = bf16_rne(x[e]);
      v[e] = (m >> 3) ? bf16_rne(x[e] - __uint_as_float(hi << 16)) : hi;  // x - hi is exact in f32
    }
    simg[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
  }
}

//  table     Q8_0 [V][hidden / 32 blocks], row_bytes = 34 hidden / 32, a multiple of 16
//  steps     8-block steps per row (hidden / 256)
//  chunk     steps of the residual image staged in LDS at a time
//  wbuf_off  byte offset of the waves' step buffers in dynamic LDS
// The rest as for stream_logits_kernel (8 residual rows per pass).
__global__ void __launch_bounds__(1024) stream_q8_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden, const void* __restrict__ R,
    int wire, int64_t B, int steps, int chunk, int wbuf_off, int k, uint64_t* __restrict__ cand, int64_t ngroups,
    int max_groups, float* __restrict__ logits, float2* __restrict__ lse, float lse_c) {
  constexpr int NBC = 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4* simg = (u32x4*)smem;
  float* slog = (float*)smem;  // after the K loop
  __shared__ int64_t sg0[kStreamWaves];
  __shared__ int sng[kStreamWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b0 = (int64_t)blockIdx.y * NBC;
  unsigned char* wb = smem + wbuf_off + wv * kQ8mWaveBuf;

  // waves own contiguous runs of 16-row tiles (pairs of 8-row groups), as in the bf16 path
  const int64_t nw = (int64_t)gridDim.x * kStreamWaves;
  const int64_t gw = (int64_t)blockIdx.x * kStreamWaves + wv;
  const int64_t npairs_all = (ngroups + 1) >> 1;
  const int64_t pb = gw * npairs_all / nw;
  const int npairs = (int)((gw + 1) * npairs_all / nw - pb);
  const int64_t g_begin = 2 * pb;
  const int ng = (int)min((int64_t)(2 * npairs), ngroups - g_begin);
  if (lane == 0) {
    sg0[wv] = g_begin;
    sng[wv] = ng;
  }
  const int n = lane & 15, g = lane >> 4;

  f32x4 acc[kQ8mMaxPairs];
#pragma unroll
  for (int p = 0; p < kQ8mMaxPairs; p++) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < steps; c0 += chunk) {
    const int c1 = min(steps, c0 + chunk), ns = c1 - c0;
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    stream_q8_stage_image(simg, R, wire, B, hidden, b0, kQ8mBlocks * c0, kQ8mBlocks * ns);
    __syncthreads();
    // iterations (tile p, step c0 + s), tile-major; the loads of iteration it + 1
    // are issued once those of iteration it are in the wave's buffer, before its
    // blocks (a second register set for two steps ahead measured slower)
    const int nit = npairs * ns;
    u32x4 nx[kQ8mLoads];
    auto issue = [&](int it) {
      const int p = it / ns, st = c0 + it % ns;
      const int64_t rbase = (g_begin + 2 * p) * 8;
#pragma unroll
      for (int u = 0; u < kQ8mLoads; u++) {
        // chunk c = lane + 64 u of the step: row c / 17, 16-byte piece c % 17
        const int c = min(lane + 64 * u, kQ8mTileChunks - 1), cr = c / 17;
        const int64_t row = min(rbase + cr, V - 1);  // rows past V: never ranked
        // a plain load: the 128-byte lines at the piece's ends are touched again by
        // the neighbouring step, which should find them in L2
        nx[u] = *(const u32x4*)(table + (uint64_t)row * (uint64_t)row_bytes + kQ8mRowStep * st + 16 * (c - 17 * cr));
      }
    };
    if (nit > 0) issue(0);
    for (int it = 0; it < nit; it++) {
#pragma unroll
      for (int u = 0; u < kQ8mLoads; u++)
        if (lane + 64 * u < kQ8mTileChunks) *(u32x4*)(wb + 16 * (lane + 64 * u)) = nx[u];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (it + 1 < nit) issue(it + 1);
      const int p = it / ns, s = it % ns;
      const u32x4* bl = simg + (size_t)s * kQ8mBlocks * 64 + lane;
      const unsigned char* rowb = wb + n * kQ8mRowStep;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kQ8mBlocks; j++) {
        // values 8 g .. 8 g + 7 of block j: bytes 34 j + 2 + 8 g ..; the scale: bytes 34 j, 34 j + 1
        uint32_t w0, w1;
        if ((34 * j + 2) % 4 == 0) {
          const uint32_t* q = (const uint32_t*)(rowb + 34 * j + 2 + 8 * g);
          w0 = q[0];
          w1 = q[1];
        } else {
          const uint32_t* q = (const uint32_t*)(rowb + 34 * j + 8 * g);
          const uint32_t a = q[0], b = q[1], c = q[2];
          w0 = __builtin_amdgcn_alignbit(b, a, 16);
          w1 = __builtin_amdgcn_alignbit(c, b, 16);
        }
        const float sc = f16_bits_to_f32(*(const uint16_t*)(rowb + 34 * j));
        const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bl[j * 64]),
                                                                q8_to_bf16x8(w0, w1), f32x4{0.f, 0.f, 0.f, 0.f},
                                                                0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) sacc[i] = __builtin_fmaf(sc, d[i], sacc[i]);
      }
#pragma unroll
      for (int q = 0; q < kQ8mMaxPairs; q++)
        if (q == p) acc[q] += sacc;  // p is the same for the whole wave
      // the buffer is rewritten by the next iteration
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();  // the image area becomes the logit area

  // lanes L < 32: residual rows 4 (L / 16) + i, table row L % 16 of each tile (hi + lo)
  float* mylog = slog + (size_t)wv * max_groups * 8 * NBC;
#pragma unroll
  for (int p = 0; p < kQ8mMaxPairs; p++) {
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = acc[p][i] + lane_plus32(acc[p][i]);
    if (p < npairs && lane < 32) {
#pragma unroll
      for (int i = 0; i < 4; i++) mylog[(16 * p + n) * NBC + 4 * g + i] = y[i];
    }
  }
  __syncthreads();

  stream_epilogue<NBC>(slog, sg0, sng, mylog, g_begin, ng, max_groups, V, B, b0, k, cand, logits, lse, lse_c);
}

hipError_t launch_stream_q8(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                            const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_dynamic_lds((const void*)stream_q8_kernel, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(stream_q8_kernel, dim3((unsigned)p.nblk, (unsigned)p.npass), dim3(64 * kStreamWaves),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, R, (int)x.wire, p.batch, p.steps,
                     p.chunk, (int)(p.lds_bytes - (size_t)kStreamWaves * kQ8mWaveBuf), p.k, cand, p.ngroups,
                     p.max_groups, x.logits, x.lse, x.lse_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

int32_t plan_stream_q8(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  if (t.dtype != DT_Q8_0 || t.hidden % (32 * kQ8mBlocks) != 0) {
    *why = "the Q8_0 matrix-core kernel needs hidden a multiple of 256";
    return -5;
  }
  p->nbc = 8;
  p->steps = (int32_t)(t.hidden / (32 * kQ8mBlocks));
  p->ngroups = cdiv(t.V, 8);
  p->npass = (int32_t)cdiv(batch, 8);
  const int64_t npairs_all = cdiv(p->ngroups, 2);
  p->nblk = (int32_t)std::max<int64_t>(cdiv(npairs_all, (int64_t)kStreamWaves * kQ8mMaxPairs),
                                       std::min<int64_t>(kTargetBlocks, cdiv(npairs_all, kStreamWaves)));
  p->max_groups = (int32_t)(2 * cdiv(npairs_all, (int64_t)p->nblk * kStreamWaves));
  const size_t log_bytes = (size_t)kStreamWaves * p->max_groups * 8 * p->nbc * 4;
  const size_t wbuf = (size_t)kStreamWaves * kQ8mWaveBuf;
  const size_t step_img = (size_t)kQ8mBlocks * 1024;  // image bytes per step
  const int64_t max_chunk = (int64_t)((kMaxLds - 1024 - wbuf) / step_img);
  const int64_t nchunks = cdiv(p->steps, max_chunk);
  p->chunk = (int32_t)cdiv(p->steps, nchunks);
  p->lds_bytes = std::max((size_t)p->chunk * step_img, log_bytes) + wbuf;
  if (p->lds_bytes > kMaxLds - 1024) {
    *why = "the Q8_0 matrix-core kernel's LDS";
    return -5;
  }
  p->q8_mfma = 1;
  p->img_bytes = 0;
  p->ncand = p->nblk * k;
  return 0;
}

int32_t plan_stream(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  (void)why;
    p->nimg = batch <= 4 ? 1 : 2;
    p->nbc = p->nimg == 1 ? 4 : 8;
    p->steps = (int32_t)cdiv(t.hidden, 64);
    p->ngroups = cdiv(t.V, 8);
    p->npass = (int32_t)cdiv(batch, p->nbc);
    // one block per CU, unless a wave would then own more than 2 kStreamMaxPairs
    // groups; fewer blocks for tables of under a pair per wave
    p->nblk = (int32_t)std::max<int64_t>(cdiv(p->ngroups, (int64_t)kStreamWaves * 2 * kStreamMaxPairs),
                                         std::min<int64_t>(kTargetBlocks, cdiv(p->ngroups, 2 * kStreamWaves)));
    p->max_groups = (int32_t)cdiv(p->ngroups, (int64_t)p->nblk * kStreamWaves);
    const size_t log_bytes = (size_t)kStreamWaves * p->max_groups * 8 * p->nbc * 4;
    const size_t img_room = kMaxLds - 4096 - log_bytes;  // static LDS: wave runs and the threshold selection
    const int64_t max_chunk = (int64_t)(img_room / ((size_t)p->nimg * 1024)) / kStreamUnroll * kStreamUnroll;
    // equal chunks (multiples of the unroll), as few as fit
    const int64_t nchunks = cdiv(p->steps, max_chunk);
    p->chunk = (int32_t)std::min<int64_t>(max_chunk, cdiv(cdiv(p->steps, nchunks), kStreamUnroll) * kStreamUnroll);
    p->lds_bytes = (size_t)p->chunk * p->nimg * 1024 + log_bytes;
    p->img_bytes = 0;
    p->ncand = p->nblk * k;
  return 0;
}

}  // namespace etg
