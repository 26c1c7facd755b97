// Tied lm_head projection fused with per-row top-k.
//
// ADR-0008 "POST /v1/logits": logits = residual @ lm_head.T over every vocabulary
// row (every row is needed for the argmax, HELIX Columnar Embedding proposal
// section 5), answered as the top_k tokens in descending order.  The V-wide
// logits never reach HBM: each block keeps the logits of its slice of the
// vocabulary in LDS, emits its k best per residual row as 64-bit order keys,
// and topk_merge_kernel reduces those lists to the final answer.
//
// Paths (chosen by the host, see plan_logits):
//  * stream: bf16 tables, memory-bound batches.  One pass over the table per 8
//    residual rows (per 4 when packed), the residual entering as a hi+lo pair of
//    bf16 values.  bf16 MFMA (v_mfma_f32_16x16x32_bf16) is only the dot engine;
//    the table is read once, straight into VGPRs.
//  * wide:   bf16 tables, batches up to a few hundred rows.  One table pass per
//    up to 64 residual rows, still streamed into VGPRs; the residual operand is
//    staged through LDS and no MFMA lane is idle.
//  * gemm:   bf16 tables, large batches: a tiled MFMA contraction.
//  * q8:     Q8_0 tables: lanes split each row's 34-byte blocks, f32 FMAs, one
//    table pass per up to 2 residual rows (q8.hip).
//  * row:    f32 / bf16 / f16 tables, one or two residual rows per table pass: a
//    wave reads a row as 1 KiB contiguous loads, f32 FMAs against the residual in
//    LDS (row.hip).
//  * valu:   any dtype (f32, bf16, f16, Q8_0); f32 FMAs per lane, one table pass per
//    up to 8 residual rows.
// Every path can also write its raw logits and per-block log-partition partials
// (probabilities at a temperature), and reads the residual in any wire format.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// VALU path: any dtype.  Block = 4 waves over a contiguous slice of rows; a wave
// takes one row at a time, each lane accumulates RB residual rows over values
// lane, lane + 64, ... with f32 FMAs, then a butterfly sum per residual row.
// A lane sums its products in chunks of kValuChunk values (64 kValuChunk apart in
// the row) and adds each chunk's sum to its total, so a logit carries at most
// kValuChunk + hidden / (64 kValuChunk) + 6 roundings of 2^-24 relative to
// sum_i |r_i e_i|: 70 for the widest rows (65,536 values), 4.2e-6 in all, inside
// the f32 tables' 1e-5 bound at every supported width.
// ---------------------------------------------------------------------------
static constexpr int kValuChunk = 32;

// logits (nullable [B][V]) receives the raw logits, lse (nullable [B][nblk]) the
// log-partition partial of the block's rows at lse_c = log2(e) / temperature.
template <int DT, int RB>
__global__ void __launch_bounds__(256) valu_logits_kernel(const uint8_t* __restrict__ table, int64_t V,
                                                          int64_t row_bytes, int hidden,
                                                          const void* __restrict__ R, int wire, int64_t B, int k,
                                                          uint64_t* __restrict__ cand, float* __restrict__ logits,
                                                          float2* __restrict__ lse, float lse_c) {
  extern __shared__ float vlog[];  // [rows of this block][RB]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nblk = gridDim.x;
  const int64_t r_begin = (int64_t)blockIdx.x * V / nblk;
  const int nrows = (int)(((int64_t)blockIdx.x + 1) * V / nblk - r_begin);
  const int64_t b0 = (int64_t)blockIdx.y * RB;
  const int nb = (int)((B - b0) < RB ? (B - b0) : RB);
  for (int lr = wv; lr < nrows; lr += 4) {
    const uint8_t* row = table + (uint64_t)(r_begin + lr) * (uint64_t)row_bytes;
    float acc[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) acc[b] = 0.f;
    for (int c0 = lane; c0 < hidden; c0 += 64 * kValuChunk) {
      const int c1 = min(hidden, c0 + 64 * kValuChunk);
      float part[RB];
#pragma unroll
      for (int b = 0; b < RB; b++) part[b] = 0.f;
      if (wire == WIRE_F32) {
        const float* Rf = (const float*)R;
        for (int c = c0; c < c1; c += 64) {
          const float x = deq_value<DT>(row, c);
#pragma unroll
          for (int b = 0; b < RB; b++)
            if (b < nb) part[b] = __builtin_fmaf(x, Rf[(b0 + b) * hidden + c], part[b]);
        }
      } else {
        for (int c = c0; c < c1; c += 64) {
          const float x = deq_value<DT>(row, c);
#pragma unroll
          for (int b = 0; b < RB; b++)
            if (b < nb) part[b] = __builtin_fmaf(x, residual_value(R, wire, b0 + b, hidden, c), part[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < RB; b++) acc[b] += part[b];
    }
#pragma unroll
    for (int b = 0; b < RB; b++) {
      const float s = wave_sum(acc[b]);
      if (lane == 0) vlog[lr * RB + b] = s;
    }
  }
  __syncthreads();
  for (int b = wv; b < nb; b += 4) {
    if (logits != nullptr)
      for (int i = lane; i < nrows; i += 64) logits[(b0 + b) * V + r_begin + i] = vlog[i * RB + b];
    if (lse != nullptr) {
      float m = -__builtin_inff();
      for (int i = lane; i < nrows; i += 64) m = fmaxf(m, vlog[i * RB + b]);
      m = wave_max_f32(m);
      float sum = 0.f;
      if (m > -__builtin_inff())
        for (int i = lane; i < nrows; i += 64) sum += exp2f((vlog[i * RB + b] - m) * lse_c);
      sum = wave_sum(sum);
      if (lane == 0) lse[(b0 + b) * nblk + blockIdx.x] = make_float2(m, sum);
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

// ---------------------------------------------------------------------------
// Cross-block merge: per residual row (blockIdx.x), the k largest of n keys.
// Each thread keeps up to KPT keys in registers.  Every wave first takes the k
// best of its own keys (round t: the largest key below round t - 1's, by a wave
// max); wave 0 then does the same over the 16 per-wave lists.  The k best of
// the union of the waves' k best are the k best overall.
// ---------------------------------------------------------------------------
static constexpr int kMergeThreads = 1024;
static constexpr int kMergeWaves = kMergeThreads / 64;

// Log-partition of one residual row from its n partials (m_i, s_i), returned to
// every thread as (M, log2 S), S = sum_i s_i exp2((m_i - M) c).  Each thread
// combines a strided subset, each wave reduces (max, then rescaled sum) and
// every thread combines the kMergeWaves wave results in the same order.
__device__ float2 block_log_partition(const float2* __restrict__ part, int n, float c, float2* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float2 a = make_float2(-__builtin_inff(), 0.f);
  for (int i = tid; i < n; i += kMergeThreads) a = lse_combine(a, part[i], c);
  const float m = wave_max_f32(a.x);
  const float s = wave_sum(m > -__builtin_inff() ? a.y * exp2f((a.x - m) * c) : 0.f);
  if (lane == 0) red[wv] = make_float2(m, s);
  __syncthreads();
  float2 r = red[0];
  for (int w = 1; w < kMergeWaves; w++) r = lse_combine(r, red[w], c);
  return make_float2(r.x, log2f(r.y));
}

// prob = exp(score / T - lse) with lse = (M c + log2 S) ln 2, computed as
// exp2((score - M) c - log2 S).
__device__ __forceinline__ float prob_of(float score, float2 ml, float c) {
  return exp2f((score - ml.x) * c - ml.y);
}

// Wave 0's final rounds over the kMergeWaves * k per-wave bests in part (N per lane).
template <int N>
__device__ __forceinline__ void merge_final(const uint64_t* part, int k, int32_t* ids, float* scores, float* probs,
                                            float2 ml, float lc) {
  const int lane = threadIdx.x & 63;
  uint64_t key2[N];
#pragma unroll
  for (int j = 0; j < N; j++) {
    const int i = lane + 64 * j;
    key2[j] = i < kMergeWaves * k ? part[i] : 0;
  }
  for (int t = 0; t < k; t++) {
    const uint64_t best = wave_pop_max(key2);
    if (lane == 0) {
      const float sc = ord_score((uint32_t)(best >> 32));
      ids[t] = (int32_t)(~(uint32_t)(best & 0xffffffffu));
      scores[t] = sc;
      if (probs != nullptr) probs[t] = prob_of(sc, ml, lc);
    }
  }
}

// probs (nullable [B][k]): probabilities of the selected ids from the partials
// lse [B][nparts] at c = log2(e) / temperature.
template <int KPT>
__global__ void __launch_bounds__(1024) topk_merge_kernel(const uint64_t* __restrict__ cand, int n, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ scores,
                                                          const float2* __restrict__ lse, int nparts, float lc,
                                                          float* __restrict__ probs) {
  __shared__ uint64_t part[kMergeWaves * 64];
  __shared__ float2 red[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const float2 ml = probs != nullptr ? block_log_partition(lse + b * nparts, nparts, lc, red) : float2{};
  const uint64_t* c = cand + b * (int64_t)n;
  uint64_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; j++) {
    const int i = tid + j * kMergeThreads;
    key[j] = i < n ? c[i] : 0;
  }
  // each wave's k best, then wave 0 merges the kMergeWaves lists
  for (int t = 0; t < k; t++) {
    const uint64_t best = wave_pop_max(key);
    if (lane == 0) part[wv * k + t] = best;
  }
  __syncthreads();
  if (wv == 0) {
    // kMergeWaves * k keys: 4 per lane for k <= 16, else up to 16
    if (k <= 16) {
      merge_final<4>(part, k, ids + b * k, scores + b * k, probs != nullptr ? probs + b * k : nullptr, ml, lc);
    } else {
      merge_final<kMergeWaves>(part, k, ids + b * k, scores + b * k, probs != nullptr ? probs + b * k : nullptr,
                               ml, lc);
    }
  }
}

// Same, for more keys than fit in registers: every round rescans global memory.
__global__ void __launch_bounds__(1024) topk_merge_wide_kernel(const uint64_t* __restrict__ cand, int n, int k,
                                                               int32_t* __restrict__ ids, float* __restrict__ scores,
                                                               const float2* __restrict__ lse, int nparts, float lc,
                                                               float* __restrict__ probs) {
  __shared__ uint64_t red[2][kMergeWaves];
  __shared__ float2 lred[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const float2 ml = probs != nullptr ? block_log_partition(lse + b * nparts, nparts, lc, lred) : float2{};
  const uint64_t* c = cand + b * (int64_t)n;
  uint64_t prev = ~0ull;
  for (int t = 0; t < k; t++) {
    uint64_t best = 0;
    for (int i = tid; i < n; i += kMergeThreads) {
      const uint64_t key = c[i];
      best = (key < prev && key > best) ? key : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) red[t & 1][wv] = best;
    __syncthreads();
    uint64_t m = red[t & 1][0];
    for (int w = 1; w < kMergeWaves; w++) m = red[t & 1][w] > m ? red[t & 1][w] : m;
    if (tid == 0) {
      const float sc = ord_score((uint32_t)(m >> 32));
      ids[b * k + t] = (int32_t)(~(uint32_t)(m & 0xffffffffu));
      scores[b * k + t] = sc;
      if (probs != nullptr) probs[b * k + t] = prob_of(sc, ml, lc);
    }
    prev = m;
  }
}

// Per residual row, the k largest of nl lists of k keys each, every list in
// descending order with its empty (0) slots at the end (the lists of the stream,
// wide, VALU, q8 and row kernels): k rounds of taking the largest list head.
// The workgroup combines the row's log-partition partials when probabilities are
// asked for and stages the row's nl k keys in LDS (a few loads per thread, all in
// flight); then wave 0 keeps the heads of lists l + 64 j (j < PL) in lane l.
//
// For k <= 16 and at least 16 k lists, a threshold pass first, which usually
// replaces those rounds: thread l holds list l (nl <= 1,024) in registers; the
// lists form groups of 16 (a row of 16 lanes), and the k-th largest of the groups'
// largest heads is a lower bound T on the row's k-th largest key (the k groups
// reaching it hold a key each at or above it), so the answer is among the keys
// >= T, a prefix of each list.  Those keys (k to a few k) are gathered in LDS and
// each is written to the slot of its rank among them (keys are unique).  More than
// kMergeThrCap of them falls back to the rounds.
static constexpr int kSortedMergeMaxKeys = 8192;  // 64 KiB of LDS
static constexpr int kMergeThrKeys = 16;          // keys per list held by a thread
static constexpr int kMergeThrCap = 256;
template <int PL>
__global__ void __launch_bounds__(kMergeThreads) topk_merge_sorted_kernel(const uint64_t* __restrict__ cand, int nl,
                                                                          int k, int32_t* __restrict__ ids,
                                                                          float* __restrict__ scores,
                                                                          const float2* __restrict__ lse, int nparts,
                                                                          float lc, float* __restrict__ probs) {
  extern __shared__ uint64_t sk[];  // [nl * k]
  __shared__ float2 red[kMergeWaves];
  __shared__ uint64_t gmax[kMergeThreads / 16];
  __shared__ uint64_t tbuf[kMergeThrCap];
  __shared__ uint64_t sthr;
  __shared__ uint32_t scnt;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const float2 ml = probs != nullptr ? block_log_partition(lse + b * nparts, nparts, lc, red) : float2{};
  const int n = nl * k;
  const uint64_t* c = cand + b * (int64_t)n;
  const int ngr = (nl + 15) >> 4;
  if (k <= kMergeThrKeys && nl <= kMergeThreads && ngr >= k) {
    uint64_t key[kMergeThrKeys];
#pragma unroll
    for (int j = 0; j < kMergeThrKeys; j++) key[j] = (tid < nl && j < k) ? c[(int64_t)tid * k + j] : 0;
    // the largest head of each group of 16 lists, left in the row's lane 15
    uint64_t m = key[0];
    m = dpp_max_u64<0x111, 0xf>(m);  // row_shr:1
    m = dpp_max_u64<0x112, 0xf>(m);  // row_shr:2
    m = dpp_max_u64<0x114, 0xf>(m);  // row_shr:4
    m = dpp_max_u64<0x118, 0xf>(m);  // row_shr:8
    if ((lane & 15) == 15 && (tid >> 4) < ngr) gmax[tid >> 4] = m;
    if (tid == 0) scnt = 0;
    __syncthreads();
    if (wv == 0) {
      // T: the smallest group maximum with fewer than k group maxima above it
      const uint64_t x = lane < ngr ? gmax[lane] : ~0ull;
      int above = 0;
      for (int g = 0; g < ngr; g++) above += gmax[g] > x ? 1 : 0;
      const uint64_t t = (lane < ngr && above < k) ? x : ~0ull;
      const uint64_t tmin = ~wave_max_u64(~t);
      if (lane == 0) sthr = tmin;
    }
    __syncthreads();
    const uint64_t T = sthr;
    int nk = 0;
#pragma unroll
    for (int j = 0; j < kMergeThrKeys; j++) nk += (key[j] != 0 && key[j] >= T) ? 1 : 0;
    const uint32_t slot = nk > 0 ? atomicAdd(&scnt, (uint32_t)nk) : 0u;
    if (nk > 0 && slot + nk <= (uint32_t)kMergeThrCap) {
#pragma unroll
      for (int j = 0; j < kMergeThrKeys; j++)
        if (j < nk) tbuf[slot + j] = key[j];  // the list's prefix at or above T
    }
    __syncthreads();
    const int total = (int)scnt;
    if (total <= kMergeThrCap) {
      if (tid < total) {
        const uint64_t x = tbuf[tid];
        int rank = 0;
        for (int j = 0; j < total; j++) rank += tbuf[j] > x ? 1 : 0;
        if (rank < k) {
          const float sc = ord_score((uint32_t)(x >> 32));
          ids[b * k + rank] = (int32_t)(~(uint32_t)(x & 0xffffffffu));
          scores[b * k + rank] = sc;
          if (probs != nullptr) probs[b * k + rank] = prob_of(sc, ml, lc);
        }
      } else if (tid < k) {  // fewer than k keys in all: the empty key, as the rounds give
        ids[b * k + tid] = (int32_t)~0u;
        scores[b * k + tid] = ord_score(0u);
        if (probs != nullptr) probs[b * k + tid] = prob_of(ord_score(0u), ml, lc);
      }
      return;
    }
  }
  constexpr int LPT = kSortedMergeMaxKeys / kMergeThreads;  // keys per thread at most
  uint64_t v[LPT];
#pragma unroll
  for (int j = 0; j < LPT; j++) {
    const int i = tid + kMergeThreads * j;
    v[j] = i < n ? c[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < LPT; j++) {
    const int i = tid + kMergeThreads * j;
    if (i < n) sk[i] = v[j];
  }
  __syncthreads();
  if (tid >= 64) return;
  uint64_t head[PL];
  int pos[PL];
#pragma unroll
  for (int j = 0; j < PL; j++) {
    const int l = lane + 64 * j;
    pos[j] = 0;
    head[j] = l < nl ? sk[l * k] : 0;
  }
  for (int t = 0; t < k; t++) {
    uint64_t m = 0;
#pragma unroll
    for (int j = 0; j < PL; j++) m = head[j] > m ? head[j] : m;
    const uint64_t best = wave_max_u64(m);
    if (lane == 0) {
      const float sc = ord_score((uint32_t)(best >> 32));
      ids[b * k + t] = (int32_t)(~(uint32_t)(best & 0xffffffffu));
      scores[b * k + t] = sc;
      if (probs != nullptr) probs[b * k + t] = prob_of(sc, ml, lc);
    }
#pragma unroll
    for (int j = 0; j < PL; j++) {
      if (best != 0 && head[j] == best) {  // keys are unique: one list owns it
        pos[j]++;
        head[j] = pos[j] < k ? sk[(lane + 64 * j) * k + pos[j]] : 0;
      }
    }
  }
}

static hipError_t launch_merge(const uint64_t* cand, int64_t batch, int n, int k, int32_t* ids, float* scores,
                               const float2* lse, int nparts, float c, float* probs, hipStream_t stream,
                               bool sorted) {
  const int nl = n / k;
  if (sorted && nl <= 1024 && n <= kSortedMergeMaxKeys) {
    const size_t lds = (size_t)n * 8;
#define ETG_SMERGE_CASE(PLV)                                                                                      \
  if (nl <= 64 * PLV) {                                                                                           \
    hipLaunchKernelGGL((topk_merge_sorted_kernel<PLV>), dim3((unsigned)batch), dim3(kMergeThreads), lds, stream,    \
                       cand, nl, k, ids, scores, lse, nparts, c, probs);                                          \
    return hipGetLastError();                                                                                     \
  }
    ETG_SMERGE_CASE(1)
    ETG_SMERGE_CASE(2)
    ETG_SMERGE_CASE(4)
    ETG_SMERGE_CASE(8)
    ETG_SMERGE_CASE(16)
#undef ETG_SMERGE_CASE
  }
  const dim3 grid((unsigned)batch), block(kMergeThreads);
  const int kpt = (n + kMergeThreads - 1) / kMergeThreads;
#define ETG_MERGE_CASE(KV)                                                                                     \
  if (kpt <= KV) {                                                                                             \
    hipLaunchKernelGGL((topk_merge_kernel<KV>), grid, block, 0, stream, cand, n, k, ids, scores, lse, nparts, c, \
                       probs);                                                                                 \
  }
  ETG_MERGE_CASE(1)
  else ETG_MERGE_CASE(2) else ETG_MERGE_CASE(4) else ETG_MERGE_CASE(8) else ETG_MERGE_CASE(16)
  else ETG_MERGE_CASE(32) else hipLaunchKernelGGL(topk_merge_wide_kernel, grid, block, 0, stream, cand, n, k, ids,
                                                   scores, lse, nparts, c, probs);
#undef ETG_MERGE_CASE
  return hipGetLastError();
}


template <int DT>
static hipError_t launch_valu(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                              const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid((unsigned)p.nblk, (unsigned)p.npass), block(256);
  hipError_t e = set_dynamic_lds((const void*)valu_logits_kernel<DT, 1>, p.lds_bytes);
  if (e == hipSuccess) e = set_dynamic_lds((const void*)valu_logits_kernel<DT, 2>, p.lds_bytes);
  if (e == hipSuccess) e = set_dynamic_lds((const void*)valu_logits_kernel<DT, 4>, p.lds_bytes);
  if (e == hipSuccess) e = set_dynamic_lds((const void*)valu_logits_kernel<DT, 8>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  switch (p.rb) {
#define ETG_VALU_CASE(RBV)                                                                          \
  case RBV:                                                                                         \
    hipLaunchKernelGGL((valu_logits_kernel<DT, RBV>), grid, block, p.lds_bytes, stream, t.rows, t.V, \
                       t.row_bytes, (int)t.hidden, R, (int)x.wire, p.batch, p.k, cand, x.logits, x.lse,    \
                       x.lse_scale);                                                                        \
    break;
    ETG_VALU_CASE(1)
    ETG_VALU_CASE(2)
    ETG_VALU_CASE(4)
    ETG_VALU_CASE(8)
#undef ETG_VALU_CASE
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

hipError_t launch_logits_topk(const TableDesc& t, const LogitsPlan& p, const void* R, int32_t* ids,
                              float* scores, void* ws, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                              float* logits, float* probs, float lse_scale, int32_t wire) {
  uint8_t* base = (uint8_t*)ws;
  uint64_t* cand = (uint64_t*)(base + p.cand_offset);
  LogitsExtras x;
  x.logits = logits;
  x.lse = probs != nullptr ? (float2*)(base + p.lse_offset) : nullptr;
  x.lse_scale = lse_scale;
  x.aux = base + p.aux_offset;
  x.wire = wire;
  hipError_t e;
  if (p.path == 2) {
    e = launch_stream(t, p, R, cand, x, stream, ev0, ev1);
  } else if (p.path == 3) {
    e = launch_gemm(t, p, R, base + p.img_offset, cand, x, stream, ev0, ev1);
  } else if (p.path == 4) {
    e = launch_wide(t, p, R, base + p.img_offset, cand, (uint64_t*)(base + p.aux_offset), x, stream, ev0, ev1);
  } else if (p.path == 5) {
    e = launch_q8(t, p, R, cand, x, stream, ev0, ev1);
  } else if (p.path == 6) {
    e = launch_row(t, p, R, cand, x, stream, ev0, ev1);
  } else if (p.path == 7) {
    if (ids == nullptr || probs != nullptr || logits != nullptr) return hipErrorInvalidValue;
    return launch_rank(t, p, R, base + p.img_offset, cand, x, ids, scores, stream, ev0, ev1);
  } else {
    switch (t.dtype) {
      case DT_F32: e = launch_valu<DT_F32>(t, p, R, cand, x, stream, ev0, ev1); break;
      case DT_BF16: e = launch_valu<DT_BF16>(t, p, R, cand, x, stream, ev0, ev1); break;
      case DT_F16: e = launch_valu<DT_F16>(t, p, R, cand, x, stream, ev0, ev1); break;
      default: e = launch_valu<DT_Q8_0>(t, p, R, cand, x, stream, ev0, ev1); break;
    }
  }
  if (e != hipSuccess || ids == nullptr) return e;
  // every path but the split contraction (heaps) emits each block's keys best first
  return launch_merge(cand, p.batch, p.ncand, p.k, ids, scores, x.lse, p.nparts, lse_scale, probs, stream,
                      p.path != 3);
}

// ---------------------------------------------------------------------------
// Planning (host only, no device calls).
// ---------------------------------------------------------------------------
// Smallest bf16 batch the automatic choice sends to the rank path (top-k only).
static constexpr int64_t kRankMinBatch = 17;

int32_t plan_logits(const TableDesc& t, int64_t batch, int32_t k, int32_t path, LogitsPlan* p,
                    const char** why, bool extras) {
  *p = LogitsPlan{};
  p->k = k;
  p->batch = batch;
  // auto, bf16 tables past kRankMinBatch residual rows: the rank path for the
  // top-k alone, the wide kernel (up to 64 rows) or the split contraction when
  // probabilities or raw logits are wanted; the workspace covers both
  if (path == 0 && t.dtype == DT_BF16 && batch >= kRankMinBatch) {
    LogitsPlan r, g;
    const char* w = "";
    const bool rank_ok = plan_logits(t, batch, k, 7, &r, &w, false) == 0;
    const int32_t st = plan_logits(t, batch, k, batch > 64 ? 3 : 4, &g, why, false);
    if (st != 0) return st;
    *p = (rank_ok && !extras) ? r : g;
    if (rank_ok) p->ws_bytes = std::max(r.ws_bytes, g.ws_bytes);
    return 0;
  }
  // auto: bf16 tables stream for up to 64 residual rows (one table pass per 8
  // or per 64 rows), then switch to the tiled contraction
  // auto: Q8_0 tables take the q8 path and f32 / f16 tables the row path (passes of
  // 2 residual rows) when the row fits it, else the VALU path
  if (path == 0 && t.dtype != DT_BF16) {
    LogitsPlan q;
    const char* w = "";
    if (t.dtype == DT_Q8_0) path = plan_q8(t, batch, k, &q, &w) == 0 ? 5 : 1;
    else path = plan_row(t, batch, k, &q, &w) == 0 ? 6 : 1;
  }
  if (path == 0) path = (t.dtype != DT_BF16) ? 1 : (batch <= 8 ? 2 : 4);
  if ((path == 2 || path == 3 || path == 4) && t.dtype != DT_BF16) {
    *why = "the stream, gemm and wide paths need a bf16 table";
    return -5;
  }
  if (path == 5 && t.dtype != DT_Q8_0) {
    *why = "the q8 path needs a Q8_0 table";
    return -5;
  }
  if (path == 7 && t.dtype != DT_BF16) {
    *why = "the rank path needs a bf16 table";
    return -5;
  }
  if (path == 7 && extras) {
    *why = "the rank path returns neither probabilities nor raw logits";
    return -5;
  }
  if (path < 1 || path > 7) {
    *why = "unknown path";
    return -5;
  }
  p->path = path;
  int32_t st = 0;
  if (path == 2) {
    st = plan_stream(t, batch, k, p, why);
  } else if (path == 4) {
    st = plan_wide(t, batch, k, p, why);
  } else if (path == 3) {
    st = plan_gemm(t, batch, k, p, why);
  } else if (path == 5) {
    st = plan_q8(t, batch, k, p, why);
  } else if (path == 6) {
    st = plan_row(t, batch, k, p, why);
  } else if (path == 7) {
    st = plan_rank(t, batch, k, p, why);
  } else {
    p->rb = batch >= 8 ? 8 : batch >= 4 ? 4 : batch >= 2 ? 2 : 1;
    p->npass = (int32_t)cdiv(batch, p->rb);
    // at most 4096 rows per block (16 KiB of logits per residual row in the pass)
    int64_t nblk = std::max<int64_t>(cdiv(t.V, 64), 1);
    nblk = std::min<int64_t>(nblk, 4 * kTargetBlocks);
    nblk = std::max<int64_t>(nblk, cdiv(t.V * p->rb, 16384));
    p->nblk = (int32_t)nblk;
    p->rows_per_blk = cdiv(t.V, nblk);
    p->lds_bytes = (size_t)p->rows_per_blk * p->rb * 4;
    p->img_bytes = 0;
    p->ncand = p->nblk * k;
  }
  if (st != 0) return st;
  p->img_offset = 0;
  p->cand_offset = align_up(p->img_bytes, 256);
  p->cand_bytes = (size_t)batch * p->ncand * 8;
  p->aux_offset = align_up(p->cand_offset + p->cand_bytes, 256);
  p->nparts = p->ncand / k;
  p->lse_offset = align_up(p->aux_offset + p->aux_bytes, 256);
  p->lse_bytes = (size_t)batch * p->nparts * 8;
  p->ws_bytes = align_up(p->lse_offset + p->lse_bytes, 256);
  return 0;
}

}  // namespace etg
