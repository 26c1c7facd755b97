// Rank path (ADR-0008 "POST /v1/logits", the top_k answer): the certified
// rescoring that completes the ranking kernels of gemm.hip (batches past 64 rows)
// and wide.hip (up to 64), and the reduction of the table row norms they measure.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// Squared row norms from the column tiles' parts npart [ngrp][V]; block x writes
// the largest of its rows' norms to nrm2[x].
__global__ void __launch_bounds__(256) rank_norm_kernel(const float* __restrict__ npart, int ngrp, int64_t V,
                                                        float* __restrict__ nrm2) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  float m = 0.f;
  for (int j = 0; j < kRankNormRows / 256; j++) {
    const int64_t v = (int64_t)blockIdx.x * kRankNormRows + j * 256 + tid;
    if (v < V) {
      float sum = 0.f;
      for (int g = 0; g < ngrp; g++) sum += npart[(int64_t)g * V + v];
      m = fmaxf(m, sum);
    }
  }
  m = wave_max_f32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) nrm2[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

hipError_t launch_rank_norm(const float* npart, int ngrp, int64_t V, float* nrm2, hipStream_t stream) {
  hipLaunchKernelGGL(rank_norm_kernel, dim3((unsigned)cdiv(V, kRankNormRows)), dim3(256), 0, stream, npart, ngrp, V,
                     nrm2);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ranking mode: exact rescoring with a certificate.
//
// In ranking mode the contraction sees hi = bf16(r) only, so its value a_v for
// table row e_v misses lo . e_v (lo = r - hi, exact in f32) and carries the f32
// accumulation error of hi . e_v (its products of two bf16 values are exact).
// By Cauchy-Schwarz, with N >= max_v |e_v| measured by the contraction,
//   |a_v - r . e_v| <= (|lo| + g |hi|) N = slack,   g = kpad 2^-22
// (g allows a few ulp of accumulation error per term).  Each candidate is then
// rescored from the f32 residual (lane-strided f32 FMAs and a butterfly sum),
// which is within eps = (hidden / 64 + 8) 2^-23 |r| N of r . e_v.
//
// One workgroup per residual row:
//  * U = the heap keys of every vocabulary range (kb per range, approximate);
//  * A = the k-th largest approximate logit in U (-inf with fewer than k keys);
//  * phase 1 rescores the keys of U with a_v >= lo1 = A - 9/8 slack - 2 eps (the
//    window phase 2 will want, guessed from A), and T1 is the k-th largest
//    rescored value (-inf with fewer than k);
//  * thr = T1 - slack - 2 eps;
//  * a range whose heap is full and whose smallest kept key reaches thr may have
//    dropped a row above thr: all its rows are rescored;
//  * every other key of U with thr <= a_v < lo1 is rescored (none unless T1 fell
//    more than slack / 8 below A);
//  * the answer is the k best rescored keys (logit desc, id asc; a row rescored
//    twice enters a heap once).
// Why this is the top-k: the final k-th rescored value T >= T1.  A row that is
// not rescored has a_v < thr (dropped rows lie at or below their range's
// smallest kept key), so r . e_v < thr + slack = T1 - 2 eps <= T - 2 eps, below
// the exact logit of every selected row (each >= T - eps).
// ---------------------------------------------------------------------------
// Waves per residual row, rows per wave and 1 KiB chunk loads per row in flight:
// 4 waves x 2 rows x 6 chunks for large batches (with the LDS below, four or more
// residual rows share a CU, so a 1,024-row batch is rescored in one round, bound
// by HBM); 16 waves x 2 rows x 6 chunks for batches of up to kRescoreWideBatch
// rows (few workgroups, each latency-bound: 32 rows are rescored in one round of
// rows; more chunks or rows per wave in flight measured no faster, as the time
// goes to first touches of randomly placed table rows).
static constexpr int kRescoreWideBatch = 256;

// LDS of rank_rescore_kernel: U [n rounded up to even] keys, heaps [waves][k]
// keys, the residual [hidden rounded up to 8] f32, S [n] rows, flags [nvr],
// rescan list [nvr].  Rounding n up keeps the residual 16-byte aligned (the
// rescoring reads it as f32x4; the wave counts are even).
static size_t rescore_lds_bytes(int64_t hidden, int n, int nvr, int k, int nw) {
  return (size_t)((n + 1) & ~1) * 8 + (size_t)nw * k * 8 + (size_t)((hidden + 7) & ~7) * 4 + (size_t)n * 4 +
         (size_t)nvr * 8;
}

int32_t rescore_waves(int64_t batch) { return batch <= kRescoreWideBatch ? 16 : 4; }

size_t rescore_lds(int64_t hidden, int n, int nvr, int k, int64_t batch) {
  return rescore_lds_bytes(hidden, n, nvr, k, rescore_waves(batch));
}

// Order value of the k-th largest key among the nonzero keys U[0, n) (counted
// with multiplicity), or 0 with fewer than k.  Radix selection, 8 bits per
// pass from the top, counts in an LDS histogram; NT threads.
template <int NT>
__device__ uint32_t block_kth_ord(const uint64_t* U, int n, int k, uint32_t* hist, uint32_t* sel) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint64_t key = U[i];
      const uint32_t o = (uint32_t)(key >> 32);
      if (key != 0 && (o & pmask) == prefix) atomicAdd(&hist[(o >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l takes bins 255 - 4 l - j (j < 4), largest first
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        c[j] = hist[255 - 4 * lane - j];
        sum += c[j];
      }
      uint32_t inc = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
      }
      const uint64_t m = __ballot(inc >= kk);
      if (m == 0) {
        if (lane == 0) sel[0] = 0xffffffffu;
      } else if (lane == __builtin_ctzll(m)) {
        uint32_t cum = inc - sum;
        int j = 0;
        while (j < 3 && cum + c[j] < kk) cum += c[j++];
        sel[0] = (uint32_t)(255 - 4 * lane - j);
        sel[1] = kk - cum;
      }
    }
    __syncthreads();
    const uint32_t bin = sel[0], rest = sel[1];
    __syncthreads();  // sel and hist are rewritten by the next pass
    if (bin == 0xffffffffu) return 0u;
    prefix |= bin << shift;
    pmask |= 255u << shift;
    kk = rest;
  }
  return prefix;
}

// Order value of the k-th largest key of nl lists of kb keys each (each list in
// descending order, empty slots 0 at its end), or 0 with fewer than k keys: k
// rounds of taking the largest list head (keys are unique, so one list owns it).
// One wave; lane l keeps the heads of lists l + 64 j, j < PL.
template <int PL>
__device__ uint32_t wave_kth_sorted(const uint64_t* U, int nl, int kb, int k) {
  const int lane = threadIdx.x & 63;
  uint64_t head[PL];
  int pos[PL];
#pragma unroll
  for (int j = 0; j < PL; j++) {
    const int l = lane + 64 * j;
    pos[j] = 0;
    head[j] = l < nl ? U[l * kb] : 0;
  }
  uint64_t best = 0;
  for (int t = 0; t < k; t++) {
    uint64_t m = 0;
#pragma unroll
    for (int j = 0; j < PL; j++) m = head[j] > m ? head[j] : m;
    best = wave_max_u64(m);
    if (best == 0) return 0u;
#pragma unroll
    for (int j = 0; j < PL; j++) {
      if (head[j] == best) {
        pos[j]++;
        head[j] = pos[j] < kb ? U[(lane + 64 * j) * kb + pos[j]] : 0;
      }
    }
  }
  return (uint32_t)(best >> 32);
}

// The k largest keys of src[0, c) (k rounds of wave maxima; a key present twice
// counts once), written to top[0, k) in descending order with 0 past the last
// one (top may be null); returns the order value of the k-th, or 0 with fewer
// than k keys.  One wave; lane l takes keys l + 64 j, j < PL (c <= 64 PL).  With
// idx, key i is src[idx[i]].
template <int PL>
__device__ uint32_t wave_top_keys(const uint64_t* src, const uint32_t* idx, int c, int k, uint64_t* top) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PL];
#pragma unroll
  for (int j = 0; j < PL; j++) {
    const int i = lane + 64 * j;
    key[j] = i < c ? src[idx != nullptr ? idx[i] : i] : 0;
  }
  uint64_t best = 0;
  for (int t = 0; t < k; t++) {
    best = wave_pop_max(key);
    if (top != nullptr && lane == 0) top[t] = best;
  }
  return (uint32_t)(best >> 32);
}

// wave_top_keys with the register count chosen for c keys (c <= 1024).
__device__ __forceinline__ uint32_t wave_top_keys_any(const uint64_t* src, const uint32_t* idx, int c, int k,
                                                      uint64_t* top) {
  if (c <= 64) return wave_top_keys<1>(src, idx, c, k, top);
  if (c <= 128) return wave_top_keys<2>(src, idx, c, k, top);
  if (c <= 256) return wave_top_keys<4>(src, idx, c, k, top);
  if (c <= 512) return wave_top_keys<8>(src, idx, c, k, top);
  return wave_top_keys<16>(src, idx, c, k, top);
}

// Most candidate keys the selections below rank at once, and the largest k for
// which the rescoring selects that way (else by radix selection).
static constexpr int kSelMaxCand = 512;
static constexpr int kSelSmallK = 16;

// The k largest of the c distinct keys src[idx[i]] (0 = no key), c <= kSelMaxCand,
// into fin[0, k) in descending order with 0 past the last; returns the order
// value of the k-th, or 0 with fewer than k.  Each key's rank is the number of
// larger keys, counted by NT / c threads per key over a share of the others
// (no serial rounds).  rk [c] is LDS scratch; every thread of the block calls it.
template <int NT>
__device__ uint32_t block_top_distinct(const uint64_t* src, const uint32_t* idx, int c, int k, uint32_t* rk,
                                       uint64_t* fin) {
  const int tid = threadIdx.x;
  for (int i = tid; i < c; i += NT) rk[i] = 0;
  for (int t = tid; t < k; t += NT) fin[t] = 0;
  __syncthreads();
  if (c > 0) {
    const int parts = c <= NT ? NT / c : 1;
    for (int p = tid; p < c * parts; p += NT) {
      const int i = p % c, part = p / c;
      const uint64_t ki = src[idx[i]];
      uint32_t n = 0;
      for (int j = part; j < c; j += parts) n += src[idx[j]] > ki ? 1u : 0u;
      if (n != 0) atomicAdd(&rk[i], n);
    }
  }
  __syncthreads();
  for (int i = tid; i < c; i += NT) {
    const uint64_t key = src[idx[i]];
    if (key != 0 && rk[i] < (uint32_t)k) fin[rk[i]] = key;
  }
  __syncthreads();
  return (uint32_t)(fin[k - 1] >> 32);
}

// Order value of the k-th largest nonzero key of U[0, n) (ranges of kb keys; keys
// unique), or 0 with fewer than k, without serial rounds over U:
//  * thread t takes the largest key of ranges t, t + NT, ...; 16-lane rows reduce
//    theirs by DPP, and row x joins group x % k;
//  * L = the smallest of the k group maxima.  They are k distinct keys, all >= L,
//    so the k-th largest key is >= L too (an empty group gives L = 0: every key
//    qualifies);
//  * C = the keys >= L, listed by index in idx (for random scores about 3 k);
//  * the k largest of C are ranked as above (fin receives them).
// Returns false, with nothing selected, when C holds more than kSelMaxCand keys.
// gmax [k], idx [n], rk [kSelMaxCand], fin [k] are LDS scratch; every thread of
// the block calls it.
template <int NT>
__device__ bool block_kth_small(const uint64_t* U, int n, int kb, int k, uint64_t* gmax, uint32_t* idx,
                                uint32_t* cnt, uint32_t* rk, uint64_t* fin, uint32_t* ord) {
  const int tid = threadIdx.x;
  for (int g = tid; g < k; g += NT) gmax[g] = 0;
  if (tid == 0) cnt[0] = 0;
  __syncthreads();
  uint64_t m = 0;
  for (int i = tid * kb; i < n; i += NT * kb)
    for (int j = 0; j < kb; j++) m = max(m, U[i + j]);
  m = dpp_max_u64<0x111, 0xf>(m);  // row_shr:1, 2, 4, 8: lane 15 of the row holds its maximum
  m = dpp_max_u64<0x112, 0xf>(m);
  m = dpp_max_u64<0x114, 0xf>(m);
  m = dpp_max_u64<0x118, 0xf>(m);
  if ((tid & 15) == 15 && m != 0) atomicMax((unsigned long long*)&gmax[(tid >> 4) % k], (unsigned long long)m);
  __syncthreads();
  uint64_t L = ~0ull;
  for (int g = 0; g < k; g++) L = min(L, gmax[g]);
  for (int i = tid; i < n; i += NT) {
    const uint64_t key = U[i];
    if (key != 0 && key >= L) idx[atomicAdd(&cnt[0], 1u)] = (uint32_t)i;
  }
  __syncthreads();
  const int c = (int)cnt[0];
  __syncthreads();  // every thread has read the count
  if (c > kSelMaxCand) return false;
  *ord = block_top_distinct<NT>(U, idx, c, k, rk, fin);
  return true;
}

// f32 value rounded toward -inf from a finite double.
__device__ __forceinline__ float f32_round_down(double x) {
  float f = (float)x;
  if ((double)f > x) {
    const uint32_t u = __float_as_uint(f);
    f = f > 0.f ? __uint_as_float(u - 1u) : f < 0.f ? __uint_as_float(u + 1u) : -__uint_as_float(1u);
  }
  return f;
}

//  table   bf16 [V][hidden], row_bytes = 2 hidden (a multiple of 16)
//  R       residual rows (wire format `wire`)
//  cand    [B][nvr][kb] candidate keys of the ranking kernel per range of
//          range_rows table rows (unordered, 0 = empty; a range with fewer than kb
//          keys kept every row it has)
//  nrm2    [nnrm] largest squared row norms of blocks of table rows
//  kpad    terms the ranking kernel accumulated per logit
//  sorted  each range's keys are in descending order (the wide kernel's lists)
//  ids, scores  [B][k] the answer, best first
template <int NW, int ROWS, int CH>
__global__ void __launch_bounds__(64 * NW) rank_rescore_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden, int kpad,
    const void* __restrict__ R, int wire, const uint64_t* __restrict__ cand, int nvr, int kb, int64_t range_rows,
    const float* __restrict__ nrm2, int nnrm, int k, int32_t* __restrict__ ids, float* __restrict__ scores,
    int sorted) {
  static_assert(NW % 2 == 0, "the residual's LDS offset must stay 16-byte aligned");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float red[NW][4];
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];  // also gmax [k] and fin [k] keys below
  __shared__ uint32_t sel[2];
  __shared__ uint32_t cnt[2];  // rows in S, ranges to rescan
  __shared__ uint32_t scnt[1];
  __shared__ uint32_t rk[kSelMaxCand];
  const int n = nvr * kb;
  uint64_t* U = (uint64_t*)smem;
  uint64_t* heaps = U + ((n + 1) & ~1);                       // [waves][k], 16-byte aligned
  float* r = (float*)(heaps + NW * k);                         // [hidden], 16-byte aligned (NW is even)
  uint32_t* S = (uint32_t*)(r + ((hidden + 7) & ~7));          // [n]
  uint32_t* flag = S + n;                                      // [nvr] 1: rescanned
  uint32_t* rl = flag + nvr;                                   // [nvr]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;

  // residual row and the squared norms of lo, hi and r
  float s_lo = 0.f, s_hi = 0.f, s_r = 0.f, n2 = 0.f;
  auto take = [&](int c, float x) {
    r[c] = x;
    const float hi = __uint_as_float(bf16_rne(x) << 16);
    const float lo = x - hi;  // exact
    s_lo = __builtin_fmaf(lo, lo, s_lo);
    s_hi = __builtin_fmaf(hi, hi, s_hi);
    s_r = __builtin_fmaf(x, x, s_r);
  };
  if (wire == WIRE_F32 && ((uintptr_t)R & 15) == 0) {  // hidden is a multiple of 8: 16-byte rows
    const f32x4* src = (const f32x4*)((const float*)R + b * hidden);
    for (int c4 = tid; c4 < hidden / 4; c4 += (64 * NW)) {
      const f32x4 x = src[c4];
      take(4 * c4, x.x);
      take(4 * c4 + 1, x.y);
      take(4 * c4 + 2, x.z);
      take(4 * c4 + 3, x.w);
    }
  } else {
    for (int c = tid; c < hidden; c += (64 * NW)) take(c, residual_value(R, wire, b, hidden, c));
  }
  for (int i = tid; i < nnrm; i += (64 * NW)) n2 = fmaxf(n2, nrm2[i]);
  for (int i = tid; i < n; i += (64 * NW)) U[i] = cand[b * n + i];
  for (int i = tid; i < NW * k; i += (64 * NW)) heaps[i] = 0;
  if (tid == 0) cnt[0] = cnt[1] = 0;
  s_lo = wave_sum(s_lo);
  s_hi = wave_sum(s_hi);
  s_r = wave_sum(s_r);
  n2 = wave_max_f32(n2);
  if (lane == 0) {
    red[wv][0] = s_lo;
    red[wv][1] = s_hi;
    red[wv][2] = s_r;
    red[wv][3] = n2;
  }
  __syncthreads();
  double lo2 = 0, hi2 = 0, r2 = 0, nn2 = 0;
  for (int w = 0; w < NW; w++) {
    lo2 += red[w][0];
    hi2 += red[w][1];
    r2 += red[w][2];
    nn2 = fmax(nn2, (double)red[w][3]);
  }
  // the f32 sums above are within a few hundred ulp of the exact ones: inflate
  // them by 2^-10 (sums of squares) before the square roots; the row norms
  // (up to kpad / 4 roundings per lane) by 2^-9
  const double inf2 = 1.0 + 0x1p-10;
  const double N = sqrt(nn2 * (1.0 + 0x1p-9));
  // inputs or products below the f32 normal range (flushed to zero or not)
  const double tiny = 0x1p-100 * ((double)kpad + sqrt((double)kpad) * (N + sqrt(hi2 * inf2) + sqrt(r2 * inf2)));
  const double slack = (sqrt(lo2 * inf2) + (double)kpad * 0x1p-22 * sqrt(hi2 * inf2)) * N + tiny;
  const double eps = ((double)hidden / 64.0 + 8.0) * 0x1p-23 * sqrt(r2 * inf2) * N + tiny;

  // k <= kSelSmallK: the selections take k rounds of wave maxima over a few
  // registers per lane; the k best rescored keys of phase 1 are kept in fin.
  const bool small = k <= kSelSmallK;
  uint64_t* gmax = (uint64_t*)hist;
  uint64_t* fin = (uint64_t*)(hist + 128);
  uint32_t a_ord = 0;
  if (small && block_kth_small<64 * NW>(U, n, kb, k, gmax, S, scnt, rk, fin, &a_ord)) {
  } else if (sorted && nvr <= 512) {
    if (wv == 0) {
      const uint32_t o = nvr <= 64    ? wave_kth_sorted<1>(U, nvr, kb, k)
                         : nvr <= 128 ? wave_kth_sorted<2>(U, nvr, kb, k)
                         : nvr <= 256 ? wave_kth_sorted<4>(U, nvr, kb, k)
                                      : wave_kth_sorted<8>(U, nvr, kb, k);
      if (lane == 0) sel[0] = o;
    }
    __syncthreads();
    a_ord = sel[0];
    __syncthreads();  // sel is reused
  } else {
    a_ord = block_kth_ord<64 * NW>(U, n, k, hist, sel);
  }
  const float A = a_ord == 0u ? -__builtin_inff() : ord_score(a_ord);

  // One wave per row: f32 FMAs over values 8 lane + 512 j + e (j ascending), then
  // a butterfly; every lane holds the same key, and the wave checks its heap for
  // it.  A wave takes ROWS rows at a time and issues CH 1 KiB loads of each
  // together (the last block's loads past hidden read the row's last chunk and are
  // not used), so each row's sum has the same order whatever ROWS and CH are.
  uint64_t* hp = heaps + wv * k;
  auto insert = [&](float acc, int64_t v) {
    const uint64_t key = make_key(acc, (uint32_t)v);
    if (key > hp[0] && __ballot(lane < k && hp[lane] == key) == 0 && lane == 0) heap_replace_root(hp, k, key);
  };
  auto rescore_rows = [&](const int64_t (&v)[ROWS]) {  // v[j] < 0: no row (v[0] is a row)
    const uint8_t* row[ROWS];
    float acc[ROWS];
#pragma unroll
    for (int j = 0; j < ROWS; j++) {
      row[j] = table + (uint64_t)(v[j] >= 0 ? v[j] : v[0]) * (uint64_t)row_bytes;
      acc[j] = 0.f;
    }
    for (int c0 = 8 * lane; c0 < hidden; c0 += 512 * CH) {
      u32x4 w[ROWS][CH];
#pragma unroll
      for (int q = 0; q < CH; q++) {
        const int c = min(c0 + 512 * q, hidden - 8);
#pragma unroll
        for (int j = 0; j < ROWS; j++) w[j][q] = *(const u32x4*)(row[j] + 2 * c);
      }
#pragma unroll
      for (int q = 0; q < CH; q++) {
        const int c = c0 + 512 * q;
        if (c < hidden) {
          const f32x4 x0 = *(const f32x4*)(r + c), x1 = *(const f32x4*)(r + c + 4);
#pragma unroll
          for (int j = 0; j < ROWS; j++) {
            acc[j] = __builtin_fmaf(bf16_lo(w[j][q].x), x0.x, acc[j]);
            acc[j] = __builtin_fmaf(bf16_hi(w[j][q].x), x0.y, acc[j]);
            acc[j] = __builtin_fmaf(bf16_lo(w[j][q].y), x0.z, acc[j]);
            acc[j] = __builtin_fmaf(bf16_hi(w[j][q].y), x0.w, acc[j]);
            acc[j] = __builtin_fmaf(bf16_lo(w[j][q].z), x1.x, acc[j]);
            acc[j] = __builtin_fmaf(bf16_hi(w[j][q].z), x1.y, acc[j]);
            acc[j] = __builtin_fmaf(bf16_lo(w[j][q].w), x1.z, acc[j]);
            acc[j] = __builtin_fmaf(bf16_hi(w[j][q].w), x1.w, acc[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ROWS; j++) acc[j] = wave_sum(acc[j]);
#pragma unroll
    for (int j = 0; j < ROWS; j++)
      if (v[j] >= 0) insert(acc[j], v[j]);
  };
  // rows S[i], S[i + NW], ... of a list, ROWS at a time per wave
  auto rescore_list = [&](int cnt) {
    for (int i = wv; i < cnt; i += ROWS * NW) {
      int64_t v[ROWS];
#pragma unroll
      for (int j = 0; j < ROWS; j++) v[j] = i + j * NW < cnt ? (int64_t)S[i + j * NW] : -1;
      rescore_rows(v);
    }
  };

  // phase 1: the keys of U at or above lo1
  const float lo1 = a_ord == 0u ? -__builtin_inff() : f32_round_down((double)A - 1.125 * slack - 2.0 * eps);
  for (int i = tid; i < n; i += (64 * NW)) {
    const uint64_t key = U[i];
    if (key != 0 && ord_score((uint32_t)(key >> 32)) >= lo1) S[atomicAdd(&cnt[0], 1u)] = ~(uint32_t)key;
  }
  __syncthreads();
  const int ns1 = (int)cnt[0];
  rescore_list(ns1);
  __syncthreads();
  if (tid == 0) cnt[0] = 0;
  uint32_t t_ord;
  if (small) {
    // the rescored keys of phase 1 (distinct rows, at most ns1 <= n of them), listed in S
    if (tid == 0) scnt[0] = 0;
    __syncthreads();
    for (int i = tid; i < NW * k; i += (64 * NW))
      if (heaps[i] != 0) S[atomicAdd(&scnt[0], 1u)] = (uint32_t)i;
    __syncthreads();
    t_ord = block_top_distinct<64 * NW>(heaps, S, (int)scnt[0], k, rk, fin);
  } else {
    t_ord = block_kth_ord<64 * NW>(heaps, NW * k, k, hist, sel);
  }
  const float thr =
      t_ord == 0u ? -__builtin_inff() : f32_round_down((double)ord_score(t_ord) - slack - 2.0 * eps);

  // phase 2: ranges to rescan (a full heap whose smallest key reaches thr), then
  // the keys of U in [thr, lo1) outside them
  for (int vr = tid; vr < nvr; vr += (64 * NW)) {
    uint64_t mn = ~0ull;
    for (int j = 0; j < kb; j++) mn = min(mn, U[vr * kb + j]);
    const bool rescan = mn != 0 && ord_score((uint32_t)(mn >> 32)) >= thr;
    flag[vr] = rescan;
    if (rescan) rl[atomicAdd(&cnt[1], 1u)] = (uint32_t)vr;
  }
  __syncthreads();
  for (int i = tid; i < n; i += (64 * NW)) {
    const uint64_t key = U[i];
    if (key == 0 || flag[i / kb] != 0) continue;
    const float a = ord_score((uint32_t)(key >> 32));
    if (a >= thr && a < lo1) S[atomicAdd(&cnt[0], 1u)] = ~(uint32_t)key;
  }
  __syncthreads();
  const int ns = (int)cnt[0], nres = (int)cnt[1];
  rescore_list(ns);
  for (int q = 0; q < nres; q++) {
    const int64_t v0 = (int64_t)rl[q] * range_rows, v1 = min(V, v0 + range_rows);
    for (int64_t v = v0 + wv; v < v1; v += ROWS * NW) {
      int64_t vs[ROWS];
#pragma unroll
      for (int j = 0; j < ROWS; j++) vs[j] = v + j * NW < v1 ? v + j * NW : -1;
      rescore_rows(vs);
    }
  }
  __syncthreads();
  // the answer: fin still holds it when phase 2 rescored nothing
  if (!(small && ns == 0 && nres == 0)) {
    if (wv == 0) wave_top_keys_any(heaps, nullptr, NW * k, k, fin);
    __syncthreads();
  }
  for (int t = tid; t < k; t += (64 * NW)) {
    const uint64_t best = fin[t];
    ids[b * k + t] = (int32_t)(~(uint32_t)(best & 0xffffffffu));
    scores[b * k + t] = ord_score((uint32_t)(best >> 32));
  }
}

hipError_t launch_rescore(const TableDesc& t, const LogitsPlan& p, const void* R, int wire, const uint64_t* cand,
                          int nranges, int64_t range_rows, const float* nrm2, int nnrm, int kpad, int32_t* ids,
                          float* scores, hipStream_t stream, int sorted) {
  const int nw = rescore_waves(p.batch);
  const void* fn = nw == 16 ? (const void*)rank_rescore_kernel<16, 2, 6> : (const void*)rank_rescore_kernel<4, 2, 6>;
  hipError_t e = set_dynamic_lds(fn, p.rescore_lds);
  if (e != hipSuccess) return e;
  if (nw == 16) {
    hipLaunchKernelGGL((rank_rescore_kernel<16, 2, 6>), dim3((unsigned)p.batch), dim3(64 * 16), p.rescore_lds, stream, t.rows,
                       t.V, t.row_bytes, (int)t.hidden, kpad, R, wire, cand, nranges, p.kb, range_rows, nrm2, nnrm, p.k,
                       ids, scores, sorted);
  } else {
    hipLaunchKernelGGL((rank_rescore_kernel<4, 2, 6>), dim3((unsigned)p.batch), dim3(64 * 4), p.rescore_lds, stream, t.rows,
                       t.V, t.row_bytes, (int)t.hidden, kpad, R, wire, cand, nranges, p.kb, range_rows, nrm2, nnrm, p.k,
                       ids, scores, sorted);
  }
  return hipGetLastError();
}

}  // namespace etg
