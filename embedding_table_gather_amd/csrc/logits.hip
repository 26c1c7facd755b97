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
//  * valu:   any dtype (f32, bf16, Q8_0); f32 FMAs per lane, one table pass per
//    up to 8 residual rows.
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
// the fp32 residual rows of this pass.  Image slot (s, im, lane) holds the 8
// values of B column n = lane % 16, K-group g = lane / 16 (layout above).
template <int NIMG>
__device__ __forceinline__ void stream_stage_image(u32x4* simg, const float* __restrict__ R, int64_t B,
                                                   int hidden, int64_t b0, int c0, int n) {
  constexpr int NBC = NIMG == 1 ? 4 : 8;
  for (int i = threadIdx.x; i < n * NIMG * 64; i += blockDim.x) {
    const int lane = i & 63;
    const int q = i >> 6;
    const int im = q % NIMG;
    const int s = c0 + q / NIMG;
    const int nn = lane & 15, g = lane >> 4;
    const int h = nn >> 3, j8 = nn & 7;
    const int part = NIMG == 1 ? j8 / NBC : im;
    const int64_t b = b0 + j8 % NBC;
    const int cbase = 64 * s + 16 * g + 8 * h;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int c = cbase + e;
      const float x = (b < B && c < hidden) ? R[b * hidden + c] : 0.0f;
      const uint32_t hi = bf16_rne(x);
      // part 1 carries the remainder x - hi (exact in f32), rounded to bf16
      v[e] = part == 1 ? bf16_rne(x - __uint_as_float(hi << 16)) : hi;
    }
    simg[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
  }
}

template <int NBC>
__device__ __forceinline__ void stream_store_group(f32x4 acc, float* dst, int lane) {
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; i++) y[i] = acc[i] + __shfl(acc[i], (lane + 40) & 63, 64);
  if (NBC == 4) {
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = y[i] + __shfl(y[i], (lane + 4) & 63, 64);
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

// One pass over the table for NBC residual rows (pass = blockIdx.y).
//  table      bf16 [V][hidden], row_bytes = 2 * hidden
//  R          fp32 [B][hidden]
//  steps      64-value K steps, ceil(hidden / 64)
//  chunk      K steps staged in LDS at a time (a multiple of the unroll)
// Out-of-range rows and K positions are read from clamped in-range addresses and
// meet zero residual values or are never ranked, so no load is predicated (table
// entries are assumed finite).
template <int NIMG>
__global__ void __launch_bounds__(1024) stream_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden,
    const float* __restrict__ R, int64_t B, int steps, int chunk, int k, uint64_t* __restrict__ cand,
    int64_t ngroups, int max_groups) {
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

  // Waves own contiguous runs of group pairs (16 rows); only the last pair of the
  // table can be half empty.
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
  const int r = lane & 7, ck = lane >> 3;
  const int64_t last_off = row_bytes - 16;

  f32x4 acc0[kStreamMaxPairs], acc1[kStreamMaxPairs];
#pragma unroll
  for (int p = 0; p < kStreamMaxPairs; p++) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < steps; c0 += chunk) {
    const int c1 = min(steps, c0 + chunk);
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    stream_stage_image<NIMG>(simg, R, B, hidden, b0, c0, c1 - c0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kStreamMaxPairs; p++) {
      if (p < npairs) {
        const int64_t row0 = min((g_begin + 2 * p) * 8 + r, V - 1);
        const int64_t row1 = min((g_begin + 2 * p) * 8 + 8 + r, V - 1);
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

  if (wv < NBC && b0 + wv < B) {
    uint64_t* out = cand + ((b0 + wv) * gridDim.x + blockIdx.x) * (int64_t)k;
    stream_block_topk<NBC>(slog, sg0, sng, wv, lane, max_groups, V, k, out);
  }
}

// ---------------------------------------------------------------------------
// Wide stream path: bf16 tables, batches beyond the stream path's 8 rows.
//
// Still one HBM pass over the table per pass of up to 64 residual rows, with
// the table read straight into VGPRs; the residual operand comes from LDS.
// A block owns 512 table rows (8 waves x 4 M-tiles of 16 rows).
//
// Loads: per 16-row M-tile and 64-value K step, two load instructions X (rows
// 0-7) and Y (rows 8-15); lane l reads row l % 8 of its half, 16-byte chunk
// l / 8 of the 128-byte step, so each instruction reads 8 whole 128-byte lines.
// Two DPP moves per dword exchange the upper 8 lanes of each 16-lane row of X
// with the lower 8 lanes of Y:
//   P: lanes 0-7 of each row from X, lanes 8-15 from Y (row_shr:8)
//   Q: lanes 0-7 from X (row_shl:8), lanes 8-15 from Y
// after which lane l of P holds row l % 16, chunk 2 (l / 16) and lane l of Q the
// same row, chunk 2 (l / 16) + 1.  P and Q are complete 16x16x32 A operands
// over the even and odd 16-byte chunks of the step (values 64 s + 16 g + e and
// 64 s + 16 g + 8 + e for K-group g), so no MFMA lane is wasted.
//
// The residual enters as hi + lo bf16 pairs (as on the stream path).  Per step
// and 16-column N-tile there are four B fragments (P/Q x hi/lo), all four
// accumulating into the same 16x16 tile: logit = D after the K loop.
// The operand image [pass][step][nt][pq][hl][lane] x 16 bytes is built once per
// call by wide_prep_kernel; blocks stage it through LDS kWideCK steps at a time
// in two buffers, the next chunk's image being copied in while the current one is
// used, with one LDS-only barrier per chunk (table loads stay in flight across it).
// ---------------------------------------------------------------------------
static constexpr int kWideWaves = 8;
static constexpr int kWideMT = 4;                            // 16-row M-tiles per wave
static constexpr int kWideRows = kWideWaves * kWideMT * 16;  // table rows per block
static constexpr int kWideCK = 3;  // K steps per staged chunk = depth of the table-load ring
static constexpr int kWideMaxTiles = 4;                      // 16-column N-tiles: 64 residual rows

// Barrier that orders LDS accesses only: outstanding global loads are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Image slot i = ((((pass * steps_pad + s) * ntile + nt) * 2 + pq) * 2 + hl) * 64 + lane
// holds residual row 16 (ntile pass + nt) + lane % 16, values
// 64 s + 16 (lane / 16) + 8 pq + e (e = 0..7), as bf16 hi (hl = 0) or lo (hl = 1).
// Rows past the batch and values past hidden are zero.
// It also clears the per-row top-k lower bounds thr[B] (total >= B).
__global__ void __launch_bounds__(256) wide_prep_kernel(const float* __restrict__ R, int64_t B, int hidden,
                                                        int steps_pad, int ntile, int64_t total,
                                                        u32x4* __restrict__ img, uint64_t* __restrict__ thr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < B) thr[i] = 0;
  if (i >= total) return;
  const int lane = (int)(i & 63);
  const int f = (int)((i >> 6) & 3);
  int64_t q = i >> 8;
  const int nt = (int)(q % ntile);
  q /= ntile;
  const int s = (int)(q % steps_pad);
  const int64_t pass = q / steps_pad;
  const int64_t b = (pass * ntile + nt) * 16 + (lane & 15);
  const int c0 = 64 * s + 16 * (lane >> 4) + 8 * (f >> 1);
  const bool lo = (f & 1) != 0;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int c = c0 + e;
    const float x = (b < B && c < hidden) ? R[b * hidden + c] : 0.0f;
    const uint32_t hi = bf16_rne(x);
    v[e] = lo ? bf16_rne(x - __uint_as_float(hi << 16)) : hi;  // x - hi is exact in f32
  }
  img[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

// One pass (blockIdx.y) over the table for 16 NTILE residual rows.
//  table      bf16 [V][hidden], row_bytes = 2 hidden, a multiple of 16
//  img        operand image (wide_prep_kernel), steps_pad K steps per pass
//  steps_pad  ceil(hidden / 64) rounded up to kWideCK
// Rows past V are read from row V - 1 and never ranked; 16-byte chunks past the
// row end are read from the row's last 16 bytes and meet zero image values.
template <int NTILE>
__global__ void __launch_bounds__(64 * kWideWaves) wide_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, const u32x4* __restrict__ img, int64_t B,
    int steps_pad, int k, uint64_t* __restrict__ cand, uint64_t* __restrict__ thr) {
  constexpr int STEP_U4 = NTILE * 4 * 64;  // image slots per K step
  constexpr int CHUNK_U4 = kWideCK * STEP_U4;
  constexpr int NTHR = 64 * kWideWaves;
  constexpr int NPER = (STEP_U4 + NTHR - 1) / NTHR;
  constexpr int NC = NTILE * 16;
  constexpr int LS = NC + 1;  // logit row stride in LDS (odd: conflict-free column reads)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4* sbuf = (u32x4*)smem;  // two chunk buffers
  float* slog = (float*)smem;  // after the K loop: [kWideRows][LS]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kWideRows;
  const u32x4* pimg = img + (size_t)blockIdx.y * steps_pad * STEP_U4;
  const uint8_t* tbase = table + (uint64_t)row0 * (uint64_t)row_bytes;
  const int r8 = lane & 7, ck = lane >> 3;
  const uint32_t last_off = (uint32_t)(row_bytes - 16);

  // byte offsets of this lane's X and Y rows from the block's first row (32-bit:
  // the planner bounds kWideRows * row_bytes)
  uint32_t xoff[kWideMT], yoff[kWideMT];
#pragma unroll
  for (int mt = 0; mt < kWideMT; mt++) {
    const int64_t rx = min(row0 + wv * (kWideMT * 16) + 16 * mt + r8, V - 1) - row0;
    const int64_t ry = min(row0 + wv * (kWideMT * 16) + 16 * mt + 8 + r8, V - 1) - row0;
    xoff[mt] = (uint32_t)(rx * row_bytes);
    yoff[mt] = (uint32_t)(ry * row_bytes);
  }
  // offset of this lane's 16-byte chunk of K step s within a row
  auto koff = [&](int s) { return min(128u * (uint32_t)s + 16u * (uint32_t)ck, last_off); };

  f32x4 acc[kWideMT][NTILE];
#pragma unroll
  for (int mt = 0; mt < kWideMT; mt++)
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // first chunk of the image: loads issued before the table loads, so the LDS
  // writes below do not wait for those
  constexpr int NPRE = (CHUNK_U4 + NTHR - 1) / NTHR;
  u32x4 pre[NPRE];
#pragma unroll
  for (int q = 0; q < NPRE; q++) pre[q] = pimg[min(tid + q * NTHR, CHUNK_U4 - 1)];

  // ring of table loads: the j-th step of a chunk lives in slot j and is loaded
  // kWideCK - 1 steps ahead of its use
  u32x4 ax[kWideCK][kWideMT], ay[kWideCK][kWideMT];
#pragma unroll
  for (int r = 0; r < kWideCK - 1; r++) {
    const uint32_t ko = koff(r);
#pragma unroll
    for (int mt = 0; mt < kWideMT; mt++) {
      ax[r][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (xoff[mt] + ko)));
      ay[r][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (yoff[mt] + ko)));
    }
  }
#pragma unroll
  for (int q = 0; q < NPRE; q++) sbuf[min(tid + q * NTHR, CHUNK_U4 - 1)] = pre[q];
  lds_barrier();

  const int nchunks = steps_pad / kWideCK;
  for (int c = 0; c < nchunks; c++) {
    const u32x4* cur = sbuf + (c & 1) * CHUNK_U4;
    u32x4* nxt = sbuf + ((c + 1) & 1) * CHUNK_U4;
    // the next chunk; past the last one these are spare loads of the last chunk
    // (never used)
    const int pn = min(c + 1, nchunks - 1);
    const int pc = c;
#pragma unroll
    for (int j = 0; j < kWideCK; j++) {
      const int cb = j, nb = (j + kWideCK - 1) % kWideCK;
      // image piece j of the next chunk
      u32x4 st[NPER];
      const u32x4* ps = pimg + ((size_t)pn * kWideCK + j) * STEP_U4;
#pragma unroll
      for (int q = 0; q < NPER; q++) st[q] = ps[min(tid + q * NTHR, STEP_U4 - 1)];
      // table loads of the step kWideCK - 1 ahead: the last step of this chunk for
      // j = 0, else step j - 1 of the next chunk (clamped to the row end)
      const uint32_t ko = koff(j == 0 ? pc * kWideCK + kWideCK - 1 : pn * kWideCK + j - 1);
#pragma unroll
      for (int mt = 0; mt < kWideMT; mt++) {
        ax[nb][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (xoff[mt] + ko)));
        ay[nb][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (yoff[mt] + ko)));
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 P[kWideMT], Q[kWideMT];
#pragma unroll
      for (int mt = 0; mt < kWideMT; mt++) {
        const u32x4 x = ax[cb][mt], y = ay[cb][mt];
        u32x4 p, qv;
#pragma unroll
        for (int d = 0; d < 4; d++) {
          p[d] = __builtin_amdgcn_update_dpp(x[d], y[d], 0x118, 0xf, 0xc, false);   // row_shr:8 into lanes 8-15
          qv[d] = __builtin_amdgcn_update_dpp(y[d], x[d], 0x108, 0xf, 0x3, false);  // row_shl:8 into lanes 0-7
        }
        P[mt] = __builtin_bit_cast(bf16x8, p);
        Q[mt] = __builtin_bit_cast(bf16x8, qv);
      }
      const u32x4* bl = cur + j * STEP_U4 + lane;
      // fragment f = 2 pq + hl of N-tile nt; consecutive MFMAs go to different
      // accumulators
#pragma unroll
      for (int nt = 0; nt < NTILE; nt++) {
#pragma unroll
        for (int f = 0; f < 4; f++) {
          const bf16x8 bop = __builtin_bit_cast(bf16x8, bl[(4 * nt + f) * 64]);
#pragma unroll
          for (int mt = 0; mt < kWideMT; mt++)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f < 2 ? P[mt] : Q[mt], bop, acc[mt][nt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < NPER; q++) nxt[j * STEP_U4 + min(tid + q * NTHR, STEP_U4 - 1)] = st[q];
    }
    lds_barrier();
  }

  // Per residual row b: the block's k best keys, largest first, then empty (0)
  // slots.  thr[b] is a running lower bound on the k-th best key of row b over
  // the whole table (the largest k-th best any block has found so far), so
  // entries whose order value is below its order value cannot be among the final
  // k and are skipped.  Whatever value a block reads, every key of the final
  // top k is still emitted, so the merged result does not depend on timing.
  // Only the order value (the upper 32 bits) of each bound is used; the bounds
  // of this wave's rows are loaded together, before the logits pass through LDS.
  constexpr int PER_LANE = kWideRows / 64;
  constexpr int MAXC = (NC + kWideWaves - 1) / kWideWaves;
  const int64_t bcol0 = (int64_t)blockIdx.y * NC + wv;
  uint32_t tords[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; i++)
    tords[i] = __hip_atomic_load((const uint32_t*)(thr + min(bcol0 + i * kWideWaves, B - 1)) + 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);

  // logits of the block's rows through LDS (the image buffers are free now)
#pragma unroll
  for (int mt = 0; mt < kWideMT; mt++)
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rl = wv * (kWideMT * 16) + 16 * mt + 4 * (lane >> 4) + i;
        slog[rl * LS + 16 * nt + (lane & 15)] = acc[mt][nt][i];
      }
  lds_barrier();

  // into scalars before any store, so that no later wait covers the stores
#pragma unroll
  for (int i = 0; i < MAXC; i++) tords[i] = __builtin_amdgcn_readfirstlane(tords[i]);

  // The wave's columns are selected together, round by round, so that their
  // reduction chains interleave.  v[i][q]: order value (score_ord, > 0 for any
  // score) of row lane + 64 q for column i if it passes the bound, else 0.
  // Round t takes, per column, the largest order value left and the smallest row
  // holding it, and removes that entry; a column whose largest value is 0 has no
  // entries left.  The rounds stop after k or when no column has entries left.
  uint32_t v[MAXC][PER_LANE];
  bool live[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; i++) {
    const int col = min(wv + i * kWideWaves, NC - 1);
    live[i] = wv + i * kWideWaves < NC && bcol0 + i * kWideWaves < B;
#pragma unroll
    for (int q = 0; q < PER_LANE; q++) {
      const int rl = lane + 64 * q;
      const uint32_t o = score_ord(slog[rl * LS + col]);
      v[i][q] = (row0 + rl < V && live[i] && o >= tords[i]) ? o : 0u;
    }
  }
  int rnd[MAXC];  // keys emitted per column
  uint64_t key[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; i++) rnd[i] = 0, key[i] = 0;
  for (int t = 0; t < k; t++) {
    uint32_t M[MAXC], Rw[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
      uint32_t lm = v[i][0];
#pragma unroll
      for (int q = 1; q < PER_LANE; q++) lm = max(lm, v[i][q]);
      M[i] = lm;
    }
    wave_minmax_u32_multi<true>(M);
    bool any = false;
#pragma unroll
    for (int i = 0; i < MAXC; i++) any |= M[i] != 0u;
    if (!any) break;
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
      uint32_t rq = 0xffffffffu;
#pragma unroll
      for (int q = PER_LANE - 1; q >= 0; q--) rq = v[i][q] == M[i] ? (uint32_t)(lane + 64 * q) : rq;
      Rw[i] = rq;
    }
    wave_minmax_u32_multi<false>(Rw);
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
      const bool hit = M[i] != 0u;
#pragma unroll
      for (int q = 0; q < PER_LANE; q++) v[i][q] = (hit && lane + 64 * q == (int)Rw[i]) ? 0u : v[i][q];
      key[i] = hit ? ((uint64_t)M[i] << 32) | (uint64_t)(~(uint32_t)(row0 + Rw[i])) : key[i];
      rnd[i] += hit ? 1 : 0;
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < MAXC; i++)
        if (M[i] != 0u) cand[((bcol0 + i * kWideWaves) * gridDim.x + blockIdx.x) * (int64_t)k + t] = key[i];
    }
  }
#pragma unroll
  for (int i = 0; i < MAXC; i++) {
    if (!live[i]) break;
    uint64_t* out = cand + ((bcol0 + i * kWideWaves) * gridDim.x + blockIdx.x) * (int64_t)k;
    for (int t = rnd[i] + lane; t < k; t += 64) out[t] = 0;
    if (rnd[i] == k && lane == 0)
      atomicMax((unsigned long long*)(thr + bcol0 + i * kWideWaves), (unsigned long long)key[i]);
  }
}

// ---------------------------------------------------------------------------
// GEMM path: bf16 tables, larger batches.
//
// C[v][j] = sum_i E[v][i] * Rs[j][i] with Rs the residual rows as hi and lo bf16
// rows, so logit[v][b] = C[v][hi(b)] + C[v][lo(b)].  A workgroup (4 waves, 2 x 2)
// owns a tile of TN split columns (TN / 2 residual rows) and walks a range of
// 256-row vocabulary tiles; per tile it runs the K loop in stages of TK values
// through double-buffered LDS and v_mfma_f32_32x32x16_bf16.  Wave (mw, nw)
// computes rows [128 mw, +128) x split columns [TN/2 nw, +TN/2) as 4 x NT
// 32x32 tiles: N-tiles [0, NT/2) hold hi rows and [NT/2, NT) the matching lo
// rows, so the hi + lo sum is a register add.
//
// An LDS row holds the TK values of one table or residual row (2 TK bytes, P =
// TK / 8 pieces of 16 bytes); piece p of row r is stored at p ^ ((r / W) % P),
// W = 128 / TK rows per 256-byte bank window.  That keeps the stage stores and
// the MFMA fragment reads (one piece of 16 consecutive rows per 16 lanes) free
// of bank conflicts.
//
// Top-k: every (wave, residual row) keeps a min-heap of k keys in LDS, owned by
// one lane.  After a vocabulary tile the logits pass through LDS and each lane
// offers its row's logits to its heap; only those that beat the root (rare
// after the first tiles) are inserted.  At the end the heaps are written out,
// unordered, as candidates: [batch][vocab range][MW row slices][k].
//
// Workgroup ids are mapped so the column tiles of one vocabulary range sit on
// the same XCD (ids go round-robin over the 8 XCDs): a table tile is fetched
// from HBM once and served to the other column tiles from that XCD's L2.
// ---------------------------------------------------------------------------
static constexpr int kGemmTM = 256;  // vocabulary rows per tile
static constexpr int kXcds = 8;
static constexpr int kGemmWideMW = 2;    // 4 waves: 128-row wave tiles

template <int TK>
__device__ __forceinline__ int gemm_swz(int r, int piece) {
  constexpr int P = TK / 8, W = 128 / TK;
  return r * (2 * TK) + 16 * (piece ^ ((r / W) % P));
}

// fp32 residual [B][hidden] -> split bf16 rows [nct][TN][kpad].  Row j of tile ct
// belongs to wave nw = j / (TN/2), N-tile t = (j % (TN/2)) / 32; it is the hi
// (t < NT/2) or lo part of residual row ct TN/2 + nw TN/4 + (t % (NT/2)) 32 + j % 32.
template <int TN>
__global__ void __launch_bounds__(256) gemm_prep_kernel(const float* __restrict__ R, int64_t B, int hidden, int kpad,
                                                        int64_t nrows, u32x4* __restrict__ Rs) {
  constexpr int NT = TN / 64;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int kc = kpad / 8;
  if (t >= nrows * kc) return;
  const int64_t row = t / kc;
  const int c0 = (int)(t % kc) * 8;
  const int64_t ct = row / TN;
  const int j = (int)(row % TN);
  const int nw = j / (TN / 2), tt = (j % (TN / 2)) / 32;
  const int part = tt >= NT / 2;
  const int64_t b = ct * (TN / 2) + nw * (TN / 4) + (tt % (NT / 2)) * 32 + j % 32;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int c = c0 + e;
    const float x = (b < B && c < hidden) ? R[b * hidden + c] : 0.0f;
    const uint32_t hi = bf16_rne(x);
    v[e] = part == 1 ? bf16_rne(x - __uint_as_float(hi << 16)) : hi;
  }
  Rs[t] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Min-heap of k keys in LDS (root = smallest kept key = admission threshold).
// Replacing the root and sifting down costs at most log2(k) levels.
__device__ __forceinline__ void heap_replace_root(uint64_t* h, int k, uint64_t key) {
  int i = 0;
  while (true) {
    int c = 2 * i + 1;
    if (c >= k) break;
    uint64_t cv = h[c];
    if (c + 1 < k) {
      const uint64_t c2 = h[c + 1];
      if (c2 < cv) {
        cv = c2;
        c = c + 1;
      }
    }
    if (cv >= key) break;
    h[i] = cv;
    i = c;
  }
  h[i] = key;
}

template <int TN, int TK, int MW>
struct GemmCfg {
  static constexpr int NWAVES = 2 * MW;                     // MW along the vocabulary, 2 along the columns
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int WROWS = kGemmTM / MW;                // vocabulary rows per wave
  static constexpr int MT = WROWS / 32;                     // 32-row M-tiles per wave
  static constexpr int NT = TN / 64;                        // 32-column N-tiles per wave
  static constexpr int KS = TK / 16;                        // MFMA K sub-steps per stage
  static constexpr int P = TK / 8;                          // 16-byte pieces per LDS row
  static constexpr int RPT = THREADS / P;                   // rows one pass of the block covers
  static constexpr int LA = kGemmTM / RPT;                  // table loads per thread per stage
  static constexpr int LB = TN / RPT;                       // residual loads per thread per stage
  static constexpr int STAGE = (kGemmTM + TN) * TK * 2;     // bytes
  static constexpr int COLS = TN / 4;                       // residual rows per wave
  static constexpr int EPI_ROWS = WROWS / 2;                // epilogue rows per pass
  static_assert(kGemmTM % RPT == 0 && TN % RPT == 0, "stage must split evenly over the block");
  static_assert(NWAVES * EPI_ROWS * 64 * 4 <= 2 * STAGE, "epilogue staging must fit the stage buffers");
};

template <int TN, int TK, int MW>
__global__ void __launch_bounds__(64 * 2 * MW) gemm_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden,
    const uint8_t* __restrict__ Rs, int kpad, int64_t B, int k, uint64_t* __restrict__ cand,
    int nct, int nvr, int tiles_per_range) {
  using C = GemmCfg<TN, TK, MW>;
  constexpr int NT = C::NT, MT = C::MT, KS = C::KS, P = C::P, RPT = C::RPT, LA = C::LA, LB = C::LB;
  constexpr int WROWS = C::WROWS, THREADS = C::THREADS, ER = C::EPI_ROWS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* stage_buf = smem;                                   // 2 x STAGE
  uint64_t* heaps = (uint64_t*)(smem + 2 * C::STAGE);                // [waves][COLS][k]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int mw = wv >> 1, nw = wv & 1;

  // XCD-aware placement: ids {x, x + 8, ...} run on XCD x.
  const int id = blockIdx.x;
  const int xcd = id % kXcds, local = id / kXcds;
  const int ct = local % nct;
  const int vr = xcd + kXcds * (local / nct);
  if (vr >= nvr) return;  // whole workgroup; no barrier has been reached

  for (int i = tid; i < C::NWAVES * C::COLS * k; i += THREADS) heaps[i] = 0;

  const int nstage = kpad / TK;
  const uint8_t* rs_tile = Rs + (size_t)ct * TN * kpad * 2;
  const int64_t last_off = row_bytes - 16;
  // loader mapping: chunk c = tid + THREADS j -> row c / P, piece c % P
  const int lrow = tid / P, lpiece = tid % P;

  for (int vt = 0; vt < tiles_per_range; vt++) {
    const int64_t v0 = ((int64_t)vr * tiles_per_range + vt) * kGemmTM;
    if (v0 >= V) break;
    const uint8_t* arow[LA];
#pragma unroll
    for (int j = 0; j < LA; j++) arow[j] = table + (uint64_t)min(v0 + lrow + RPT * j, V - 1) * (uint64_t)row_bytes;
    f32x16 acc[MT][NT];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
      for (int t = 0; t < NT; t++) acc[a][t] = f32x16{};

    // Two register stage buffers; stage s lives in buffer s % 2 from its load
    // until its store.  Step st computes stage st from LDS, stores stage st + 1
    // into the other LDS buffer and reuses that register buffer for the loads of
    // stage st + 3, which have two compute stages to arrive.  Loads and stores
    // are unconditional (stage indices past the end are clamped) so the wait
    // counts do not depend on the path taken.
    u32x4 pa0[LA], pb0[LB], pa1[LA], pb1[LB];
    auto load_stage = [&](int st, u32x4* pa, u32x4* pb) {
      const int64_t kb = (int64_t)min(st, nstage - 1) * (2 * TK) + 16 * lpiece;
      const int64_t koff = min(kb, last_off);
#pragma unroll
      for (int j = 0; j < LA; j++) pa[j] = *(const u32x4*)(arow[j] + koff);
#pragma unroll
      for (int j = 0; j < LB; j++) pb[j] = *(const u32x4*)(rs_tile + (size_t)(lrow + RPT * j) * kpad * 2 + kb);
    };
    auto store_stage = [&](int buf, const u32x4* pa, const u32x4* pb) {
      unsigned char* base = stage_buf + buf * C::STAGE;
#pragma unroll
      for (int j = 0; j < LA; j++) *(u32x4*)(base + gemm_swz<TK>(lrow + RPT * j, lpiece)) = pa[j];
#pragma unroll
      for (int j = 0; j < LB; j++)
        *(u32x4*)(base + kGemmTM * 2 * TK + gemm_swz<TK>(lrow + RPT * j, lpiece)) = pb[j];
    };
    // MFMA fragments for K sub-step ks are read while sub-step ks - 1 computes
    // (narrow tile; the wide tile reads them just before use)
    auto compute_stage = [&](int buf) {
      const unsigned char* A = stage_buf + buf * C::STAGE;
      const unsigned char* Bt = A + kGemmTM * 2 * TK;
      constexpr int FS = MT * NT > 8 ? 1 : 2;  // fragment sets (the largest wave tile has no registers for two)
      bf16x8 af[FS][MT], bfr[FS][NT];
      auto read = [&](int ks, int set) {
        const int piece = 2 * ks + (lane >> 5);
#pragma unroll
        for (int a = 0; a < MT; a++)
          af[set][a] =
              __builtin_bit_cast(bf16x8, *(const u32x4*)(A + gemm_swz<TK>(WROWS * mw + 32 * a + (lane & 31), piece)));
#pragma unroll
        for (int t = 0; t < NT; t++)
          bfr[set][t] = __builtin_bit_cast(
              bf16x8, *(const u32x4*)(Bt + gemm_swz<TK>((TN / 2) * nw + 32 * t + (lane & 31), piece)));
      };
      if (FS == 2) read(0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int cur = FS == 2 ? (ks & 1) : 0;
        if (FS == 1) read(ks, 0);
        else if (ks + 1 < KS) read(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int a = 0; a < MT; a++)
#pragma unroll
          for (int t = 0; t < NT; t++)
            acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][a], bfr[cur][t], acc[a][t], 0, 0, 0);
      }
    };
    auto step = [&](int st, u32x4* npa, u32x4* npb) {
      compute_stage(st & 1);
      store_stage((st + 1) & 1, npa, npb);
      load_stage(st + 3, npa, npb);
      __syncthreads();
    };

    load_stage(0, pa0, pb0);
    load_stage(1, pa1, pb1);
    __syncthreads();  // previous tile's readers of both buffers are done
    store_stage(0, pa0, pb0);
    load_stage(2, pa0, pb0);
    __syncthreads();
    int st = 0;
    for (; st + 1 < nstage; st += 2) {
      step(st, pa1, pb1);
      step(st + 1, pa0, pb0);
    }
    if (st < nstage) step(st, pa1, pb1);

    // Epilogue, in two passes of WROWS / 2 rows: the hi + lo sums go to this
    // wave's slice of the (now idle) stage buffers as [rows][64 columns]; then
    // lane c walks column c (residual row ct TN/2 + nw TN/4 + c) and offers each
    // logit that beats its heap root.  Row of register i of M-tile a:
    // WROWS mw + 32 a + 8 (i / 4) + 4 (lane / 32) + i % 4.
    float* tl = (float*)(stage_buf + (size_t)wv * ER * 64 * 4);
    const int64_t bcol = (int64_t)ct * (TN / 2) + nw * (TN / 4) + lane;
    const bool own = lane < C::COLS && bcol < B;
    uint64_t* heap = heaps + ((size_t)wv * C::COLS + (own ? lane : 0)) * k;
#pragma unroll
    for (int pass = 0; pass < 2; pass++) {
#pragma unroll
      for (int aa = 0; aa < MT / 2; aa++) {
        const int a = (MT / 2) * pass + aa;
#pragma unroll
        for (int t = 0; t < NT / 2; t++) {
          __builtin_amdgcn_sched_barrier(0);  // one 32 x 32 tile in flight at a time
#pragma unroll
          for (int i = 0; i < 16; i++)
            tl[(32 * aa + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)) * 64 + 32 * t + (lane & 31)] =
                acc[a][t][i] + acc[a][t + NT / 2][i];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (own) {
        uint64_t thr = heap[0];
        const int64_t r0 = v0 + WROWS * mw + ER * pass;
        for (int r = 0; r < ER; r++) {
          const int64_t row = r0 + r;
          const uint64_t key = row < V ? make_key(tl[r * 64 + lane], (uint32_t)row) : 0;
          if (key > thr) {
            heap_replace_root(heap, k, key);
            thr = heap[0];
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  __syncthreads();
  // heaps -> candidates [B][nvr][MW][k]
  {
    const int64_t b = (int64_t)ct * (TN / 2) + nw * (TN / 4) + lane;
    if (lane < C::COLS && b < B) {
      const uint64_t* heap = heaps + ((size_t)wv * C::COLS + lane) * k;
      uint64_t* out = cand + ((b * nvr + vr) * MW + mw) * (int64_t)k;
      for (int j = 0; j < k; j++) out[j] = heap[j];
    }
  }
}

// ---------------------------------------------------------------------------
// VALU path: any dtype.  Block = 4 waves over a contiguous slice of rows; a wave
// takes one row at a time, each lane accumulates RB residual rows over values
// lane, lane + 64, ... with f32 FMAs, then a butterfly sum per residual row.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float deq_value(const uint8_t* row, int c) {
  if constexpr (DT == DT_F32) {
    return ((const float*)row)[c];
  } else if constexpr (DT == DT_BF16) {
    return __uint_as_float((uint32_t)((const uint16_t*)row)[c] << 16);
  } else {
    const uint8_t* blk = row + 34 * (c >> 5);
    const float s = f16_bits_to_f32(*(const uint16_t*)blk);
    return (float)(int8_t)blk[2 + (c & 31)] * s;
  }
}

template <int DT, int RB>
__global__ void __launch_bounds__(256) valu_logits_kernel(const uint8_t* __restrict__ table, int64_t V,
                                                          int64_t row_bytes, int hidden,
                                                          const float* __restrict__ R, int64_t B, int k,
                                                          uint64_t* __restrict__ cand) {
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
    for (int c = lane; c < hidden; c += 64) {
      const float x = deq_value<DT>(row, c);
#pragma unroll
      for (int b = 0; b < RB; b++)
        if (b < nb) acc[b] = __builtin_fmaf(x, R[(b0 + b) * hidden + c], acc[b]);
    }
#pragma unroll
    for (int b = 0; b < RB; b++) {
      const float s = wave_sum(acc[b]);
      if (lane == 0) vlog[lr * RB + b] = s;
    }
  }
  __syncthreads();
  for (int b = wv; b < nb; b += 4) {
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

template <int KPT>
__global__ void __launch_bounds__(1024) topk_merge_kernel(const uint64_t* __restrict__ cand, int n, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ scores) {
  __shared__ uint64_t part[kMergeWaves * 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const uint64_t* c = cand + b * (int64_t)n;
  uint64_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; j++) {
    const int i = tid + j * kMergeThreads;
    key[j] = i < n ? c[i] : 0;
  }
  uint64_t prev = ~0ull;
  for (int t = 0; t < k; t++) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < KPT; j++) best = (key[j] < prev && key[j] > best) ? key[j] : best;
    best = wave_max_u64(best);
    if (lane == 0) part[wv * k + t] = best;
    prev = best;
  }
  __syncthreads();
  if (wv == 0) {
    // kMergeWaves * k <= 1024 keys: 16 per lane
    uint64_t key2[kMergeWaves];
#pragma unroll
    for (int j = 0; j < kMergeWaves; j++) {
      const int i = lane + 64 * j;
      key2[j] = i < kMergeWaves * k ? part[i] : 0;
    }
    prev = ~0ull;
    for (int t = 0; t < k; t++) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < kMergeWaves; j++) best = (key2[j] < prev && key2[j] > best) ? key2[j] : best;
      best = wave_max_u64(best);
      if (lane == 0) {
        ids[b * k + t] = (int32_t)(~(uint32_t)(best & 0xffffffffu));
        scores[b * k + t] = ord_score((uint32_t)(best >> 32));
      }
      prev = best;
    }
  }
}

// Same, for more keys than fit in registers: every round rescans global memory.
__global__ void __launch_bounds__(1024) topk_merge_wide_kernel(const uint64_t* __restrict__ cand, int n, int k,
                                                               int32_t* __restrict__ ids, float* __restrict__ scores) {
  __shared__ uint64_t red[2][kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
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
      ids[b * k + t] = (int32_t)(~(uint32_t)(m & 0xffffffffu));
      scores[b * k + t] = ord_score((uint32_t)(m >> 32));
    }
    prev = m;
  }
}

static hipError_t launch_merge(const uint64_t* cand, int64_t batch, int n, int k, int32_t* ids, float* scores,
                               hipStream_t stream) {
  const dim3 grid((unsigned)batch), block(kMergeThreads);
  const int kpt = (n + kMergeThreads - 1) / kMergeThreads;
#define ETG_MERGE_CASE(KV) \
  if (kpt <= KV) { hipLaunchKernelGGL((topk_merge_kernel<KV>), grid, block, 0, stream, cand, n, k, ids, scores); }
  ETG_MERGE_CASE(1)
  else ETG_MERGE_CASE(2) else ETG_MERGE_CASE(4) else ETG_MERGE_CASE(8) else ETG_MERGE_CASE(16)
  else ETG_MERGE_CASE(32) else hipLaunchKernelGGL(topk_merge_wide_kernel, grid, block, 0, stream, cand, n, k, ids,
                                                   scores);
#undef ETG_MERGE_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static hipError_t set_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return e;
}

static hipError_t record(hipEvent_t ev, hipStream_t stream) {
  return ev ? hipEventRecord(ev, stream) : hipSuccess;
}

template <int DT>
static hipError_t launch_valu(const TableDesc& t, const LogitsPlan& p, const float* R, uint64_t* cand,
                              hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid((unsigned)p.nblk, (unsigned)p.npass), block(256);
  hipError_t e = set_lds((const void*)valu_logits_kernel<DT, 1>, p.lds_bytes);
  if (e == hipSuccess) e = set_lds((const void*)valu_logits_kernel<DT, 2>, p.lds_bytes);
  if (e == hipSuccess) e = set_lds((const void*)valu_logits_kernel<DT, 4>, p.lds_bytes);
  if (e == hipSuccess) e = set_lds((const void*)valu_logits_kernel<DT, 8>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record(ev0, stream)) != hipSuccess) return e;
  switch (p.rb) {
#define ETG_VALU_CASE(RBV)                                                                          \
  case RBV:                                                                                         \
    hipLaunchKernelGGL((valu_logits_kernel<DT, RBV>), grid, block, p.lds_bytes, stream, t.rows, t.V, \
                       t.row_bytes, (int)t.hidden, R, p.batch, p.k, cand);                          \
    break;
    ETG_VALU_CASE(1)
    ETG_VALU_CASE(2)
    ETG_VALU_CASE(4)
    ETG_VALU_CASE(8)
#undef ETG_VALU_CASE
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record(ev1, stream);
}

template <int NIMG>
static hipError_t launch_stream(const TableDesc& t, const LogitsPlan& p, const float* R, uint64_t* cand,
                                hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_lds((const void*)stream_logits_kernel<NIMG>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((stream_logits_kernel<NIMG>), dim3((unsigned)p.nblk, (unsigned)p.npass),
                     dim3(64 * kStreamWaves), p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, R,
                     p.batch, p.steps, p.chunk, p.k, cand, p.ngroups, p.max_groups);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record(ev1, stream);
}

template <int NTILE>
static hipError_t launch_wide_nt(const TableDesc& t, const LogitsPlan& p, const u32x4* img, uint64_t* cand,
                                 uint64_t* thr, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_lds((const void*)wide_logits_kernel<NTILE>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((wide_logits_kernel<NTILE>), dim3((unsigned)p.nblk, (unsigned)p.npass), dim3(64 * kWideWaves),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, img, p.batch, p.steps, p.k, cand, thr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record(ev1, stream);
}

static hipError_t launch_wide(const TableDesc& t, const LogitsPlan& p, const float* R, uint8_t* img,
                              uint64_t* cand, uint64_t* thr, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t total = (int64_t)p.npass * p.steps * p.ntile * 256;  // >= 768 npass >= batch
  hipLaunchKernelGGL(wide_prep_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, R, p.batch,
                     (int)t.hidden, p.steps, p.ntile, total, (u32x4*)img, thr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.ntile) {
    case 1: return launch_wide_nt<1>(t, p, (const u32x4*)img, cand, thr, stream, ev0, ev1);
    case 2: return launch_wide_nt<2>(t, p, (const u32x4*)img, cand, thr, stream, ev0, ev1);
    case 3: return launch_wide_nt<3>(t, p, (const u32x4*)img, cand, thr, stream, ev0, ev1);
    case 4: return launch_wide_nt<4>(t, p, (const u32x4*)img, cand, thr, stream, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

template <int TN, int TK, int MW>
static hipError_t launch_gemm_cfg(const TableDesc& t, const LogitsPlan& p, const float* R, uint8_t* rs,
                                  uint64_t* cand, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t nrows = (int64_t)p.nct * TN;
  const int64_t nprep = nrows * (p.kpad / 8);
  hipLaunchKernelGGL((gemm_prep_kernel<TN>), dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, stream, R, p.batch,
                     (int)t.hidden, p.kpad, nrows, (u32x4*)rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = set_lds((const void*)gemm_logits_kernel<TN, TK, MW>, p.lds_bytes)) != hipSuccess) return e;
  if ((e = record(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_logits_kernel<TN, TK, MW>), dim3((unsigned)p.nblk), dim3(GemmCfg<TN, TK, MW>::THREADS),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, (const uint8_t*)rs, p.kpad, p.batch,
                     p.k, cand, p.nct, p.nvr, p.tiles_per_range);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record(ev1, stream);
}

static hipError_t launch_gemm(const TableDesc& t, const LogitsPlan& p, const float* R, uint8_t* rs, uint64_t* cand,
                              hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.tn == 256) return launch_gemm_cfg<256, 32, kGemmWideMW>(t, p, R, rs, cand, stream, ev0, ev1);
  if (p.gemm_mw == 4) return launch_gemm_cfg<128, 64, 4>(t, p, R, rs, cand, stream, ev0, ev1);
  return launch_gemm_cfg<128, 64, 2>(t, p, R, rs, cand, stream, ev0, ev1);
}

hipError_t launch_logits_topk(const TableDesc& t, const LogitsPlan& p, const float* R, int32_t* ids,
                              float* scores, void* ws, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  uint8_t* base = (uint8_t*)ws;
  uint64_t* cand = (uint64_t*)(base + p.cand_offset);
  hipError_t e;
  if (p.path == 2) {
    e = p.nimg == 1 ? launch_stream<1>(t, p, R, cand, stream, ev0, ev1)
                    : launch_stream<2>(t, p, R, cand, stream, ev0, ev1);
  } else if (p.path == 3) {
    e = launch_gemm(t, p, R, base + p.img_offset, cand, stream, ev0, ev1);
  } else if (p.path == 4) {
    e = launch_wide(t, p, R, base + p.img_offset, cand, (uint64_t*)(base + p.aux_offset), stream, ev0, ev1);
  } else {
    switch (t.dtype) {
      case DT_F32: e = launch_valu<DT_F32>(t, p, R, cand, stream, ev0, ev1); break;
      case DT_BF16: e = launch_valu<DT_BF16>(t, p, R, cand, stream, ev0, ev1); break;
      default: e = launch_valu<DT_Q8_0>(t, p, R, cand, stream, ev0, ev1); break;
    }
  }
  if (e != hipSuccess) return e;
  return launch_merge(cand, p.batch, p.ncand, p.k, ids, scores, stream);
}

// ---------------------------------------------------------------------------
// Planning (host only, no device calls).
// ---------------------------------------------------------------------------
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t plan_logits(const TableDesc& t, int64_t batch, int32_t k, int32_t path, LogitsPlan* p,
                    const char** why) {
  *p = LogitsPlan{};
  p->k = k;
  p->batch = batch;
  const int kTargetBlocks = 256;  // one block per MI355X compute unit
  // auto: bf16 tables stream for up to 64 residual rows (one table pass per 8
  // or per 64 rows), then switch to the tiled contraction
  if (path == 0) path = (t.dtype != DT_BF16) ? 1 : (batch <= 8 ? 2 : batch <= 64 ? 4 : 3);
  if ((path == 2 || path == 3 || path == 4) && t.dtype != DT_BF16) {
    *why = "the stream, gemm and wide paths need a bf16 table";
    return -5;
  }
  if (path != 1 && path != 2 && path != 3 && path != 4) {
    *why = "unknown path";
    return -5;
  }
  p->path = path;
  if (path == 2) {
    p->nimg = batch <= 4 ? 1 : 2;
    p->nbc = p->nimg == 1 ? 4 : 8;
    p->steps = (int32_t)cdiv(t.hidden, 64);
    p->ngroups = cdiv(t.V, 8);
    p->npass = (int32_t)cdiv(batch, p->nbc);
    // one block per CU, unless a wave would then own more than kStreamMaxPairs pairs
    const int64_t npairs_all = cdiv(p->ngroups, 2);
    p->nblk = (int32_t)std::max<int64_t>(cdiv(npairs_all, (int64_t)kStreamWaves * kStreamMaxPairs),
                                         std::min<int64_t>(kTargetBlocks, cdiv(npairs_all, kStreamWaves)));
    p->max_groups = (int32_t)(2 * cdiv(npairs_all, (int64_t)p->nblk * kStreamWaves));
    const size_t log_bytes = (size_t)kStreamWaves * p->max_groups * 8 * p->nbc * 4;
    const size_t img_room = kMaxLds - 1024 - log_bytes;
    const int64_t max_chunk = (int64_t)(img_room / ((size_t)p->nimg * 1024)) / kStreamUnroll * kStreamUnroll;
    // equal chunks (multiples of the unroll), as few as fit
    const int64_t nchunks = cdiv(p->steps, max_chunk);
    p->chunk = (int32_t)std::min<int64_t>(max_chunk, cdiv(cdiv(p->steps, nchunks), kStreamUnroll) * kStreamUnroll);
    p->lds_bytes = (size_t)p->chunk * p->nimg * 1024 + log_bytes;
    p->img_bytes = 0;
    p->ncand = p->nblk * k;
  } else if (path == 4) {
    // passes of at most 64 residual rows, split evenly into 16-row N-tiles
    if ((uint64_t)(kWideRows + 1) * (uint64_t)t.row_bytes >= (1ull << 32)) {
      *why = "rows too long for the wide path";
      return -5;
    }
    p->npass = (int32_t)cdiv(batch, kWideMaxTiles * 16);
    p->ntile = (int32_t)cdiv(cdiv(batch, p->npass), 16);
    p->steps = (int32_t)(cdiv(cdiv(t.hidden, 64), kWideCK) * kWideCK);
    p->nblk = (int32_t)cdiv(t.V, kWideRows);
    const size_t img_lds = (size_t)2 * kWideCK * p->ntile * 4 * 1024;
    const size_t log_lds = (size_t)kWideRows * (16 * p->ntile + 1) * 4;
    p->lds_bytes = std::max(img_lds, log_lds);
    p->img_bytes = (size_t)p->npass * p->steps * p->ntile * 4 * 1024;
    p->ncand = p->nblk * k;
  } else if (path == 3) {
    // Wide column tiles (128 residual rows) when the batch fills them; otherwise
    // 64-row tiles with 8 waves, or 4 waves when the per-wave heaps of a large k
    // would not fit beside the stage buffers.
    using Wide = GemmCfg<256, 32, kGemmWideMW>;
    using N8 = GemmCfg<128, 64, 4>;
    using N4 = GemmCfg<128, 64, 2>;
    auto lds_of = [&](size_t stage, int nwaves, int cols) { return 2 * stage + (size_t)nwaves * cols * k * 8; };
    int tk, nwaves, mw;
    size_t stage;
    if (batch > 64 && lds_of(Wide::STAGE, Wide::NWAVES, Wide::COLS) <= kMaxLds) {
      p->tn = 256, tk = 32, stage = Wide::STAGE, nwaves = Wide::NWAVES, mw = kGemmWideMW;
    } else if (lds_of(N8::STAGE, N8::NWAVES, N8::COLS) <= kMaxLds) {
      p->tn = 128, tk = 64, stage = N8::STAGE, nwaves = N8::NWAVES, mw = 4;
    } else {
      p->tn = 128, tk = 64, stage = N4::STAGE, nwaves = N4::NWAVES, mw = 2;
    }
    p->gemm_mw = mw;
    p->kpad = (int32_t)(cdiv(t.hidden, tk) * tk);
    p->nct = (int32_t)cdiv(batch, p->tn / 2);
    const int64_t vtiles = cdiv(t.V, kGemmTM);
    // about one workgroup per CU; vocabulary ranges in multiples of the XCD count
    int64_t nvr = std::max<int64_t>(1, kTargetBlocks / p->nct);
    nvr = std::min<int64_t>(nvr, vtiles);
    nvr = cdiv(nvr, kXcds) * kXcds;
    p->tiles_per_range = (int32_t)cdiv(vtiles, nvr);
    p->nvr = (int32_t)nvr;
    p->nblk = (int32_t)(p->nct * nvr);
    p->npass = 1;
    p->lds_bytes = 2 * stage + (size_t)nwaves * (p->tn / 4) * k * 8;
    if (p->lds_bytes > kMaxLds) {
      *why = "k too large for the gemm path's LDS heaps";
      return -5;
    }
    p->img_bytes = (size_t)p->nct * p->tn * p->kpad * 2;
    p->ncand = (int32_t)(nvr * mw * k);
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
  p->img_offset = 0;
  p->cand_offset = align_up(p->img_bytes, 256);
  p->cand_bytes = (size_t)batch * p->ncand * 8;
  p->aux_offset = align_up(p->cand_offset + p->cand_bytes, 256);
  p->aux_bytes = path == 4 ? (size_t)batch * 8 : 0;
  p->ws_bytes = align_up(p->aux_offset + p->aux_bytes, 256);
  return 0;
}

}  // namespace etg
