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
  if (path == 0) path = (t.dtype != DT_BF16) ? 1 : (batch <= 8 ? 2 : 3);
  if ((path == 2 || path == 3) && t.dtype != DT_BF16) {
    *why = "the stream and gemm paths need a bf16 table";
    return -5;
  }
  if (path != 1 && path != 2 && path != 3) {
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
  p->ws_bytes = align_up(p->cand_offset + p->cand_bytes, 256);
  return 0;
}

}  // namespace etg
