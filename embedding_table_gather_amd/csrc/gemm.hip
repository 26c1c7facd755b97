// GEMM path of the tied lm_head projection (bf16 tables, large batches):
// ADR-0008 "POST /v1/logits", logits = residual @ lm_head.T over every vocabulary
// row, as a tiled bf16 MFMA contraction with the top-k fused into the epilogue.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// GEMM path.
//
// C[v][j] = sum_i E[v][i] * Rs[j][i] with Rs the residual rows as hi and lo bf16
// rows, so logit[v][b] = C[v][hi(b)] + C[v][lo(b)].  A workgroup owns one
// column tile of 256 split columns (128 residual rows) and walks a range of
// 256-row vocabulary tiles.  Per tile the K loop runs in stages of 32 values:
// the table and residual slices of a stage (256 rows x 64 bytes each) are
// copied HBM/L2 -> LDS by global_load_lds_dwordx4 (no staging registers), the
// table slices into a ring of NA buffers and the residual slices into a ring of
// NB buffers, NA - 1 and NB - 1 stages ahead of the MFMAs
// (v_mfma_f32_32x32x16_bf16); half of the waves issue each kind.  One barrier
// per stage, preceded by an explicit wait for the stage that is due next
// (vmcnt counts loads in issue order, so later stages stay in flight) and for
// this wave's LDS reads.  Fragment reads are software-pipelined: each group of
// six reads (one 16-value sub-step) overlaps the 8 MFMAs of the previous group,
// across the barrier too.
//
// Waves form a WM x WN grid; wave (mw, nw) computes rows [WR mw, +WR) x split
// columns [WC nw, +WC) as MT x NT 32x32 tiles.  N-tiles [0, NT/2) hold hi rows
// and [NT/2, NT) the lo rows of the same residual rows, so hi + lo is a register
// add in the epilogue.
//
// LDS rows are 64 bytes (32 bf16 values, 4 pieces of 16 bytes); piece p of row
// r is stored at p ^ ((r / 4) % 4).  One DMA instruction writes 1 KiB in lane
// order (16 rows), so lane l fetches row l / 4, piece (l % 4) ^ (l / 16) of its
// 16-row group; the MFMA fragment reads (16 consecutive rows of one piece per
// 16 lanes) are then free of bank conflicts.
//
// Top-k: one descending list of k keys per residual row of the column tile, in
// LDS.  After a vocabulary tile each lane offers its logits (hi + lo, in
// registers) that reach its row's k-th key (on the first tile, a lower bound
// from group maxima) to an append buffer, and one thread per row inserts them
// (few after the first tiles).  At the end the lists are written out, best
// first, as candidates [batch][vocabulary range][k].
//
// Workgroup ids are mapped so the column tiles of one vocabulary range sit on
// the same XCD (ids go round-robin over the 8 XCDs): a table stage is fetched
// from HBM once and served to the other column tiles from that XCD's L2.
// ---------------------------------------------------------------------------
static constexpr int kGemmBM = 256;                                   // vocabulary rows per tile
static constexpr int kGemmBN = 256;                                   // split columns per tile
static constexpr int kGemmBK = 32;                                    // K values per stage
static constexpr int kGemmStage = (kGemmBM + kGemmBN) * kGemmBK * 2;  // bytes per stage
static constexpr int kGemmCols = kGemmBN / 2;                         // residual rows per column tile
static constexpr int kXcds = 8;
// List length merged in registers (the ranking contraction's usual heap size).
static constexpr int kGemmRegList = 16;

template <int WM, int WN>
struct GemmCfg {
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WR = kGemmBM / WM;  // vocabulary rows per wave
  static constexpr int WC = kGemmBN / WN;  // split columns per wave
  static constexpr int MT = WR / 32;
  static constexpr int NT = WC / 32;
  static constexpr int DPW = kGemmStage / 1024 / NW;  // DMA instructions per wave per stage
  static_assert(NT % 2 == 0 && DPW * NW * 1024 == kGemmStage, "tile split");
};

__device__ __forceinline__ int gemm_swz(int r, int piece) { return r * 64 + 16 * (piece ^ ((r >> 2) & 3)); }

// vmcnt(n) lgkmcnt(0), then a workgroup barrier that no memory access crosses.
template <int N>
__device__ __forceinline__ void gemm_stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);  // expcnt(7) lgkmcnt(0) vmcnt(N)
  asm volatile("s_barrier" ::: "memory");
}

// gemm_stage_barrier<groups * G> for a run-time number of outstanding load groups.
template <int G>
__device__ __forceinline__ void gemm_stage_barrier_groups(int groups) {
  switch (groups) {
    case 0: gemm_stage_barrier<0>(); break;
    case 1: gemm_stage_barrier<G>(); break;
    case 2: gemm_stage_barrier<2 * G>(); break;
    default: gemm_stage_barrier<3 * G>(); break;
  }
}

// residual [B][hidden] (f32, or decoded from its wire format) -> split bf16 rows [nct][256][kpad].  Row j of column
// tile ct belongs to wave column nw = j / WC, N-tile t = (j % WC) / 32; it is the
// hi (t < NT/2) or lo part of residual row 128 ct + nw WC/2 + (t % (NT/2)) 32 + j % 32.
// Rows past the batch and values past hidden are zero.
__global__ void __launch_bounds__(256) gemm_prep_kernel(const void* __restrict__ R, int wire, int64_t B, int hidden,
                                                        int kpad,
                                                        int wc, int64_t nrows, u32x4* __restrict__ Rs) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int kc = kpad / 8;
  if (t >= nrows * kc) return;
  const int64_t row = t / kc;
  const int c0 = (int)(t % kc) * 8;
  const int64_t ct = row / kGemmBN;
  const int j = (int)(row % kGemmBN);
  const int nt = wc / 32;
  const int nw = j / wc, tt = (j % wc) / 32;
  const int part = tt >= nt / 2;
  const int64_t b = ct * kGemmCols + nw * (wc / 2) + (tt % (nt / 2)) * 32 + j % 32;
  float x[8];
  residual_values8(R, wire, B, b, hidden, c0, x);
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint32_t hi = bf16_rne(x[e]);
    v[e] = part == 1 ? bf16_rne(x[e] - __uint_as_float(hi << 16)) : hi;  // x - hi is exact in f32
  }
  Rs[t] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

// residual [B][hidden] -> bf16 rows [nct][256][kpad] for the ranking mode: image
// row j of column tile ct is bf16(residual row 256 ct + j) (round to nearest
// even); rows past the batch and values past hidden are zero.
__global__ void __launch_bounds__(256) gemm_prep_hi_kernel(const void* __restrict__ R, int wire, int64_t B,
                                                           int hidden, int kpad, int64_t nrows,
                                                           u32x4* __restrict__ Rs) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int kc = kpad / 8;
  if (t >= nrows * kc) return;
  const int64_t b = t / kc;
  const int c0 = (int)(t % kc) * 8;
  float x[8];
  residual_values8(R, wire, B, b, hidden, c0, x);
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) v[e] = bf16_rne(x[e]);
  Rs[t] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

typedef float f32x16 __attribute__((ext_vector_type(16)));


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// s + the squares of 8 bf16 values: four v_dot2c_f32_bf16 (two exact products
// and one f32 accumulation each), in element-pair order.
__device__ __forceinline__ float sumsq_bf16x8(bf16x8 f, float s) {
  const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w[j]);
    s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
  }
  return s;
}

//  table  bf16 [V][hidden], row_bytes = 2 hidden (a multiple of 16)
//  Rs     split residual rows [nct][256][kpad] (gemm_prep_kernel), kpad = hidden
//         rounded up to 32
//  logits  nullable [B][V]: raw logits
//  lse     nullable [B][nvr]: log-partition partial of each vocabulary range at
//          lse_c = log2(e) / temperature
//  lse_run [gridDim.x][64 WM WN]: each thread's running partial over the tiles
//          of its range (kept in memory, not in registers, across the K loops)
// Table rows past V are read from row V - 1 and never ranked; table bytes past
// the row end are read from the row's last 16 bytes and meet zero residual values.
template <int WM, int WN, int NA, int NB, bool SPLIT>
__global__ void __launch_bounds__(64 * WM * WN) gemm_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, const uint8_t* __restrict__ Rs, int kpad,
    int64_t B, int k, uint64_t* __restrict__ cand, int nct, int nvr, int tiles_per_range,
    float* __restrict__ logits, float2* __restrict__ lse, float lse_c, float2* __restrict__ lse_run,
    float* __restrict__ npart, int ngrp) {
  using C = GemmCfg<WM, WN>;
  constexpr int MT = C::MT, NT = C::NT, WR = C::WR, WC = C::WC, DPW = C::DPW;
  constexpr int COLS = SPLIT ? kGemmCols : kGemmBN;  // residual rows per column tile
  constexpr int WCR = SPLIT ? WC / 2 : WC;            // residual rows per wave column
  constexpr int NTR = SPLIT ? 1 : NT;                 // N-tiles holding distinct residual rows
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  static_assert(NA >= 2 && NB >= 2 && NA <= 5 && NB <= 5, "ring depths");
  static_assert(NT == 2 && MT == WN, "one hi and one lo N-tile (split) or two N-tiles; one M-tile per wave column");
  constexpr int SLICE = kGemmBM * 64;                     // one stage of 256 table or residual rows
  uint64_t* heaps = (uint64_t*)(smem + (NA + NB) * SLICE);  // [COLS][k] lists or heaps
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave choices scalar
  const int mw = wv / WN, nw = wv % WN;

  // XCD-aware placement: ids {x, x + 8, ...} run on XCD x.
  const int id = blockIdx.x;
  const int xcd = id % kXcds, local = id / kXcds;
  const int ct = local % nct;
  const int vr = xcd + kXcds * (local / nct);
  if (vr >= nvr) return;  // whole workgroup; no barrier has been reached

  for (int i = tid; i < COLS * k; i += C::THREADS) heaps[i] = 0;
  // ranking mode: partial squared norms of this wave's table rows (M-tile nw, one
  // K half per lane half) over the K stages s with s % ngrp == ct; column tiles
  // ct >= ngrp measure none
  float nsq = 0.f;
  bool nrm_on = false;

  const int nstage = kpad / kGemmBK;
  const uint8_t* rs_tile = Rs + (size_t)ct * kGemmBN * kpad * 2;
  // DMA: this wave's instructions q = wv DPW + j (j < DPW) cover 16-row groups,
  // q < 16 of the table slice and q >= 16 of the residual slice.  Lane l fetches
  // row l / 4 of the group, logical piece (l % 4) ^ (l / 16).
  const bool dma_a = wv * DPW < 16;
  const int lrow = lane >> 2, lpiece = (lane & 3) ^ (lane >> 4);
  const uint32_t lim = dma_a ? (uint32_t)(row_bytes - 16) : 0xffffffffu;
  const uint8_t* bsrc[DPW];
  if (!dma_a) {
#pragma unroll
    for (int j = 0; j < DPW; j++)
      bsrc[j] = rs_tile + (size_t)(16 * ((wv * DPW + j) % 16) + lrow) * kpad * 2;
  }

  for (int vt = 0; vt < tiles_per_range; vt++) {
    const int64_t v0 = ((int64_t)vr * tiles_per_range + vt) * kGemmBM;
    if (v0 >= V) break;
    const uint8_t* src[DPW];
#pragma unroll
    for (int j = 0; j < DPW; j++)
      src[j] = dma_a ? table + (uint64_t)min(v0 + 16 * ((wv * DPW + j) % 16) + lrow, V - 1) * (uint64_t)row_bytes
                     : bsrc[j];
    // Table slices go to a ring of NA buffers, residual slices to a ring of NB
    // buffers after it; a wave issues only one kind, depth - 1 stages ahead.
    const int depth = dma_a ? NA : NB;
    unsigned char* ring = smem + (dma_a ? 0 : NA * SLICE);
    auto issue = [&](int st, int slot) {
      const uint32_t off = min((uint32_t)st * 64u + 16u * (uint32_t)lpiece, lim);
      unsigned char* dst = ring + slot * SLICE;
#pragma unroll
      for (int j = 0; j < DPW; j++)
        __builtin_amdgcn_global_load_lds((const void*)(src[j] + off),
                                         (__attribute__((address_space(3))) void*)(dst + ((wv * DPW + j) % 16) * 1024),
                                         16, 0, 0);
    };
    f32x16 acc[MT][NT];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
      for (int t = 0; t < NT; t++) acc[a][t] = f32x16{};

    // Fragments of K sub-step ks (16 values) of the stage in ring slots (sa, sb).
    bf16x8 fa0[MT], fb0[NT], fa1[MT], fb1[NT];
    auto read = [&](int sa_, int sb_, int ks, bf16x8* fa, bf16x8* fb) {
      const unsigned char* A = smem + sa_ * SLICE;
      const unsigned char* Bt = smem + (NA + sb_) * SLICE;
      const int piece = 2 * ks + (lane >> 5);
#pragma unroll
      for (int a = 0; a < MT; a++)
        fa[a] = __builtin_bit_cast(bf16x8, *(const u32x4*)(A + gemm_swz(WR * mw + 32 * a + (lane & 31), piece)));
#pragma unroll
      for (int t = 0; t < NT; t++)
        fb[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Bt + gemm_swz(WC * nw + 32 * t + (lane & 31), piece)));
    };
    auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
      for (int a = 0; a < MT; a++)
#pragma unroll
        for (int t = 0; t < NT; t++)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[t], acc[a][t], 0, 0, 0);
      if constexpr (!SPLIT) {
#pragma unroll
        for (int a = 0; a < MT; a++)
          if (nrm_on && a == nw) nsq = sumsq_bf16x8(fa[a], nsq);
      }
    };

    const int pre = min(depth - 1, nstage);
    for (int st = 0; st < pre; st++) issue(st, st);
    gemm_stage_barrier_groups<DPW>(pre - 1);  // stage 0 has landed
    int sa = 0, sb = 0, sm = 0;  // ring slots of stage s (table, residual, this wave's ring)
    read(0, 0, 0, fa0, fb0);
    // Each group of fragment reads overlaps the 8 MFMAs of the previous group:
    // stage s sub-step 1 is read while sub-step 0 computes, and after the barrier
    // stage s + 1 sub-step 0 is read while stage s sub-step 1 computes.
    for (int s = 0; s < nstage; s++) {
      if constexpr (!SPLIT) nrm_on = s % ngrp == ct;
      // stage s + depth - 1 goes to the slot stage s - 1 has left
      if (s + depth - 1 < nstage) issue(s + depth - 1, sm == 0 ? depth - 1 : sm - 1);
      read(sa, sb, 1, fa1, fb1);
      mma(fa0, fb0);
      // stage s + 1 is due next; the stages this wave issued after it may stay in
      // flight.  The wait also covers this wave's reads of stage s, whose slot the
      // next iteration refills.
      gemm_stage_barrier_groups<DPW>(max(0, min(s + depth - 1, nstage - 1) - (s + 1)));
      sa = sa == NA - 1 ? 0 : sa + 1;
      sb = sb == NB - 1 ? 0 : sb + 1;
      sm = sm == depth - 1 ? 0 : sm + 1;
      if (s + 1 < nstage) read(sa, sb, 0, fa0, fb0);
      mma(fa1, fb1);
    }

    // Raw logits and the log-partition partial (register layout below; rows
    // as 32-bit offsets in the tile, stores at constant offsets from one base).
    if constexpr (!SPLIT) {
      // this column tile's part of the squared norm of row WR mw + 32 nw + lane % 32
      // (K values past hidden are copies of stored values: the sum can only grow)
      const float part = nsq + __shfl_xor(nsq, 32, 64);
      nsq = 0.f;
      const int64_t row = v0 + WR * mw + 32 * nw + (lane & 31);
      if (ct < ngrp && lane < 32 && row < V) npart[(int64_t)ct * V + row] = part;
    }
    if (SPLIT && (logits != nullptr || lse != nullptr)) {
      // an opaque copy of the thread index: the addresses below are recomputed
      // per tile instead of being hoisted out of the tile loop (no free registers
      // to keep them in across the K loop)
      int xt = tid;
      asm volatile("" : "+v"(xt));
      const int xl = xt & 63;
      const int64_t bx = (int64_t)ct * kGemmCols + nw * (WC / 2) + (xl & 31);
      const int rbase = WR * mw + 4 * (xl >> 5);
      const int vlim = (int)min((int64_t)kGemmBM, V - v0) - rbase;  // tile rows past rbase
      if (bx < B) {
        if (logits != nullptr) {
          float* lp = logits + bx * V + v0 + rbase;
#pragma unroll
          for (int a = 0; a < MT; a++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int r = 32 * a + 8 * (i >> 2) + (i & 3);
              if (r < vlim) lp[r] = acc[a][0][i] + acc[a][1][i];
            }
        }
        if (lse != nullptr) {
          float2* run_slot = lse_run + (size_t)id * C::THREADS + xt;
          float2 run = vt == 0 ? make_float2(-__builtin_inff(), 0.f) : *run_slot;
          float tm = -__builtin_inff();
#pragma unroll
          for (int a = 0; a < MT; a++)
#pragma unroll
            for (int i = 0; i < 16; i++)
              tm = 32 * a + 8 * (i >> 2) + (i & 3) < vlim ? fmaxf(tm, acc[a][0][i] + acc[a][1][i]) : tm;
          if (tm > -__builtin_inff()) {
            const float m = fmaxf(run.x, tm);
            float sum = run.y * exp2f((run.x - m) * lse_c);  // 0 while nothing was seen
#pragma unroll
            for (int a = 0; a < MT; a++)
#pragma unroll
              for (int i = 0; i < 16; i++)
                sum += 32 * a + 8 * (i >> 2) + (i & 3) < vlim ? exp2f((acc[a][0][i] + acc[a][1][i] - m) * lse_c) : 0.f;
            run = make_float2(m, sum);
          }
          *run_slot = run;
        }
      }
    }
    // Epilogue: every column (residual row) of the tile keeps its k best keys in
    // LDS (0 = empty slot): a descending list for k <= 16, else a min-heap.
    // Register i of tile (a, t) holds row WR mw + 32 a + 8 (i / 4) + 4 (lane / 32)
    // + i % 4 of operand column WC nw + 32 t + lane % 32 (split columns: N-tile 0
    // is hi and 1 is lo, so a lane sees 64 rows of one residual row; ranking
    // columns: each N-tile is its own residual row), so a column's 256 rows are
    // spread over 4 holders (two wave rows, two half-waves) of 64 values.
    //  * T = the list's k-th key (0 while not full); on the first tile and for
    //    k <= 64, at least the smallest over the 4 holders of each one's
    //    ceil(k / 4)-th largest maximum of its 16 groups of 4 rows: at least k
    //    groups, each with a row of its own, reach it, so it bounds the k-th best
    //    from below.
    //  * Each lane appends its keys at or above T to the column's append buffer (the
    //    stage rings are idle between tiles: no load is in flight after a tile's
    //    last stage and the next tile's first stages are issued after this).
    //  * One thread per column inserts the appended keys: into the list held in
    //    registers, or by replacing the heap root.
    //  * A buffer that overflowed sends the tile into another round, in which only
    //    the values not yet appended are offered against the raised T.
    // Rows past the table are never ranked.
    {
      // the smaller stage ring holds counters, the wave staging areas and the
      // append buffers
      constexpr int ACAP = (6 * SLICE - 4096 - 8 * 4096) / (COLS * 8);  // keys per column and round
      static_assert(ACAP >= 16 && C::THREADS == 512, "append buffers fit the smaller stage ring");
      uint32_t* acnt = (uint32_t*)smem;                   // [COLS] appended keys this round
      uint32_t* athr = acnt + COLS;                        // [COLS] first-tile order-value threshold
      uint32_t* aovf = athr + COLS;                        // [2] overflow flags, by round parity
      float* xs = (float*)(smem + 4096) + 1024 * wv;      // [8 waves][4][64 lanes][4] staging
      uint64_t* app = (uint64_t*)(smem + 4096 + 8 * 4096);  // [COLS][ACAP]
      // an opaque copy of the thread index keeps the per-lane rows and addresses
      // below inside the tile loop (no free registers to hold them across K)
      int xt = tid;
      asm volatile("" : "+v"(xt));
      const int xl = xt & 63;
      // The lane's rows grow with the register-order bit 16 a + i, so its rows
      // inside the table are a prefix of the bits: 16 per full M-tile, 4 per full
      // group of 8 rows, and up to 4 more.
      const int vl = max(0, (int)min((int64_t)kGemmBM, V - v0) - (WR * mw + 4 * (xl >> 5)));
      const int nvalid = vl >= 128 ? 64 : 16 * (vl >> 5) + 4 * ((vl & 31) >> 3) + min(vl & 7, 4);
      const uint64_t valid = nvalid >= 64 ? ~0ull : (1ull << nvalid) - 1;
      if constexpr (SPLIT) {
        // the column's logits, once (N-tile 1 is not read again this tile)
#pragma unroll
        for (int a = 0; a < MT; a++) acc[a][0] += acc[a][1];
      }
      constexpr int TT = SPLIT ? 1 : NT;  // accumulator N-tile of column tile t
      const bool regl = k <= kGemmRegList;  // sorted lists (else min-heaps, root = k-th key)
      uint64_t taken[NTR];
#pragma unroll
      for (int t = 0; t < NTR; t++) taken[t] = 0;
      // the first tile's bound holds for k up to the column's 64 groups
      const bool thr0 = vt == 0 && k <= 16 * MT;
      if (tid < COLS) athr[tid] = ~0u;
      if (tid < 2) aovf[tid] = 0;
      if (thr0) {
        gemm_stage_barrier<0>();
        // groups each holder vouches for (opaque: its compares below stay here
        // instead of holding scalar registers across the tile loop)
        int q = (k + 3) >> 2;
        asm volatile("" : "+s"(q));
#pragma unroll
        for (int t = 0; t < NTR; t++) {
          // the holder's 16 group maxima (groups of 4 rows: M-tile a, register
          // quad i / 4), sorted descending by insertion
          uint32_t srt[16];
#pragma unroll
          for (int g = 0; g < 16; g++) srt[g] = 0;
#pragma unroll
          for (int a = 0; a < MT; a++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
              uint32_t x = 0;
#pragma unroll
              for (int e = 0; e < 4; e++) {
                const int i = 4 * g4 + e;
                x = max(x, score_ord(acc[a][t % TT][i]) & (0u - (uint32_t)((valid >> (16 * a + i)) & 1)));
              }
#pragma unroll
              for (int g = 0; g < 16; g++) {
                const uint32_t hi = max(srt[g], x);
                x = min(srt[g], x);
                srt[g] = hi;
              }
            }
          uint32_t gq = srt[0];
#pragma unroll
          for (int g = 1; g < 16; g++) gq = g == q - 1 ? srt[g] : gq;
          atomicMin(&athr[nw * WCR + 32 * t + (xl & 31)], gq);
        }
      }
      for (int round = 0;; round++) {
        if (tid < COLS) acnt[tid] = 0;
        if (tid == 0) aovf[(round + 1) & 1] = 0;
        gemm_stage_barrier<0>();
#pragma unroll
        for (int t = 0; t < NTR; t++) {
          const int col = nw * WCR + 32 * t + (xl & 31);
          const uint64_t* list = heaps + (size_t)col * k;
          uint32_t T = (uint32_t)(list[regl ? k - 1 : 0] >> 32);
          if (thr0) T = max(T, athr[col]);
          // the values at or above T (as floats: ord_score inverts score_ord, with
          // -0 equal to +0) not offered yet, as a mask in register order
          const bool all = T == 0u;
          const float tf = ord_score(all ? 0x80000000u : T);
          uint64_t m = 0;
#pragma unroll
          for (int a = 0; a < MT; a++) {
            uint32_t ma = 0;
#pragma unroll
            for (int i = 0; i < 16; i++) ma |= (uint32_t)(acc[a][t % TT][i] >= tf) << i;
            m |= (uint64_t)ma << (16 * a);
          }
          m = (int64_t)ct * COLS + col < B ? (all ? ~0ull : m) & valid & ~taken[t] : 0ull;
          // one slot reservation per lane; the keys that fit go in register order
          const uint32_t nm = (uint32_t)__builtin_popcountll(m);
          const uint32_t base = nm != 0 ? atomicAdd(&acnt[col], nm) : 0u;
          uint64_t st = m;
          if (base + nm > (uint32_t)ACAP) {
            uint64_t rest = m;  // drop the lowest set bits that still fit
            for (uint32_t q = base; q < (uint32_t)ACAP; q++) rest &= rest - 1;
            st = m ^ rest;
          }
          taken[t] |= st;
          if (__ballot(st != 0) != 0) {
            uint64_t* dst = app + (size_t)col * ACAP + base;
            const uint32_t r0 = (uint32_t)(v0 + WR * mw + 4 * (xl >> 5));
#pragma unroll
            for (int a = 0; a < MT; a++) {
              uint32_t ma = (uint32_t)(st >> (16 * a)) & 0xffffu;
              if (__ballot(ma != 0) == 0) continue;
              // the lane's 16 values of M-tile a, read back by index (value i at
              // float 256 (i / 4) + 4 lane + i % 4 of the wave's area)
#pragma unroll
              for (int q = 0; q < 4; q++)
                *(f32x4*)(xs + 256 * q + 4 * xl) = f32x4{acc[a][t % TT][4 * q], acc[a][t % TT][4 * q + 1],
                                                         acc[a][t % TT][4 * q + 2], acc[a][t % TT][4 * q + 3]};
              while (ma != 0) {
                const int j = __builtin_ctz(ma);
                ma &= ma - 1;
                *dst++ = make_key(xs[256 * (j >> 2) + 4 * xl + (j & 3)], r0 + 32 * a + 8 * (j >> 2) + (j & 3));
              }
            }
          }
        }
        gemm_stage_barrier<0>();
        if (tid < COLS) {
          uint32_t n = acnt[tid];
          if (n > (uint32_t)ACAP) {
            aovf[round & 1] = 1;
            n = ACAP;
          }
          if (n != 0) {
            uint64_t* list = heaps + (size_t)tid * k;
            const uint64_t* ap = app + (size_t)tid * ACAP;
            if (regl) {
              // the list in registers, padded with empty keys; each key enters by a
              // branch-free insertion (position j takes max(L[j], min(L[j - 1], key)),
              // high j first)
              uint64_t L[kGemmRegList];
#pragma unroll
              for (int j = 0; j < kGemmRegList; j++) L[j] = j < k ? list[j] : 0ull;
              for (uint32_t q = 0; q < n; q++) {
                const uint64_t key = ap[q];
#pragma unroll
                for (int j = kGemmRegList - 1; j > 0; j--) {
                  const uint64_t lo = L[j - 1] < key ? L[j - 1] : key;
                  L[j] = L[j] > lo ? L[j] : lo;
                }
                L[0] = L[0] > key ? L[0] : key;
              }
#pragma unroll
              for (int j = 0; j < kGemmRegList; j++)
                if (j < k) list[j] = L[j];
            } else {
              for (uint32_t q = 0; q < n; q++) {
                const uint64_t key = ap[q];
                if (key > list[0]) heap_replace_root(list, k, key);  // keys are unique: offered once
              }
            }
          }
        }
        gemm_stage_barrier<0>();
        if (aovf[round & 1] == 0) {
          // every wave has read the flag before the next tile's copies refill the rings
          gemm_stage_barrier<0>();
          break;
        }
      }
    }
  }
  if (SPLIT && lse != nullptr) {
    // lanes l and l + 32 hold the same residual row, then the WM = 2 wave rows
    // (the stage ring is free after the last tile's barrier)
    static_assert(WM == 2, "two wave rows");
    // a thread's slot holds its partial once the range's first tile ran
    const bool mine = (int64_t)vr * tiles_per_range * kGemmBM < V &&
                      (int64_t)ct * kGemmCols + nw * (WC / 2) + (lane & 31) < B;
    float2 run = mine ? lse_run[(size_t)id * C::THREADS + tid] : make_float2(-__builtin_inff(), 0.f);
    run = lse_combine(run, make_float2(__shfl_xor(run.x, 32, 64), __shfl_xor(run.y, 32, 64)), lse_c);
    float2* xl = (float2*)smem;  // [WN][32]
    if (mw == 1 && lane < 32) xl[nw * 32 + lane] = run;
    gemm_stage_barrier<0>();
    const int64_t b = (int64_t)ct * kGemmCols + nw * (WC / 2) + lane;
    if (mw == 0 && lane < 32 && b < B) lse[b * nvr + vr] = lse_combine(run, xl[nw * 32 + lane], lse_c);
  }
  // heaps -> candidates [B][nvr][k]; the barrier orders the heap writes (also
  // the zeroing, for a range past the table that ran no tile) before the reads
  gemm_stage_barrier<0>();
  if (tid < COLS) {
    const int64_t b = (int64_t)ct * COLS + tid;
    if (b < B) {
      const uint64_t* heap = heaps + (size_t)tid * k;
      uint64_t* out = cand + (b * nvr + vr) * (int64_t)k;
      for (int j = 0; j < k; j++) out[j] = heap[j];
    }
  }
}

// Ranking contraction planning: heap keys per residual row over all ranges, and
// keys per range heap.  A range keeps its 16 best approximate keys; the answer's
// k rows are spread over the ranges, and a range holding more of the candidates
// than that is rescanned.  Small heaps leave LDS for the deeper residual ring and
// shorten the first tile's selection.
static constexpr int kRankMaxKeys = 4096;  // heap keys per residual row (nvr kb)
static constexpr int kRankHeapKeys = 16;

template <int WM, int WN, int NA, int NB, bool SPLIT>
static hipError_t launch_gemm_cfg(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* rs,
                                  uint64_t* cand, const LogitsExtras& x, int32_t* ids, float* scores,
                                  hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  using C = GemmCfg<WM, WN>;
  const int64_t nrows = (int64_t)p.nct * kGemmBN;
  const int64_t nprep = nrows * (p.kpad / 8);
  if constexpr (SPLIT) {
    hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, stream, R, (int)x.wire,
                       p.batch, (int)t.hidden, p.kpad, C::WC, nrows, (u32x4*)rs);
  } else {
    hipLaunchKernelGGL(gemm_prep_hi_kernel, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, stream, R,
                       (int)x.wire, p.batch, (int)t.hidden, p.kpad, nrows, (u32x4*)rs);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = set_dynamic_lds((const void*)gemm_logits_kernel<WM, WN, NA, NB, SPLIT>, p.lds_bytes)) != hipSuccess)
    return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_logits_kernel<WM, WN, NA, NB, SPLIT>), dim3((unsigned)p.nblk), dim3(C::THREADS),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (const uint8_t*)rs, p.kpad, p.batch,
                     SPLIT ? p.k : p.kb, cand, p.nct, p.nvr, p.tiles_per_range, x.logits, x.lse, x.lse_scale,
                     (float2*)x.aux, (float*)x.aux, p.ngrp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record_event(ev1, stream)) != hipSuccess) return e;
  if constexpr (!SPLIT) {
    // aux: npart [ngrp][V], then nrm2 [nnrm]
    const int nnrm = (int)cdiv(t.V, kRankNormRows);
    float* nrm2 = (float*)x.aux + align_up((size_t)p.ngrp * t.V, 64);
    if ((e = launch_rank_norm((const float*)x.aux, p.ngrp, t.V, nrm2, stream)) != hipSuccess) return e;
    if ((e = launch_rescore(t, p, R, (int)x.wire, cand, p.nvr, (int64_t)p.tiles_per_range * kGemmBM, nrm2, nnrm,
                            p.kpad, ids, scores, stream, 1)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* rs, uint64_t* cand,
                       const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  // one wave layout: 2 x 4 waves of 128 x 64 (2 x 2 waves of 128 x 128 would spill)
  if (p.gemm_ring == 34)
    return launch_gemm_cfg<2, 4, 3, 4, true>(t, p, R, rs, cand, x, nullptr, nullptr, stream, ev0, ev1);
  return launch_gemm_cfg<2, 4, 3, 3, true>(t, p, R, rs, cand, x, nullptr, nullptr, stream, ev0, ev1);
}

hipError_t launch_rank(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* rs, uint64_t* cand,
                       const LogitsExtras& x, int32_t* ids, float* scores, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1) {
  if (p.rank_wide) return launch_wide_rank(t, p, R, rs, cand, x, ids, scores, stream, ev0, ev1);
  if (p.gemm_ring == 34) return launch_gemm_cfg<2, 4, 3, 4, false>(t, p, R, rs, cand, x, ids, scores, stream, ev0, ev1);
  return launch_gemm_cfg<2, 4, 3, 3, false>(t, p, R, rs, cand, x, ids, scores, stream, ev0, ev1);
}

// Column tiles, vocabulary ranges and LDS rings shared by both modes.  Split
// mode: 128 residual rows per column tile and heaps of k keys (the exact k best);
// ranking mode: 256 rows and heaps of hk_max keys, fewer when there are many
// ranges (at most kRankMaxKeys per residual row).  *hk receives the heap size.
static int32_t plan_gemm_common(const TableDesc& t, int64_t batch, bool split, int hk_max, LogitsPlan* p,
                                int32_t* hk, const char** why) {
  const int cols = split ? kGemmCols : kGemmBN;
  p->gemm_wn = 4;
  p->tn = kGemmBN;
  p->kpad = (int32_t)(cdiv(t.hidden, kGemmBK) * kGemmBK);
  p->nct = (int32_t)cdiv(batch, cols);
  const int64_t vtiles = cdiv(t.V, kGemmBM);
  // about one workgroup per CU; vocabulary ranges in multiples of the XCD count
  int64_t nvr = std::max<int64_t>(1, kTargetBlocks / p->nct);
  nvr = std::min<int64_t>(nvr, vtiles);
  nvr = cdiv(nvr, kXcds) * kXcds;
  p->tiles_per_range = (int32_t)cdiv(vtiles, nvr);
  p->nvr = (int32_t)nvr;
  p->nblk = (int32_t)(p->nct * nvr);
  p->npass = 1;
  *hk = split ? hk_max : std::min<int32_t>(hk_max, std::max<int32_t>(1, kRankMaxKeys / (int32_t)nvr));
  // the residual ring one stage deeper when the heaps leave room
  const size_t heaps = (size_t)cols * *hk * 8;
  p->gemm_ring = 7 * (size_t)kGemmBM * 64 + heaps <= kMaxLds ? 34 : 33;
  p->lds_bytes = (p->gemm_ring == 34 ? 7 : 6) * (size_t)kGemmBM * 64 + heaps;
  if (p->lds_bytes > kMaxLds) {
    *why = "k too large for the gemm path's LDS heaps";
    return -5;
  }
  p->img_bytes = (size_t)p->nct * kGemmBN * p->kpad * 2;
  return 0;
}

int32_t plan_gemm(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  int32_t hk = 0;
  const int32_t st = plan_gemm_common(t, batch, true, k, p, &hk, why);
  if (st != 0) return st;
  p->ncand = (int32_t)(p->nvr * k);
  p->aux_bytes = (size_t)p->nblk * 64 * 8 * 8;  // running log-partition partial per thread
  return 0;
}

int32_t plan_rank(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  if (t.hidden > kRankMaxHidden) {
    *why = "hidden too large for the rank path (the residual row is kept in LDS)";
    return -5;
  }
  if (batch <= kRankWideBatch) {  // the wide kernel in ranking mode
    p->rank_wide = 1;
    return plan_wide(t, batch, k, p, why, true);
  }
  int32_t hk = 0;
  const int32_t st = plan_gemm_common(t, batch, false, std::min<int32_t>(k, kRankHeapKeys), p, &hk, why);
  if (st != 0) return st;
  p->kb = hk;
  p->ncand = (int32_t)(p->nvr * hk);
  // row norms: up to 8 column tiles each measure a share of the K stages
  p->ngrp = (int32_t)std::min<int64_t>(p->nct, 8);
  p->aux_bytes = (align_up((size_t)p->ngrp * t.V, 64) + (size_t)cdiv(t.V, kRankNormRows)) * 4;
  p->rescore_lds = rescore_lds(t.hidden, p->ncand, p->nvr, k, batch);
  if (p->rescore_lds > kMaxLds - 4096) {  // static LDS besides
    *why = "the rank path's rescoring does not fit in LDS";
    return -5;
  }
  return 0;
}

}  // namespace etg
