// Wide stream path of the tied lm_head projection (bf16 tables, up to 64 residual
// rows per table pass, 128 when ranking): ADR-0008 "POST /v1/logits", logits = residual @ lm_head.T
// over every vocabulary row, fused with a per-block top-k.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// Wide stream path: bf16 tables, batches beyond the stream path's 8 rows.
//
// Still one HBM pass over the table per pass of up to 64 residual rows (128 in
// ranking mode), with the table read straight into VGPRs; the residual operand
// comes from LDS.
// A block owns 512 table rows (8 waves x 4 M-tiles of 16 rows); past 8 N-tiles
// (ranking mode only), 256 (2 M-tiles per wave), since the accumulators of
// 4 M-tiles would fill a wave's registers.
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
// call by wide_prep_kernel; blocks stage it through LDS wide_ck steps at a time
// in two buffers, the next chunk's image being copied in while the current one is
// used, with one LDS-only barrier per chunk (table loads stay in flight across it).
// Past 4 N-tiles the accumulators leave room for a chunk (and table-load ring)
// of 2 steps only.
// ---------------------------------------------------------------------------
static constexpr int kWideWaves = 8;
// 16-row M-tiles per wave, and table rows per block
__host__ __device__ constexpr int wide_mt(int ntile) { return ntile > 8 ? 2 : 4; }
__host__ __device__ constexpr int wide_rows(int ntile) { return kWideWaves * wide_mt(ntile) * 16; }
static constexpr int kWideMaxTiles = 4;      // 16-column N-tiles per pass: 64 residual rows
static constexpr int kWideRankMaxTiles = 16;  // ranking mode: 256 residual rows
// K steps per staged chunk = depth of the table-load ring
__host__ __device__ constexpr int wide_ck(int ntile) { return ntile > 4 ? 2 : 3; }
// Ranking mode: keys kept per block and residual row.  The answer's k rows are
// spread over the blocks; a block holding more of the candidates than this is
// rescanned by the rescoring kernel.
static constexpr int kWideRankKeys = 4;
// Ranking mode: most candidate logits per block and residual row the fast
// selection keys (more, from ties, take the general selection).
static constexpr int kWideRankCap = 16;

// Barrier that orders LDS accesses only: outstanding global loads are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// s + the squares of 8 bf16 values (four v_dot2c_f32_bf16).
__device__ __forceinline__ float wide_sumsq(bf16x8 f, float s) {
  const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w[j]);
    s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
  }
  return s;
}

// Image slot i = ((((pass * steps_pad + s) * ntile + nt) * 2 + pq) * 2 + hl) * 64 + lane
// holds residual row 16 (ntile pass + nt) + lane % 16, values
// 64 s + 16 (lane / 16) + 8 pq + e (e = 0..7), as bf16 hi (hl = 0) or lo (hl = 1);
// in ranking mode (rank != 0) there is no hl level and every slot is hi.
// Rows past the batch and values past hidden are zero.
// It also clears the per-row top-k lower bounds thr[B] (total >= B; not in ranking mode).
__global__ void __launch_bounds__(256) wide_prep_kernel(const void* __restrict__ R, int wire, int64_t B, int hidden,
                                                        int steps_pad, int ntile, int64_t total,
                                                        u32x4* __restrict__ img, uint64_t* __restrict__ thr, int rank) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (!rank && i < B) thr[i] = 0;
  if (i >= total) return;
  const int lane = (int)(i & 63);
  const int nf = rank ? 2 : 4;
  const int f = rank ? 2 * (int)((i >> 6) & 1) : (int)((i >> 6) & 3);
  int64_t q = (i >> 6) / nf;
  const int nt = (int)(q % ntile);
  q /= ntile;
  const int s = (int)(q % steps_pad);
  const int64_t pass = q / steps_pad;
  const int64_t b = (pass * ntile + nt) * 16 + (lane & 15);
  const int c0 = 64 * s + 16 * (lane >> 4) + 8 * (f >> 1);
  const bool lo = (f & 1) != 0;
  float x[8];
  residual_values8(R, wire, B, b, hidden, c0, x);
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint32_t hi = bf16_rne(x[e]);
    v[e] = lo ? bf16_rne(x[e] - __uint_as_float(hi << 16)) : hi;  // x - hi is exact in f32
  }
  img[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
}

// One pass (blockIdx.y) over the table for 16 NTILE residual rows.
//  table      bf16 [V][hidden], row_bytes = 2 hidden, a multiple of 16
//  img        operand image (wide_prep_kernel), steps_pad K steps per pass
//  steps_pad  ceil(hidden / 64) rounded up to wide_ck(NTILE)
//  logits     nullable [B][V]: the block's raw logits
//  lse        nullable [B][gridDim.x]: log-partition partial of the block's rows
//             at lse_c = log2(e) / temperature
// Rows past V are read from row V - 1 and never ranked; 16-byte chunks past the
// row end are read from the row's last 16 bytes and meet zero image values.
//
// Ranking mode (RANK): the image holds bf16(residual) only (two fragments per
// N-tile), k is the number of keys kept per block and column (approximate logits,
// no running bound), and pass 0 writes the block's largest squared row norm to
// nrm2[block] (the rescoring kernel's certificate needs an upper bound on the
// table's row norms).
template <int NTILE, bool RANK>
__global__ void __launch_bounds__(64 * kWideWaves) wide_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, const u32x4* __restrict__ img, int64_t B,
    int steps_pad, int k, uint64_t* __restrict__ cand, uint64_t* __restrict__ thr, float* __restrict__ logits,
    float2* __restrict__ lse, float lse_c, float* __restrict__ nrm2) {
  static_assert(NTILE <= (RANK ? kWideRankMaxTiles : kWideMaxTiles), "N-tiles per pass");
  constexpr int CK = wide_ck(NTILE);
  constexpr int MT = wide_mt(NTILE);
  constexpr int ROWS = wide_rows(NTILE);
  constexpr int NF = RANK ? 2 : 4;          // image fragments per N-tile and step
  constexpr int STEP_U4 = NTILE * NF * 64;  // image slots per K step
  constexpr int CHUNK_U4 = CK * STEP_U4;
  constexpr int NTHR = 64 * kWideWaves;
  constexpr int NPER = (STEP_U4 + NTHR - 1) / NTHR;
  constexpr int NC = NTILE * 16;
  constexpr int LS = NC + 1;  // logit row stride in LDS (odd: conflict-free column reads)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4* sbuf = (u32x4*)smem;  // two chunk buffers
  float* slog = (float*)smem;  // after the K loop: [ROWS][LS]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS;
  const u32x4* pimg = img + (size_t)blockIdx.y * steps_pad * STEP_U4;
  const uint8_t* tbase = table + (uint64_t)row0 * (uint64_t)row_bytes;
  const int r8 = lane & 7, ck = lane >> 3;
  const uint32_t last_off = (uint32_t)(row_bytes - 16);

  // byte offsets of this lane's X and Y rows from the block's first row (32-bit:
  // the planner bounds ROWS * row_bytes)
  uint32_t xoff[MT], yoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const int64_t rx = min(row0 + wv * (MT * 16) + 16 * mt + r8, V - 1) - row0;
    const int64_t ry = min(row0 + wv * (MT * 16) + 16 * mt + 8 + r8, V - 1) - row0;
    xoff[mt] = (uint32_t)(rx * row_bytes);
    yoff[mt] = (uint32_t)(ry * row_bytes);
  }
  // offset of this lane's 16-byte chunk of K step s within a row
  auto koff = [&](int s) { return min(128u * (uint32_t)s + 16u * (uint32_t)ck, last_off); };

  f32x4 acc[MT][NTILE];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // ranking mode, pass 0: squares of this lane's table values per M-tile (lane l
  // holds row l % 16 of each M-tile, 16 of every 64 values)
  float nsq[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) nsq[mt] = 0.f;
  const bool do_nrm = RANK && blockIdx.y == 0;

  // first chunk of the image: loads issued before the table loads, so the LDS
  // writes below do not wait for those
  constexpr int NPRE = (CHUNK_U4 + NTHR - 1) / NTHR;
  u32x4 pre[NPRE];
#pragma unroll
  for (int q = 0; q < NPRE; q++) pre[q] = pimg[min(tid + q * NTHR, CHUNK_U4 - 1)];

  // ring of table loads: the j-th step of a chunk lives in slot j and is loaded
  // CK - 1 steps ahead of its use
  u32x4 ax[CK][MT], ay[CK][MT];
#pragma unroll
  for (int r = 0; r < CK - 1; r++) {
    const uint32_t ko = koff(r);
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      ax[r][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (xoff[mt] + ko)));
      ay[r][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (yoff[mt] + ko)));
    }
  }
#pragma unroll
  for (int q = 0; q < NPRE; q++) sbuf[min(tid + q * NTHR, CHUNK_U4 - 1)] = pre[q];
  lds_barrier();

  const int nchunks = steps_pad / CK;
  for (int c = 0; c < nchunks; c++) {
    const u32x4* cur = sbuf + (c & 1) * CHUNK_U4;
    u32x4* nxt = sbuf + ((c + 1) & 1) * CHUNK_U4;
    // the next chunk; past the last one these are spare loads of the last chunk
    // (never used)
    const int pn = min(c + 1, nchunks - 1);
    const int pc = c;
#pragma unroll
    for (int j = 0; j < CK; j++) {
      const int cb = j, nb = (j + CK - 1) % CK;
      // image piece j of the next chunk
      u32x4 st[NPER];
      const u32x4* ps = pimg + ((size_t)pn * CK + j) * STEP_U4;
#pragma unroll
      for (int q = 0; q < NPER; q++) st[q] = ps[min(tid + q * NTHR, STEP_U4 - 1)];
      // table loads of the step CK - 1 ahead: the last step of this chunk for
      // j = 0, else step j - 1 of the next chunk (clamped to the row end)
      const uint32_t ko = koff(j == 0 ? pc * CK + CK - 1 : pn * CK + j - 1);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        ax[nb][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (xoff[mt] + ko)));
        ay[nb][mt] = __builtin_nontemporal_load((const u32x4*)(tbase + (yoff[mt] + ko)));
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 P[MT], Q[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
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
      // fragment f = 2 pq + hl of N-tile nt (ranking mode: f = pq); consecutive
      // MFMAs go to different accumulators
#pragma unroll
      for (int nt = 0; nt < NTILE; nt++) {
#pragma unroll
        for (int f = 0; f < NF; f++) {
          const bf16x8 bop = __builtin_bit_cast(bf16x8, bl[(NF * nt + f) * 64]);
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f < NF / 2 ? P[mt] : Q[mt], bop, acc[mt][nt], 0,
                                                                   0, 0);
        }
      }
      if (do_nrm) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) nsq[mt] = wide_sumsq(P[mt], wide_sumsq(Q[mt], nsq[mt]));
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
  constexpr int PER_LANE = ROWS / 64;
  constexpr int MAXC = (NC + kWideWaves - 1) / kWideWaves;
  const int64_t bcol0 = (int64_t)blockIdx.y * NC + wv;
  uint32_t tords[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; i++)
    tords[i] = RANK ? 0u
                    : __hip_atomic_load((const uint32_t*)(thr + min(bcol0 + i * kWideWaves, B - 1)) + 1,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  if constexpr (RANK) {
    // pass 0: the block's largest squared row norm.  Lanes l, l ^ 16, l ^ 32 and
    // l ^ 48 hold the four quarters of row l % 16 of each M-tile; rows past V are
    // copies of row V - 1 and chunks past the row end copies of its last chunk, so
    // the maximum can only grow.
    __shared__ float nred[kWideWaves];
    float m = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      float x = nsq[mt] + __shfl_xor(nsq[mt], 16, 64);
      x += __shfl_xor(x, 32, 64);
      m = fmaxf(m, x);
    }
    m = wave_max_f32(m);
    if (lane == 0) nred[wv] = m;
    __syncthreads();
    if (do_nrm && tid == 0) {
      float mm = nred[0];
      for (int w = 1; w < kWideWaves; w++) mm = fmaxf(mm, nred[w]);
      nrm2[blockIdx.x] = mm;
    }
  }

  if constexpr (RANK) {
    // Ranking mode: the block's kb best keys per residual row, without passing the
    // logits through LDS.  Lane l holds 4 MT rows of column 16 nt + l % 16 in each
    // N-tile (rows 16 MT wv + 16 mt + 4 (l / 16) + i), one of the column's 32
    // groups of rows.  G = the kb-th largest group maximum bounds the column's kb-th
    // largest logit from below (kb groups reach G, each with a row of its own), so
    // only logits >= G are keyed, and the kb best keys of those are taken.  A
    // column with more than kWideRankCap of them (ties) sends the block to the
    // general selection below.
    // in the image buffers, free after the K loop (wide_rank_lds bytes)
    constexpr int GS = kWideWaves * 4 + 1;                  // group maxima stride (odd)
    uint64_t* gkey = (uint64_t*)smem;                        // [NC][kWideRankCap]
    float* gmx = (float*)(gkey + NC * kWideRankCap);         // [NC][GS] group maxima
    float* glim = gmx + NC * GS;                             // [NC]
    uint32_t* gcnt = (uint32_t*)(glim + NC);                 // [NC]
    __shared__ uint32_t govf;
    const bool tail = row0 + ROWS > V;  // the block has rows past the table
    const int rbase = wv * (MT * 16) + 4 * (lane >> 4);
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++) {
      float m = -__builtin_inff();
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
          m = (!tail || row0 + rbase + 16 * mt + i < V) ? fmaxf(m, acc[mt][nt][i]) : m;
      gmx[(16 * nt + (lane & 15)) * GS + wv * 4 + (lane >> 4)] = m;
    }
    if (tid < NC) gcnt[tid] = 0;
    if (tid == 0) govf = 0;
    lds_barrier();
    if (tid < NC) {
      float t[kWideRankKeys];  // the largest group maxima, descending
#pragma unroll
      for (int j = 0; j < kWideRankKeys; j++) t[j] = -__builtin_inff();
      for (int g = 0; g < kWideWaves * 4; g++) {
        float x = gmx[tid * GS + g];
#pragma unroll
        for (int j = 0; j < kWideRankKeys; j++) {
          const float hi = fmaxf(t[j], x);
          x = fminf(t[j], x);
          t[j] = hi;
        }
      }
      float lim = t[0];
#pragma unroll
      for (int j = 1; j < kWideRankKeys; j++) lim = j == k - 1 ? t[j] : lim;
      glim[tid] = lim;
    }
    lds_barrier();
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++) {
      const int col = 16 * nt + (lane & 15);
      const float lim = glim[col];
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int rl = rbase + 16 * mt + i;
          const float x = acc[mt][nt][i];
          if (x >= lim && (!tail || row0 + rl < V)) {
            const uint32_t slot = atomicAdd(&gcnt[col], 1u);
            if (slot < (uint32_t)kWideRankCap) gkey[col * kWideRankCap + slot] = make_key(x, (uint32_t)(row0 + rl));
          }
        }
    }
    lds_barrier();
    if (tid < NC && gcnt[tid] > (uint32_t)kWideRankCap) atomicOr(&govf, 1u);
    lds_barrier();
    if (govf == 0u) {
      const int64_t b = (int64_t)blockIdx.y * NC + tid;
      if (tid < NC && b < B) {
        const int c = (int)gcnt[tid];
        uint64_t* out = cand + (b * gridDim.x + blockIdx.x) * (int64_t)k;
        uint64_t prev = ~0ull;
        for (int t = 0; t < k; t++) {  // keys are unique (one per row)
          uint64_t best = 0;
          for (int j = 0; j < c; j++) {
            const uint64_t y = gkey[tid * kWideRankCap + j];
            best = (y < prev && y > best) ? y : best;
          }
          out[t] = best;  // 0: no key left
          prev = best;
        }
      }
      return;
    }
    // Ties: k rounds over the accumulators, each taking per column the largest
    // key below the previous round's (wave maxima through LDS, then the block's)
    uint64_t* wbest = (uint64_t*)smem;          // [kWideWaves][NC] (the image buffers are free)
    uint64_t* rsel = wbest + kWideWaves * NC;  // [NC] this round's key per column
    for (int t = 0; t < k; t++) {
#pragma unroll
      for (int nt = 0; nt < NTILE; nt++) {
        // the previous round's key of the column (read before this round's barrier)
        const uint64_t prev = t == 0 ? ~0ull : rsel[16 * nt + (lane & 15)];
        uint64_t best = 0;
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int rl = rbase + 16 * mt + i;
            const uint64_t key = (!tail || row0 + rl < V) ? make_key(acc[mt][nt][i], (uint32_t)(row0 + rl)) : 0ull;
            best = (key < prev && key > best) ? key : best;
          }
#pragma unroll
        for (int m = 16; m <= 32; m *= 2) {
          const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), m, 64) << 32) |
                             (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)best, m, 64);
          best = o > best ? o : best;
        }
        if (lane < 16) wbest[wv * NC + 16 * nt + lane] = best;
      }
      lds_barrier();
      if (tid < NC) {
        uint64_t m = 0;
#pragma unroll
        for (int w = 0; w < kWideWaves; w++) m = max(m, wbest[w * NC + tid]);
        rsel[tid] = m;
        const int64_t b = (int64_t)blockIdx.y * NC + tid;
        if (b < B) cand[(b * gridDim.x + blockIdx.x) * (int64_t)k + t] = m;  // 0: no key left
      }
      lds_barrier();
    }
    return;
  }

  // logits of the block's rows through LDS (the image buffers are free now)
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int nt = 0; nt < NTILE; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rl = wv * (MT * 16) + 16 * mt + 4 * (lane >> 4) + i;
        slog[rl * LS + 16 * nt + (lane & 15)] = acc[mt][nt][i];
      }
  lds_barrier();

  // into scalars before any store, so that no later wait covers the stores
#pragma unroll
  for (int i = 0; i < MAXC; i++) tords[i] = __builtin_amdgcn_readfirstlane(tords[i]);

  // raw logits and log-partition partials of the wave's columns
  if (!RANK && (logits != nullptr || lse != nullptr)) {
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
      const int col = wv + i * kWideWaves;
      const int64_t b = bcol0 + i * kWideWaves;
      if (col >= NC || b >= B) break;
      float x[PER_LANE];
      bool ok[PER_LANE];
#pragma unroll
      for (int q = 0; q < PER_LANE; q++) {
        const int rl = lane + 64 * q;
        ok[q] = row0 + rl < V;
        x[q] = slog[rl * LS + col];
        if (logits != nullptr && ok[q]) logits[b * V + row0 + rl] = x[q];
      }
      if (lse != nullptr) {
        const float2 part = wave_lse_part(x, ok, lse_c);
        if (lane == 0) lse[b * gridDim.x + blockIdx.x] = part;
      }
    }
  }

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
    if (!RANK && rnd[i] == k && lane == 0)
      atomicMax((unsigned long long*)(thr + bcol0 + i * kWideWaves), (unsigned long long)key[i]);
  }
}


template <int NTILE, bool RANK>
static hipError_t launch_wide_nt(const TableDesc& t, const LogitsPlan& p, const u32x4* img, uint64_t* cand,
                                 uint64_t* thr, const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0,
                                 hipEvent_t ev1) {
  hipError_t e = set_dynamic_lds((const void*)wide_logits_kernel<NTILE, RANK>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((wide_logits_kernel<NTILE, RANK>), dim3((unsigned)p.nblk, (unsigned)p.npass),
                     dim3(64 * kWideWaves), p.lds_bytes, stream, t.rows, t.V, t.row_bytes, img, p.batch, p.steps,
                     RANK ? p.kb : p.k, cand, thr, x.logits, x.lse, x.lse_scale, (float*)x.aux);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

template <bool RANK>
static hipError_t launch_wide_mode(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* img,
                                   uint64_t* cand, uint64_t* thr, const LogitsExtras& x, hipStream_t stream,
                                   hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t total = (int64_t)p.npass * p.steps * p.ntile * (RANK ? 128 : 256);  // >= 768 npass >= batch
  hipLaunchKernelGGL(wide_prep_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, R, (int)x.wire,
                     p.batch, (int)t.hidden, p.steps, p.ntile, total, (u32x4*)img, thr, (int)RANK);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.ntile) {
    case 1: return launch_wide_nt<1, RANK>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
    case 2: return launch_wide_nt<2, RANK>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
    case 3: return launch_wide_nt<3, RANK>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
    case 4: return launch_wide_nt<4, RANK>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
    default: break;
  }
  if constexpr (RANK) {
    switch (p.ntile) {
      case 5: return launch_wide_nt<5, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 6: return launch_wide_nt<6, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 7: return launch_wide_nt<7, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 8: return launch_wide_nt<8, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 9: return launch_wide_nt<9, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 10: return launch_wide_nt<10, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 11: return launch_wide_nt<11, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 12: return launch_wide_nt<12, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 13: return launch_wide_nt<13, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 14: return launch_wide_nt<14, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 15: return launch_wide_nt<15, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      case 16: return launch_wide_nt<16, true>(t, p, (const u32x4*)img, cand, thr, x, stream, ev0, ev1);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_wide(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* img, uint64_t* cand,
                       uint64_t* thr, const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  return launch_wide_mode<false>(t, p, R, img, cand, thr, x, stream, ev0, ev1);
}

// Ranking mode for batches of up to 128 rows a pass: the wide kernel ranks with bf16
// residual rows and keeps kb keys per 512-row block; the rescoring kernel
// certifies and completes the answer (aux holds the blocks' squared row norms).
hipError_t launch_wide_rank(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* img, uint64_t* cand,
                            const LogitsExtras& x, int32_t* ids, float* scores, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
  hipError_t e = launch_wide_mode<true>(t, p, R, img, cand, nullptr, x, stream, ev0, ev1);
  if (e != hipSuccess) return e;
  // the kernel emits each block's keys best first
  return launch_rescore(t, p, R, (int)x.wire, cand, p.nblk, wide_rows(p.ntile), (const float*)x.aux, p.nblk, p.steps * 64, ids,
                        scores, stream, 1);
}

int32_t plan_wide(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why, bool rank) {
    // passes of at most 64 residual rows (128 ranking), split evenly into 16-row
    // N-tiles
    if ((uint64_t)(wide_rows(1) + 1) * (uint64_t)t.row_bytes >= (1ull << 32)) {
      *why = "rows too long for the wide path";
      return -5;
    }
    const int nf = rank ? 2 : 4;  // image fragments per N-tile and step
    p->npass = (int32_t)cdiv(batch, (rank ? kWideRankMaxTiles : kWideMaxTiles) * 16);
    p->ntile = (int32_t)cdiv(cdiv(batch, p->npass), 16);
    const int ck = wide_ck(p->ntile);
    p->steps = (int32_t)(cdiv(cdiv(t.hidden, 64), ck) * ck);
    const int rows = wide_rows(p->ntile);
    p->nblk = (int32_t)cdiv(t.V, rows);
    const size_t img_lds = (size_t)2 * ck * p->ntile * nf * 1024;
    // after the K loop, in the same buffer: the logits (exact mode); ranking mode:
    // the candidate lists, group maxima, bounds and counts per column, or the
    // selection rounds' [waves + 1][columns] keys
    const size_t nc = (size_t)16 * p->ntile;
    const size_t log_lds = rank ? std::max(nc * (kWideRankCap * 8 + (kWideWaves * 4 + 1) * 4 + 8),
                                           (size_t)(kWideWaves + 1) * nc * 8)
                                : (size_t)rows * (nc + 1) * 4;
    p->lds_bytes = std::max(img_lds, log_lds);
    p->img_bytes = (size_t)p->npass * p->steps * p->ntile * nf * 1024;
    if (!rank) {
      p->ncand = p->nblk * k;
      p->aux_bytes = (size_t)batch * 8;  // running top-k bound per residual row
      return 0;
    }
    p->kb = std::min<int32_t>(k, kWideRankKeys);
    p->ncand = p->nblk * p->kb;
    p->aux_bytes = (size_t)p->nblk * 4;  // largest squared row norm per block
    p->rescore_lds = rescore_lds(t.hidden, p->ncand, p->nblk, k, batch);
    if (p->rescore_lds > kMaxLds - 4096) {
      *why = "too many vocabulary blocks for the rank path's rescoring";
      return -5;
    }
    return 0;
}

}  // namespace etg
