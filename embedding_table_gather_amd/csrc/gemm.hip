// GEMM path of the tied lm_head projection (bf16 tables, large batches):
// ADR-0008 "POST /v1/logits", logits = residual @ lm_head.T over every vocabulary
// row, as a tiled bf16 MFMA contraction with the top-k fused into the epilogue.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

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


template <int TN, int TK, int MW>
static hipError_t launch_gemm_cfg(const TableDesc& t, const LogitsPlan& p, const float* R, uint8_t* rs,
                                  uint64_t* cand, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t nrows = (int64_t)p.nct * TN;
  const int64_t nprep = nrows * (p.kpad / 8);
  hipLaunchKernelGGL((gemm_prep_kernel<TN>), dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, stream, R, p.batch,
                     (int)t.hidden, p.kpad, nrows, (u32x4*)rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = set_dynamic_lds((const void*)gemm_logits_kernel<TN, TK, MW>, p.lds_bytes)) != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_logits_kernel<TN, TK, MW>), dim3((unsigned)p.nblk), dim3(GemmCfg<TN, TK, MW>::THREADS),
                     p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, (const uint8_t*)rs, p.kpad, p.batch,
                     p.k, cand, p.nct, p.nvr, p.tiles_per_range);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

hipError_t launch_gemm(const TableDesc& t, const LogitsPlan& p, const float* R, uint8_t* rs, uint64_t* cand,
                              hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.tn == 256) return launch_gemm_cfg<256, 32, kGemmWideMW>(t, p, R, rs, cand, stream, ev0, ev1);
  if (p.gemm_mw == 4) return launch_gemm_cfg<128, 64, 4>(t, p, R, rs, cand, stream, ev0, ev1);
  return launch_gemm_cfg<128, 64, 2>(t, p, R, rs, cand, stream, ev0, ev1);
}

int32_t plan_gemm(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
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
  return 0;
}

}  // namespace etg
