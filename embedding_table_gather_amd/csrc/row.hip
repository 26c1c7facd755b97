// Row path of the lm_head projection (one or two residual rows per table pass):
// ADR-0008 "POST /v1/logits", logits = residual @ lm_head.T over every vocabulary
// row, fused with a per-block top-k.  The decode step of the service (one
// residual) is the case it is for.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// ---------------------------------------------------------------------------
// A wave reads one table row at a time as 1 KiB contiguous loads (lane l takes
// the 16-byte chunk l of each KiB), a group of up to 6 KiB (4 KiB with two
// residual rows) of loads in flight while the previous group is summed, and the
// workgroup's 16 waves own consecutive runs of rows.  Measured on MI355X, this
// shape reads HBM faster (7.27 TB/s for pure loads) than 8 rows x 128 bytes per
// load (7.07 TB/s), the shape the MFMA stream path needs.
//
// Lane l's chunk i always holds values VPI (64 i + l) .. + VPI of every row.  The
// block stages the residual in LDS as [chunk][quarter-chunk h][lane][4 floats]
// (zero past hidden), so a lane reads its values with VPI / 4 16-byte reads that
// are consecutive across lanes (no bank conflicts).  The logit is the sum over
// chunks and values of value * residual with f32 FMAs in a fixed order (each
// product exact inside the FMA), then a butterfly sum over the wave:
// error <= (NI VPI + 6) 2^-24 sum |r e|.
// ---------------------------------------------------------------------------
static constexpr int kRowWaves = 16;
static constexpr int kRowMaxNI = 16;  // KiB per row: hidden <= 8192 (bf16 / f16), 4096 (f32)

template <int DT>
__device__ __forceinline__ void row_values(const u32x4& x, float (&v)[DT == DT_F32 ? 4 : 8]) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 4; e++) v[e] = __uint_as_float(x[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      if constexpr (DT == DT_BF16) {
        v[2 * e] = bf16_lo(x[e]);
        v[2 * e + 1] = bf16_hi(x[e]);
      } else {
        v[2 * e] = f16_bits_to_f32(x[e] & 0xffffu);
        v[2 * e + 1] = f16_bits_to_f32(x[e] >> 16);
      }
    }
  }
}

//  NI      KiB loads per row, ceil(row_bytes / 1024)
//  logits  nullable [B][V] raw logits
//  lse     nullable [B][gridDim.x] log-partition partials at lse_c = log2(e) / T
// Chunks past the row end are read from the row's last 16 bytes and meet zero
// residual values.
template <int DT, int NI, int RB>
__global__ void __launch_bounds__(64 * kRowWaves) row_logits_kernel(
    const uint8_t* __restrict__ table, int64_t V, int64_t row_bytes, int hidden, const void* __restrict__ R,
    int wire, int64_t B, int k, uint64_t* __restrict__ cand, float* __restrict__ logits, float2* __restrict__ lse,
    float lse_c) {
  constexpr int VPI = DT == DT_F32 ? 4 : 8;
  constexpr int H = VPI / 4;
  extern __shared__ __attribute__((aligned(16))) float rsm[];
  constexpr int RS = NI * H * 256;     // floats per staged residual row
  float* sres = rsm;                   // [RB][NI][H][64][4]
  float* rlog = rsm + RB * RS;         // [rows of this block][RB]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nblk = gridDim.x;
  const int64_t r_begin = (int64_t)blockIdx.x * V / nblk;
  const int nrows = (int)(((int64_t)blockIdx.x + 1) * V / nblk - r_begin);
  const int64_t b0 = (int64_t)blockIdx.y * RB;  // residual rows of this pass
  const int nbr = (int)min((int64_t)RB, B - b0);

  for (int s = threadIdx.x; s < RB * RS; s += blockDim.x) {
    const int rb = s / RS, s1 = s - rb * RS;
    const int q = s1 & 3, l = (s1 >> 2) & 63, h = (s1 >> 8) % H, i = (s1 >> 8) / H;
    const int c = VPI * (64 * i + l) + 4 * h + q;
    sres[s] = (c < hidden && rb < nbr) ? residual_value(R, wire, b0 + rb, hidden, c) : 0.f;
  }
  __syncthreads();
  const f32x4* rres = (const f32x4*)sres + lane;  // + rb RS / 4 + (i H + h) 64

  const uint32_t last = (uint32_t)(row_bytes - 16);
  const int w0 = (int)((int64_t)wv * nrows / kRowWaves), w1 = (int)((int64_t)(wv + 1) * nrows / kRowWaves);
  // A row is read in NG groups of GS <= GMAX loads; the next group's loads (of this row or
  // the next) are issued before the current group's arithmetic.  A padding slot
  // of the last group (GS NG > NI) repeats the row's last chunk and meets a zero
  // residual, so no load or FMA is predicated.
  constexpr int GMAX = RB == 1 ? 6 : 4;  // KiB per group (fewer with two residual rows: registers)
  constexpr int NG = (NI + GMAX - 1) / GMAX, GS = (NI + NG - 1) / NG;
  const int nunits = (w1 - w0) * NG;
  u32x4 nx[GS];
  auto issue = [&](int u) {
    const int rl = w0 + u / NG, g = u % NG;
    const uint8_t* rp = table + (uint64_t)(r_begin + rl) * (uint64_t)row_bytes;
#pragma unroll
    for (int j = 0; j < GS; j++) {
      const int i = min(g * GS + j, NI - 1);
      nx[j] = __builtin_nontemporal_load((const u32x4*)(rp + min(16u * (uint32_t)(64 * i + lane), last)));
    }
  };
  if (nunits > 0) issue(0);
  float acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; rb++) acc[rb] = 0.f;
  for (int u = 0; u < nunits; u++) {
    u32x4 x[GS];
#pragma unroll
    for (int j = 0; j < GS; j++) x[j] = nx[j];
    if (u + 1 < nunits) issue(u + 1);
    const int g = u % NG;
#pragma unroll
    for (int j = 0; j < GS; j++) {
      const int ir = g * GS + j, i = min(ir, NI - 1);
      float v[VPI];
      row_values<DT>(x[j], v);
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
#pragma unroll
        for (int h = 0; h < H; h++) {
          const f32x4 r4 = ir < NI ? rres[rb * (RS / 4) + (i * H + h) * 64] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; q++) acc[rb] = __builtin_fmaf(v[4 * h + q], r4[q], acc[rb]);
        }
    }
    if (g == NG - 1) {
#pragma unroll
      for (int rb = 0; rb < RB; rb++) {
        const float t = wave_sum(acc[rb]);
        if (lane == 0) rlog[(w0 + u / NG) * RB + rb] = t;
        acc[rb] = 0.f;
      }
    }
  }
  __syncthreads();

  // per residual row b of the pass: wave 2 b writes raw logits and the partial,
  // wave 2 b + 1 takes the block's k best
  for (int rb = wv >> 1; rb < nbr; rb += kRowWaves / 2) {
    const int64_t b = b0 + rb;
    if ((wv & 1) == 0) {
      if (logits != nullptr)
        for (int i = lane; i < nrows; i += 64) logits[b * V + r_begin + i] = rlog[i * RB + rb];
      if (lse != nullptr) {
        float m = -__builtin_inff();
        for (int i = lane; i < nrows; i += 64) m = fmaxf(m, rlog[i * RB + rb]);
        m = wave_max_f32(m);
        float s = 0.f;
        if (m > -__builtin_inff())
          for (int i = lane; i < nrows; i += 64) s += exp2f((rlog[i * RB + rb] - m) * lse_c);
        s = wave_sum(s);
        if (lane == 0) lse[b * nblk + blockIdx.x] = make_float2(m, s);
      }
    } else {
      uint64_t* out = cand + (b * nblk + blockIdx.x) * (int64_t)k;
      uint64_t prev = ~0ull;
      for (int t = 0; t < k; t++) {
        uint64_t best = 0;
        for (int i = lane; i < nrows; i += 64) {
          const uint64_t key = make_key(rlog[i * RB + rb], (uint32_t)(r_begin + i));
          if (key < prev && key > best) best = key;
        }
        best = wave_max_u64(best);
        if (lane == 0) out[t] = best;
        prev = best;
      }
    }
  }
}

template <int DT, int NI, int RB>
static hipError_t launch_row_cfg(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                 const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = set_dynamic_lds((const void*)row_logits_kernel<DT, NI, RB>, p.lds_bytes);
  if (e != hipSuccess) return e;
  if ((e = record_event(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((row_logits_kernel<DT, NI, RB>), dim3((unsigned)p.nblk, (unsigned)p.npass),
                     dim3(64 * kRowWaves), p.lds_bytes, stream, t.rows, t.V, t.row_bytes, (int)t.hidden, R,
                     (int)x.wire, p.batch, p.k, cand, x.logits, x.lse, x.lse_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev1, stream);
}

template <int DT, int RB>
static hipError_t launch_row_rb(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  switch (p.row_ni) {
#define ETG_ROW_CASE(N) \
  case N: return launch_row_cfg<DT, N, RB>(t, p, R, cand, x, stream, ev0, ev1);
    ETG_ROW_CASE(1) ETG_ROW_CASE(2) ETG_ROW_CASE(3) ETG_ROW_CASE(4) ETG_ROW_CASE(5) ETG_ROW_CASE(6)
    ETG_ROW_CASE(7) ETG_ROW_CASE(8) ETG_ROW_CASE(9) ETG_ROW_CASE(10) ETG_ROW_CASE(11) ETG_ROW_CASE(12)
    ETG_ROW_CASE(13) ETG_ROW_CASE(14) ETG_ROW_CASE(15) ETG_ROW_CASE(16)
#undef ETG_ROW_CASE
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
static hipError_t launch_row_dt(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                                const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  return p.rb == 2 ? launch_row_rb<DT, 2>(t, p, R, cand, x, stream, ev0, ev1)
                   : launch_row_rb<DT, 1>(t, p, R, cand, x, stream, ev0, ev1);
}

hipError_t launch_row(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand, const LogitsExtras& x,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  switch (t.dtype) {
    case DT_F32: return launch_row_dt<DT_F32>(t, p, R, cand, x, stream, ev0, ev1);
    case DT_BF16: return launch_row_dt<DT_BF16>(t, p, R, cand, x, stream, ev0, ev1);
    case DT_F16: return launch_row_dt<DT_F16>(t, p, R, cand, x, stream, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

int32_t plan_row(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why) {
  if (t.dtype != DT_F32 && t.dtype != DT_BF16 && t.dtype != DT_F16) {
    *why = "the row path needs an f32, bf16 or f16 table";
    return -5;
  }
  p->row_ni = (int32_t)cdiv(t.row_bytes, 1024);
  if (p->row_ni > kRowMaxNI) {
    *why = "rows too long for the row path (at most 16 KiB)";
    return -5;
  }
  p->rb = batch >= 2 ? 2 : 1;  // residual rows per table pass
  p->npass = (int32_t)cdiv(batch, p->rb);
  // one 16-wave workgroup per CU, at most 8192 rows each
  int64_t nblk = std::min<int64_t>(kTargetBlocks, std::max<int64_t>(1, cdiv(t.V, 64)));
  nblk = std::max<int64_t>(nblk, cdiv(t.V, 8192));
  p->nblk = (int32_t)nblk;
  p->rows_per_blk = cdiv(t.V, nblk);
  p->lds_bytes = ((size_t)p->rb * p->row_ni * 1024 / (t.dtype == DT_F32 ? 4 : 2) + p->rows_per_blk * p->rb) * 4;
  p->img_bytes = 0;
  p->ncand = p->nblk * k;
  return 0;
}

}  // namespace etg
