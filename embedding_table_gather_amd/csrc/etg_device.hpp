// Device-side helpers shared by the gfx950 kernels of libetg.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace etg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_Q8_0 = 2, DT_F16 = 3 };

// ---------------------------------------------------------------------------
// Top-k ordering key.  A larger key is a better candidate: higher logit first,
// and among equal logits the smaller id.  -0.0 is mapped to +0.0 first so the
// two zeros tie (and fall back to the id) instead of ranking -0 below +0.
// key = ord(score) << 32 | ~id.  Key 0 is below every real candidate and marks
// an empty slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_ord(float s) {
  uint32_t u = __float_as_uint(s);
  if (s == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ord_score(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)score_ord(s) << 32) | (uint64_t)(~id);
}

// One DPP step of a 64-bit prefix max: lanes whose source lane is outside the
// row (or whose row is masked off) see 0, which is below every key.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROWMASK, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROWMASK, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Maximum over the wave, returned to every lane: shifts of 1, 2, 4 and 8 within
// each 16-lane row leave the row maximum in lane 15 of the row; row_bcast:15 and
// row_bcast:31 carry it across rows, so lane 63 holds the wave maximum.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_u64<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_u64<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_u64<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_u64<0x142, 0xa>(v);  // row_bcast:15
  v = dpp_max_u64<0x143, 0xc>(v);  // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// 32-bit maximum / minimum over the wave, returned to every lane (same DPP
// pattern as wave_max_u64; lanes outside the source row see the identity).
template <bool MAX>
__device__ __forceinline__ uint32_t dpp_minmax_u32(uint32_t v, uint32_t o) { return MAX ? max(v, o) : min(v, o); }

template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  constexpr uint32_t id = MAX ? 0u : 0xffffffffu;
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = dpp_minmax_u32<MAX>(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// wave_minmax_u32 on N independent values at once, stage by stage, so that each
// DPP move reads a register written N instructions earlier (no hazard stalls).
template <bool MAX, int N>
__device__ __forceinline__ void wave_minmax_u32_multi(uint32_t (&v)[N]) {
  constexpr uint32_t id = MAX ? 0u : 0xffffffffu;
#define ETG_DPP_STAGE(CTRL, RM)                                                                     \
  _Pragma("unroll") for (int i = 0; i < N; i++)                                                     \
      v[i] = dpp_minmax_u32<MAX>(v[i], __builtin_amdgcn_update_dpp(id, v[i], CTRL, RM, 0xf, false));
  ETG_DPP_STAGE(0x111, 0xf)
  ETG_DPP_STAGE(0x112, 0xf)
  ETG_DPP_STAGE(0x114, 0xf)
  ETG_DPP_STAGE(0x118, 0xf)
  ETG_DPP_STAGE(0x142, 0xa)
  ETG_DPP_STAGE(0x143, 0xc)
#undef ETG_DPP_STAGE
#pragma unroll
  for (int i = 0; i < N; i++) v[i] = __builtin_amdgcn_readlane(v[i], 63);
}

// One selection round over keys held by a wave (N per lane, 0 = empty): returns
// the largest key to every lane and removes it.  Keys are unique, so the round
// takes the largest order value (upper 32 bits) and, among keys holding it, the
// largest lower word (~id, so the smallest id); both are 32-bit DPP reductions.
template <int N>
__device__ __forceinline__ uint64_t wave_pop_max(uint64_t (&key)[N]) {
  uint32_t hi = 0;
#pragma unroll
  for (int j = 0; j < N; j++) hi = max(hi, (uint32_t)(key[j] >> 32));
  hi = wave_minmax_u32<true>(hi);
  uint32_t lo = 0;
#pragma unroll
  for (int j = 0; j < N; j++) lo = (uint32_t)(key[j] >> 32) == hi ? max(lo, (uint32_t)key[j]) : lo;
  lo = wave_minmax_u32<true>(lo);
  const uint64_t best = ((uint64_t)hi << 32) | lo;
#pragma unroll
  for (int j = 0; j < N; j++) key[j] = key[j] == best ? 0 : key[j];
  return best;
}

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

// Butterfly sum: every lane ends with the same (bitwise) value because each
// pairwise add is commutative.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Log-partition partials for probabilities at temperature T, c = log2(e) / T.
// A set of logits x is summarised as (m, s) = (max x, sum exp2((x - m) c)), so
// that ln sum exp(x / T) = (m c + log2 s) ln 2; the empty set is (-inf, 0).
// Every term is <= 1 and the largest is exactly 1, so s never overflows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 lse_combine(float2 a, float2 b, float c) {
  const float m = fmaxf(a.x, b.x);
  if (m == -__builtin_inff()) return a;  // both empty
  // an empty side contributes 0 * exp2(-inf) = 0
  return make_float2(m, a.y * exp2f((a.x - m) * c) + b.y * exp2f((b.x - m) * c));
}

// (m, s) over the wave of the values x[j] with ok[j], every lane getting the result.
template <int N>
__device__ __forceinline__ float2 wave_lse_part(const float (&x)[N], const bool (&ok)[N], float c) {
  float m = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < N; j++) m = ok[j] ? fmaxf(m, x[j]) : m;
  m = wave_max_f32(m);
  if (m == -__builtin_inff()) return make_float2(m, 0.f);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < N; j++) s += ok[j] ? exp2f((x[j] - m) * c) : 0.f;
  return make_float2(m, wave_sum(s));
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h16);
}

// f32 -> binary16 bits, round to nearest even, clamped to +-65504 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_f16_sat(float x) {
  return __builtin_bit_cast(unsigned short, (_Float16)fminf(fmaxf(x, -65504.f), 65504.f));
}

// Exact value c of a stored row (f32 copy, bf16 / f16 widening, Q8_0 int8 * scale).
template <int DT>
__device__ __forceinline__ float deq_value(const uint8_t* row, int c) {
  if constexpr (DT == DT_F32) {
    return ((const float*)row)[c];
  } else if constexpr (DT == DT_BF16) {
    return __uint_as_float((uint32_t)((const uint16_t*)row)[c] << 16);
  } else if constexpr (DT == DT_F16) {
    return f16_bits_to_f32(((const uint16_t*)row)[c]);
  } else {
    const uint8_t* blk = row + 34 * (c >> 5);
    const float s = f16_bits_to_f32(*(const uint16_t*)blk);
    return (float)(int8_t)blk[2 + (c & 31)] * s;
  }
}

// ---------------------------------------------------------------------------
// Residual wire formats (ADR-0009 "Wire Layout"), for rows of `hidden` values:
//   WIRE_F32  binary32 [B][hidden]
//   WIRE_F16  binary16 [B][hidden]
//   WIRE_I8   per row: [scale f32][zero point f32 (0)][int8 x hidden], value = q * scale
// ---------------------------------------------------------------------------
enum { WIRE_F32 = 0, WIRE_F16 = 1, WIRE_I8 = 2 };

__device__ __forceinline__ float residual_value(const void* R, int wire, int64_t b, int hidden, int c) {
  if (wire == WIRE_F32) return ((const float*)R)[b * hidden + c];
  if (wire == WIRE_F16) return f16_bits_to_f32(((const uint16_t*)R)[b * hidden + c]);
  const uint8_t* row = (const uint8_t*)R + b * (int64_t)(hidden + 8);
  return (float)(int8_t)row[8 + c] * *(const float*)row;
}

// Values c0 .. c0 + 7 of residual row b (0 past hidden or for b >= B).  f32 rows
// starting 16-byte aligned (R aligned, hidden a multiple of 4) with c0 a multiple
// of 4 and all eight inside the row are read as two 16-byte loads.
__device__ __forceinline__ void residual_values8(const void* R, int wire, int64_t B, int64_t b, int hidden, int c0,
                                                 float (&x)[8]) {
  if (b < B && wire == WIRE_F32 && ((uintptr_t)R & 15) == 0 && hidden % 4 == 0 && c0 % 4 == 0 && c0 + 8 <= hidden) {
    const f32x4* src = (const f32x4*)((const float*)R + b * hidden + c0);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int e = 0; e < 4; e++) x[e] = x0[e], x[4 + e] = x1[e];
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; e++) x[e] = (b < B && c0 + e < hidden) ? residual_value(R, wire, b, hidden, c0 + e) : 0.0f;
}

}  // namespace etg
