// Device-side helpers shared by the gfx950 kernels of libetg.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace etg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_Q8_0 = 2 };

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Butterfly sum: every lane ends with the same (bitwise) value because each
// pairwise add is commutative.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

}  // namespace etg
