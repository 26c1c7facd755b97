// Token-id row gather with per-row dequant and an optional x sqrt(d) scale.
//
// ADR-0008 "POST /v1/embed" returns one f32 row of `hidden` values per token id,
// found by one pointer offset per id; a prefill of N ids is N independent
// lookups ("Open Questions" item 2).  Rows are addressed as row i at byte
// offset i * row_bytes (HELIX Columnar Embedding proposal, section 3).  The
// embeddinggemma.c port specification ("Forward graph") scales the gathered
// Q8_0 rows by sqrt(768).
//
// f16 rows are the embed slice's binary16 store, widened per lookup (ADR-0008
// "Vindex Slice: embed" and "Memory footprint").
//
// One wavefront per output row.  f32 / bf16 / f16 rows are read with 16-byte loads
// straight into registers; Q8_0 rows (34-byte blocks, so only 2-byte aligned in
// general) are staged through the wave's slice of LDS with aligned dword loads
// and then unpacked.  Q8_0 rows whose size is a multiple of 16 bytes take a
// kernel that stages them with 16-byte loads, two rows per wave.  Stores are
// 16-byte f32x4, contiguous across the wave.
//
// Bit-exactness: dequant is exact in f32 (copy; bf16 and f16 widening; int8 * f16 has at
// most 19 significant bits) and the scale is one f32 multiply, so there is one
// rounding at most.  FP contraction is off in this file.
#include <algorithm>

#include "etg_device.hpp"
#include "etg_internal.hpp"

#pragma clang fp contract(off)

namespace etg {

static constexpr int kGatherWaves = 4;
static constexpr int kGatherUnroll = 4;
// Q8_0 blocks staged per piece by the general gather (2,176 bytes + 4 per wave).
static constexpr int kGatherPieceBlocks = 64;
// Rows per launch: a launch covers at most 2^24 rows (2^30 work-items), longer
// gathers are split into several launches on the same stream.
static constexpr int64_t kGatherLaunchRows = (int64_t)1 << 24;

template <int DT, bool SCALE>
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ table, uint32_t V,
                                                     int hidden, int64_t row_bytes,
                                                     const int32_t* __restrict__ ids, int64_t n,
                                                     float scale, float* __restrict__ out,
                                                     int32_t* __restrict__ bad, int lds_words) {
  extern __shared__ uint32_t lds_words_buf[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kGatherWaves + wv;
  if (row >= n) return;  // whole wave; the kernel has no block-level barrier
  const uint32_t id = (uint32_t)ids[row];
  f32x4* o = (f32x4*)(out + row * (int64_t)hidden);
  const int n4 = hidden >> 2;
  if (id >= V) {
    for (int c4 = lane; c4 < n4; c4 += 64) o[c4] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0 && bad != nullptr) atomicAdd(bad, 1);
    return;
  }
  const uint8_t* src = table + (uint64_t)id * (uint64_t)row_bytes;

  // f32 / bf16: groups of kGatherUnroll loads are issued before their stores, so a
  // single long row costs a few memory round trips, not one per 1 KB.  Output rows
  // are written with non-temporal stores (streamed out, not kept in the caches).
  if constexpr (DT == DT_F32) {
    const f32x4* s4 = (const f32x4*)src;
    for (int c0 = lane; c0 < n4; c0 += 64 * kGatherUnroll) {
      f32x4 v[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; u++) {
        const int c4 = c0 + 64 * u;
        if (c4 < n4) v[u] = s4[c4];
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; u++) {
        const int c4 = c0 + 64 * u;
        if (c4 < n4) __builtin_nontemporal_store(SCALE ? v[u] * scale : v[u], o + c4);
      }
    }
  } else if constexpr (DT == DT_BF16 || DT == DT_F16) {
    const u32x4* s8 = (const u32x4*)src;
    const int n8 = hidden >> 3;
    for (int c0 = lane; c0 < n8; c0 += 64 * kGatherUnroll) {
      u32x4 w[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; u++) {
        const int c8 = c0 + 64 * u;
        if (c8 < n8) w[u] = s8[c8];
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; u++) {
        const int c8 = c0 + 64 * u;
        if (c8 < n8) {
          f32x4 a, b;
          if constexpr (DT == DT_BF16) {
            a = f32x4{bf16_lo(w[u].x), bf16_hi(w[u].x), bf16_lo(w[u].y), bf16_hi(w[u].y)};
            b = f32x4{bf16_lo(w[u].z), bf16_hi(w[u].z), bf16_lo(w[u].w), bf16_hi(w[u].w)};
          } else {
            a = f32x4{f16_bits_to_f32(w[u].x & 0xffffu), f16_bits_to_f32(w[u].x >> 16),
                      f16_bits_to_f32(w[u].y & 0xffffu), f16_bits_to_f32(w[u].y >> 16)};
            b = f32x4{f16_bits_to_f32(w[u].z & 0xffffu), f16_bits_to_f32(w[u].z >> 16),
                      f16_bits_to_f32(w[u].w & 0xffffu), f16_bits_to_f32(w[u].w >> 16)};
          }
          if (SCALE) {
            a = a * scale;
            b = b * scale;
          }
          __builtin_nontemporal_store(a, o + 2 * c8);
          __builtin_nontemporal_store(b, o + 2 * c8 + 1);
        }
      }
    }
  } else {
    // Q8_0: the row is staged in pieces of up to kGatherPieceBlocks blocks.  A
    // piece [p, p + 34 nblk) is read as the aligned dwords covering it: block
    // offsets are even and the table base is 16-byte aligned, so p % 4 is 0 or 2;
    // the first dword may start 2 bytes before the piece (inside the row or the
    // previous row, never before the table), and a last dword that would run 2
    // bytes past the piece is read as u16 (past the row's end it would leave the
    // table).
    uint32_t* w = lds_words_buf + wv * lds_words;
    const uint8_t* wb = (const uint8_t*)w;
    const int nb = hidden >> 5;
    for (int b0 = 0; b0 < nb; b0 += kGatherPieceBlocks) {
      const int pb = min(kGatherPieceBlocks, nb - b0);
      const uintptr_t a = (uintptr_t)(src + 34 * b0);
      const uintptr_t a0 = a & ~(uintptr_t)3;
      const int head = (int)(a - a0);
      const int nbytes = head + 34 * pb;
      const int ndw = (nbytes + 3) >> 2;
      const uint32_t* s = (const uint32_t*)a0;
      // the previous piece's reads of w are done before it is overwritten
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int i = lane; i < ndw; i += 64) {
        uint32_t v;
        if (i == ndw - 1 && (nbytes & 3)) v = *(const uint16_t*)(s + i);
        else v = s[i];
        w[i] = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int c4 = 8 * b0 + lane; c4 < 8 * (b0 + pb); c4 += 64) {
        const int c = 4 * c4;
        const int off = head + 34 * ((c >> 5) - b0);  // even
        const float sc = f16_bits_to_f32(*(const uint16_t*)(wb + off));
        const int qo = off + 2 + (c & 31);            // even
        const uint32_t q01 = *(const uint16_t*)(wb + qo);
        const uint32_t q23 = *(const uint16_t*)(wb + qo + 2);
        f32x4 v = {(float)(int8_t)(q01 & 0xffu) * sc, (float)(int8_t)(q01 >> 8) * sc,
                   (float)(int8_t)(q23 & 0xffu) * sc, (float)(int8_t)(q23 >> 8) * sc};
        if (SCALE) v = v * scale;
        __builtin_nontemporal_store(v, o + c4);
      }
    }
  }
}

// Q8_0 rows whose size is a multiple of 16 bytes (d a multiple of 256, e.g. 768:
// 816-byte rows) start 16-byte aligned, so a wave stages a row with one 16-byte
// load per lane.  Each wave gathers kQ8Rows rows, issuing all of their loads
// before unpacking any.  One row per wave measured fastest on the 16,384-id
// EmbeddingGemma gather (9.3-9.5 us against 10.5 us for two and 11.3 us for four
// rows, all with non-temporal output stores): more waves in flight beat more
// loads per wave.
static constexpr int kQ8Rows = 1;
static constexpr int kQ8MaxChunks = 128;  // 16-byte chunks per row (row_bytes <= 2 KiB)

template <bool SCALE>
__global__ void __launch_bounds__(256) gather_q8_aligned_kernel(const uint8_t* __restrict__ table, uint32_t V,
                                                                int hidden, int64_t row_bytes,
                                                                const int32_t* __restrict__ ids, int64_t n,
                                                                float scale, float* __restrict__ out,
                                                                int32_t* __restrict__ bad) {
  constexpr int IT = kQ8MaxChunks / 64;
  __shared__ u32x4 stage[kGatherWaves][kQ8Rows][kQ8MaxChunks];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t r0 = ((int64_t)blockIdx.x * kGatherWaves + wv) * kQ8Rows;
  if (r0 >= n) return;  // whole wave; the kernel has no block-level barrier
  const int nch = (int)(row_bytes >> 4);
  const int n4 = hidden >> 2;
  uint32_t id[kQ8Rows];
  u32x4 v[kQ8Rows][IT];
#pragma unroll
  for (int r = 0; r < kQ8Rows; r++) {
    id[r] = r0 + r < n ? (uint32_t)ids[r0 + r] : V;  // past the end: no load, no store
    const u32x4* src = (const u32x4*)(table + (uint64_t)min(id[r], V - 1) * (uint64_t)row_bytes);
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int c = lane + 64 * it;
      if (id[r] < V && c < nch) v[r][it] = src[c];
    }
  }
#pragma unroll
  for (int r = 0; r < kQ8Rows; r++)
#pragma unroll
    for (int it = 0; it < IT; it++) {
      const int c = lane + 64 * it;
      if (id[r] < V && c < nch) stage[wv][r][c] = v[r][it];
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int r = 0; r < kQ8Rows; r++) {
    if (r0 + r >= n) break;
    f32x4* o = (f32x4*)(out + (r0 + r) * (int64_t)hidden);
    if (id[r] >= V) {
      for (int c4 = lane; c4 < n4; c4 += 64) o[c4] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0 && bad != nullptr) atomicAdd(bad, 1);
      continue;
    }
    const uint8_t* wb = (const uint8_t*)stage[wv][r];
    for (int c4 = lane; c4 < n4; c4 += 64) {
      const int c = 4 * c4;
      const int off = 34 * (c >> 5);  // even
      const float sc = f16_bits_to_f32(*(const uint16_t*)(wb + off));
      const int qo = off + 2 + (c & 31);
      const uint32_t q01 = *(const uint16_t*)(wb + qo);
      const uint32_t q23 = *(const uint16_t*)(wb + qo + 2);
      f32x4 x = {(float)(int8_t)(q01 & 0xffu) * sc, (float)(int8_t)(q01 >> 8) * sc,
                 (float)(int8_t)(q23 & 0xffu) * sc, (float)(int8_t)(q23 >> 8) * sc};
      if (SCALE) x = x * scale;
      __builtin_nontemporal_store(x, o + c4);
    }
  }
}

// Gather with the output rows in a residual wire format (ADR-0009 "Wire Layout";
// the embed output may travel as f16 or as per-position symmetric i8).  x is the
// value the f32 gather writes (exact dequant, then the optional scale):
//   wire 1 (f16): binary16 of x, round to nearest even, clamped to +-65504;
//   wire 2 (i8):  [scale f32][zero point 0 f32][int8 x hidden] per row with
//                 scale = max|x| / 127 and q = round-half-even(x / scale), all in
//                 f32, clamped to [-127, 127]; a row with scale 0 is all zeros.
// A bad id gives an all-zero record.  One wave per row, four consecutive values
// per lane (hidden is a multiple of 4): one load of the four stored values and
// one 8-byte (f16) or 4-byte (i8) store.  The i8 codes need the row maximum
// first: rows of up to 2,048 values keep theirs in registers, longer rows are
// read a second time (L1/L2 hits).
template <int DT>
__device__ __forceinline__ f32x4 deq4(const uint8_t* row, int c) {  // values c .. c + 3, c % 4 == 0
  if constexpr (DT == DT_F32) {
    return *(const f32x4*)(row + 4 * c);
  } else if constexpr (DT == DT_BF16 || DT == DT_F16) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = *(const u32x2*)(row + 2 * c);
    if constexpr (DT == DT_BF16) return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    return f32x4{f16_bits_to_f32(w.x & 0xffffu), f16_bits_to_f32(w.x >> 16), f16_bits_to_f32(w.y & 0xffffu),
                 f16_bits_to_f32(w.y >> 16)};
  } else {
    typedef uint32_t u32a2 __attribute__((aligned(2)));
    const uint8_t* blk = row + 34 * (c >> 5);
    const float sc = f16_bits_to_f32(*(const uint16_t*)blk);
    const uint32_t q = *(const u32a2*)(blk + 2 + (c & 31));  // 2-byte aligned, inside the block
    return f32x4{(float)(int8_t)(q & 0xffu) * sc, (float)(int8_t)((q >> 8) & 0xffu) * sc,
                 (float)(int8_t)((q >> 16) & 0xffu) * sc, (float)(int8_t)(q >> 24) * sc};
  }
}

// Rows of up to 256 kWireRegs values are read once for the i8 codes (the values
// wait in registers for the row maximum); longer rows are read twice.
static constexpr int kWireRegs = 8;

template <int DT, bool SCALE>
__global__ void __launch_bounds__(256) gather_wire_kernel(const uint8_t* __restrict__ table, uint32_t V,
                                                          int hidden, int64_t row_bytes,
                                                          const int32_t* __restrict__ ids, int64_t n, float scale,
                                                          int wire, uint8_t* __restrict__ out,
                                                          int32_t* __restrict__ bad) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kGatherWaves + (threadIdx.x >> 6);
  if (row >= n) return;  // whole wave; no block-level barrier
  const uint32_t id = (uint32_t)ids[row];
  const int64_t orb = wire == WIRE_F16 ? 2 * (int64_t)hidden : (int64_t)hidden + 8;  // a multiple of 4
  uint8_t* o = out + row * orb;
  if (id >= V) {
    for (int i = lane; i < (int)(orb >> 2); i += 64) ((uint32_t*)o)[i] = 0u;
    if (lane == 0 && bad != nullptr) atomicAdd(bad, 1);
    return;
  }
  const uint8_t* src = table + (uint64_t)id * (uint64_t)row_bytes;
  auto value4 = [&](int c) {
    const f32x4 x = deq4<DT>(src, c);
    return SCALE ? x * scale : x;
  };
  if (wire == WIRE_F16) {
    typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));  // the output is 4-byte aligned
    for (int c = 4 * lane; c < hidden; c += 256) {
      const f32x4 x = value4(c);
      *(u32x2a4*)(o + 2 * c) = u32x2a4{f32_to_f16_sat(x[0]) | (f32_to_f16_sat(x[1]) << 16),
                                   f32_to_f16_sat(x[2]) | (f32_to_f16_sat(x[3]) << 16)};
    }
    return;
  }
  auto codes = [&](int c, const f32x4& x, float sc) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float v = sc != 0.f ? fminf(fmaxf(rintf(x[e] / sc), -127.f), 127.f) : 0.f;
      w |= ((uint32_t)(int32_t)v & 0xffu) << (8 * e);
    }
    *(uint32_t*)(o + 8 + c) = w;
  };
  auto store_scale = [&](float sc) {
    if (lane == 0) {
      ((float*)o)[0] = sc;
      ((float*)o)[1] = 0.f;
    }
  };
  auto amax = [](const f32x4& x) { return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))); };
  if (hidden <= 256 * kWireRegs) {
    // one read of the row: its values stay in registers until the maximum is known
    f32x4 xs[kWireRegs];
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < kWireRegs; r++) {
      const int c = 4 * lane + 256 * r;
      xs[r] = c < hidden ? value4(c) : f32x4{0.f, 0.f, 0.f, 0.f};
      m = fmaxf(m, amax(xs[r]));
    }
    m = wave_max_f32(m);
    const float sc = m / 127.0f;  // correctly rounded f32 division
    store_scale(sc);
#pragma unroll
    for (int r = 0; r < kWireRegs; r++) {
      const int c = 4 * lane + 256 * r;
      if (c < hidden) codes(c, xs[r], sc);
    }
    return;
  }
  float m = 0.f;
  for (int c = 4 * lane; c < hidden; c += 256) m = fmaxf(m, amax(value4(c)));
  m = wave_max_f32(m);
  const float sc = m / 127.0f;  // correctly rounded f32 division
  store_scale(sc);
  for (int c = 4 * lane; c < hidden; c += 256) codes(c, value4(c), sc);
}

template <int DT>
static hipError_t launch_wire_dt(const TableDesc& t, const int32_t* ids, int64_t n, float scale, int32_t wire,
                                 uint8_t* out, int32_t* bad, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kGatherWaves - 1) / kGatherWaves)), block(64 * kGatherWaves);
  if (!(scale == 1.0f))
    hipLaunchKernelGGL((gather_wire_kernel<DT, true>), grid, block, 0, stream, t.rows, (uint32_t)t.V,
                       (int)t.hidden, t.row_bytes, ids, n, scale, (int)wire, out, bad);
  else
    hipLaunchKernelGGL((gather_wire_kernel<DT, false>), grid, block, 0, stream, t.rows, (uint32_t)t.V,
                       (int)t.hidden, t.row_bytes, ids, n, scale, (int)wire, out, bad);
  return hipGetLastError();
}

hipError_t launch_gather_wire(const TableDesc& t, const int32_t* ids, int64_t n, float scale, int32_t wire,
                              uint8_t* out, int32_t* bad, hipStream_t stream) {
  const int64_t rb = wire == WIRE_F16 ? 2 * t.hidden : t.hidden + 8;
  for (int64_t r0 = 0; r0 < n; r0 += kGatherLaunchRows) {
    const int64_t m = std::min(kGatherLaunchRows, n - r0);
    uint8_t* o = out + r0 * rb;
    hipError_t e;
    switch (t.dtype) {
      case DT_F32: e = launch_wire_dt<DT_F32>(t, ids + r0, m, scale, wire, o, bad, stream); break;
      case DT_BF16: e = launch_wire_dt<DT_BF16>(t, ids + r0, m, scale, wire, o, bad, stream); break;
      case DT_F16: e = launch_wire_dt<DT_F16>(t, ids + r0, m, scale, wire, o, bad, stream); break;
      default: e = launch_wire_dt<DT_Q8_0>(t, ids + r0, m, scale, wire, o, bad, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT>
static hipError_t launch_dt(const TableDesc& t, const int32_t* ids, int64_t n, float scale, float* out,
                            int32_t* bad, hipStream_t stream) {
  const bool sc = !(scale == 1.0f);
  const dim3 grid((unsigned)((n + kGatherWaves - 1) / kGatherWaves));
  const dim3 block(64 * kGatherWaves);
  int lds_words = 0;
  size_t lds = 0;
  if (DT == DT_Q8_0) {
    if (t.row_bytes % 16 == 0 && t.row_bytes <= 16 * kQ8MaxChunks) {
      const dim3 g((unsigned)((n + kGatherWaves * kQ8Rows - 1) / (kGatherWaves * kQ8Rows)));
      if (sc)
        hipLaunchKernelGGL((gather_q8_aligned_kernel<true>), g, block, 0, stream, t.rows, (uint32_t)t.V,
                           (int)t.hidden, t.row_bytes, ids, n, scale, out, bad);
      else
        hipLaunchKernelGGL((gather_q8_aligned_kernel<false>), g, block, 0, stream, t.rows, (uint32_t)t.V,
                           (int)t.hidden, t.row_bytes, ids, n, scale, out, bad);
      return hipGetLastError();
    }
    lds_words = (34 * kGatherPieceBlocks + 4) / 4;
    lds = (size_t)kGatherWaves * lds_words * 4;
  }
  if (sc)
    hipLaunchKernelGGL((gather_kernel<DT, true>), grid, block, lds, stream, t.rows, (uint32_t)t.V,
                       (int)t.hidden, t.row_bytes, ids, n, scale, out, bad, lds_words);
  else
    hipLaunchKernelGGL((gather_kernel<DT, false>), grid, block, lds, stream, t.rows, (uint32_t)t.V,
                       (int)t.hidden, t.row_bytes, ids, n, scale, out, bad, lds_words);
  return hipGetLastError();
}

hipError_t launch_gather(const TableDesc& t, const int32_t* ids, int64_t n, float scale, float* out,
                         int32_t* bad, hipStream_t stream) {
  for (int64_t r0 = 0; r0 < n; r0 += kGatherLaunchRows) {
    const int64_t m = std::min(kGatherLaunchRows, n - r0);
    float* o = out + r0 * t.hidden;
    hipError_t e;
    switch (t.dtype) {
      case DT_F32: e = launch_dt<DT_F32>(t, ids + r0, m, scale, o, bad, stream); break;
      case DT_BF16: e = launch_dt<DT_BF16>(t, ids + r0, m, scale, o, bad, stream); break;
      case DT_F16: e = launch_dt<DT_F16>(t, ids + r0, m, scale, o, bad, stream); break;
      default: e = launch_dt<DT_Q8_0>(t, ids + r0, m, scale, o, bad, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace etg
