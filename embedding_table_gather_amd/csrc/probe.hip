// Plain read and write streams of a device buffer: the measured HBM read and
// write bandwidths that the table-streaming kernels (reads) and the gathers
// (mostly writes) are compared with, beside the nominal 8 TB/s.
#include "etg_device.hpp"
#include "etg_internal.hpp"

namespace etg {

// Each wave owns a contiguous range of 1 KiB blocks of the buffer and reads it
// as 1 KiB non-temporal load instructions (lane l: 16-byte chunk l of a block),
// 8 blocks per iteration (indices past the range end are clamped to its last
// block and not folded), folding each word into a running XOR once.  The XOR is stored only if it
// equals a fixed word, so the loads stay live and nothing is written in practice.
// Chunks past the last whole block are read by wave 0.
static constexpr int kProbeThreads = 1024;  // 16 waves, one workgroup per CU
__global__ void __launch_bounds__(kProbeThreads) hbm_read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                       uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t gw = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t nb = n16 / 64;
  const int64_t b0 = gw * nb / nw, b1 = (gw + 1) * nb / nw;
  uint32_t x = 0;
  for (int64_t b = b0; b < b1; b += 8) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = __builtin_nontemporal_load(src + min(b + j, b1 - 1) * 64 + lane);
#pragma unroll
    for (int j = 0; j < 8; j++) x ^= b + j < b1 ? v[j].x ^ v[j].y ^ v[j].z ^ v[j].w : 0u;  // clamped copies: not folded
  }
  if (gw == 0) {
    for (int64_t c = nb * 64 + lane; c < n16; c += 64) {
      const u32x4 v = src[c];
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(kTargetBlocks), dim3(kProbeThreads), 0, stream, (const u32x4*)src,
                     bytes / 16, sink);
  return hipGetLastError();
}

// Each wave owns a contiguous range of 1 KiB blocks and writes it with 1 KiB
// non-temporal store instructions (lane l: 16-byte chunk l of a block), 8 blocks
// per iteration; chunks past the last whole block are written by wave 0.  Every
// 32-bit word of the buffer receives `value`.
__global__ void __launch_bounds__(kProbeThreads) hbm_write_probe_kernel(u32x4* __restrict__ dst, int64_t n16,
                                                                        uint32_t value) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t gw = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t nb = n16 / 64;
  const int64_t b0 = gw * nb / nw, b1 = (gw + 1) * nb / nw;
  const u32x4 v = {value, value, value, value};
  for (int64_t b = b0; b < b1; b += 8) {
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (b + j < b1) __builtin_nontemporal_store(v, dst + (b + j) * 64 + lane);
  }
  if (gw == 0)
    for (int64_t c = nb * 64 + lane; c < n16; c += 64) dst[c] = v;
}

hipError_t launch_write_probe(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_write_probe_kernel, dim3(kTargetBlocks), dim3(kProbeThreads), 0, stream, (u32x4*)dst,
                     bytes / 16, value);
  return hipGetLastError();
}

}  // namespace etg
