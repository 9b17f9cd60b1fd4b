// zf_probe.hip - a plain streaming read and a plain streaming copy of device memory (gfx950):
// the practically achievable HBM read rate, against which the attention kernel's bandwidth is
// read, and the achievable read-plus-write rate, against which the codec kernels' is.
// Measurement aids, outside the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/zf.h"

namespace zf {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

// Block b reads its contiguous share of the buffer, 4 x 16 bytes per thread in flight with the
// non-temporal hint (the fastest plain read measured on gfx950), and
// leaves the XOR of everything it read in sink[b] (so no load can be dropped).
__global__ __launch_bounds__(kProbeThreads) void stream_read_k(const uint4* __restrict__ p, uint64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t b0 = (uint64_t)blockIdx.x * per, b1 = min(n16, b0 + per);
  uint32_t x = 0;
  for (uint64_t i = b0 + threadIdx.x; i < b1; i += kProbeUnroll * kProbeThreads) {
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const uint64_t j = i + (uint64_t)u * kProbeThreads;
      if (j < b1) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + j);  // streamed
        x ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  // XOR over the block: wave, then waves through LDS
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t s_x[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= s_x[w];
    sink[blockIdx.x] = y;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// Grid-stride copy, 4 x 16 bytes per thread per pass, non-temporal loads and stores (the
// fastest plain copy measured on gfx950 among 1024-262144 workgroups, unroll 1-8 and each
// cache hint on or off: ~6.3 TB/s read plus written at 32768 workgroups).
__global__ __launch_bounds__(kCopyThreads) void stream_copy_k(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                              uint64_t n16) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint64_t chunk = (uint64_t)kCopyThreads * kCopyUnroll;
  for (uint64_t b0 = (uint64_t)blockIdx.x * chunk; b0 < n16; b0 += (uint64_t)gridDim.x * chunk) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t j = b0 + threadIdx.x + (uint64_t)u * kCopyThreads;
      if (j < n16) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + j);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t j = b0 + threadIdx.x + (uint64_t)u * kCopyThreads;
      if (j < n16) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst) + j);
    }
  }
}

}  // namespace zf

extern "C" zf_status zf_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, zf_stream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0) return ZF_EINVAL;
  const uint64_t n16 = bytes / 16;
  const uint64_t per_block = (uint64_t)zf::kProbeThreads * zf::kProbeUnroll;
  const uint32_t blocks = (uint32_t)std::min<uint64_t>(ZF_PROBE_BLOCKS, (n16 + per_block - 1) / per_block);
  hipLaunchKernelGGL(zf::stream_read_k, dim3(blocks), dim3(zf::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? ZF_OK : ZF_EHIP;
}

extern "C" zf_status zf_stream_copy_probe(const void* src, void* dst, size_t bytes, zf_stream_t stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0)
    return ZF_EINVAL;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return ZF_EINVAL;  // overlapping ranges
  const uint64_t n16 = bytes / 16;
  const uint64_t per_block = (uint64_t)zf::kCopyThreads * zf::kCopyUnroll;
  const uint32_t blocks = (uint32_t)std::min<uint64_t>(ZF_COPY_PROBE_BLOCKS, (n16 + per_block - 1) / per_block);
  hipLaunchKernelGGL(zf::stream_copy_k, dim3(blocks), dim3(zf::kCopyThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? ZF_OK : ZF_EHIP;
}
