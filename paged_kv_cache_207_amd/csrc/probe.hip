// Streaming probes: a read of every byte of a buffer (16-byte non-temporal
// loads, four in flight per thread) and a plain copy.  They give the
// achievable-bandwidth denominator next to the 8 TB/s HBM peak, and a copy
// of known size against which hardware traffic counters are calibrated.
// Measured over grid sizes and load kinds, the read is fastest with many
// small workgroups and non-temporal loads, the form used here.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 32768;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{t.x, t.y, t.z, t.w};
}

__global__ __launch_bounds__(kThreads) void probe_read(const uint4* src, uint64_t n, float* sink) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = nt_load(src + i), b = nt_load(src + i + stride),
                c = nt_load(src + i + 2 * stride), d = nt_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = nt_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = __uint_as_float(red[0]);
}

__global__ __launch_bounds__(kThreads) void probe_copy(const uint4* src, uint4* dst, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

int probe_blocks(uint64_t bytes) {
  const uint64_t n = bytes / 16;
  uint64_t blocks = (n + kThreads - 1) / kThreads;
  return (int)(blocks < 1 ? 1 : (blocks > kMaxBlocks ? kMaxBlocks : blocks));
}

hipError_t launch_probe(const void* src, void* dst, float* sink, uint64_t bytes, int mode,
                        hipStream_t s) {
  const uint64_t n = bytes / 16;
  const int blocks = probe_blocks(bytes);
  if (mode == 0)
    hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(src), n, sink);
  else
    hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

}  // namespace pkv
