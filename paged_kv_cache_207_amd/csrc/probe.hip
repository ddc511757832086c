// Streaming probes: a read of every byte of a buffer, in order or as 4 KiB
// blocks in a scrambled order (the access of a fragmented page pool: each
// page slab of a (16-token, 128-dim, bf16) page is one 4 KiB block), and a
// plain copy.  They give the achievable-bandwidth denominators next to the
// 8 TB/s HBM peak, and a copy of known size against which hardware traffic
// counters are calibrated.  The reads use single-wave workgroups of 16
// blocks each, 16-byte non-temporal loads and four blocks (16 KiB) in flight
// per wave: measured faster than a grid-stride loop over the whole buffer
// (7.0-7.1 against 6.85 TB/s in order).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kCopyBlocks = 32768;
constexpr int kBlockBytes = 4096;  // 64 lanes x 64 bytes
constexpr int kPerWave = 16;       // blocks per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A bijection of [0, 2^bits): two rounds of an odd multiply and a
// xor-shift, each invertible on bits-wide integers.
__device__ __forceinline__ uint32_t scramble(uint32_t x, int bits) {
  const uint32_t mask = bits >= 32 ? 0xffffffffu : (1u << bits) - 1u;
  const int sh = bits / 2 + 1;
  x = (x * 0x9E3779B1u + 0x7F4A7C15u) & mask;
  x ^= x >> sh;
  x = (x * 0x85EBCA77u + 0x165667B1u) & mask;
  x ^= x >> sh;
  return x;
}

// Read blocks [kPerWave w, kPerWave (w + 1)) of n_blk 4 KiB blocks (their
// scrambled ids when bits > 0), then, in workgroup 0, the tail_16 16-byte
// words past the last whole block.
__global__ __launch_bounds__(64) void probe_read(const char* src, uint32_t n_blk, int bits,
                                                 uint32_t tail_16, float* sink) {
  const int lane = threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  const uint32_t b0 = blockIdx.x * kPerWave;
  const uint32_t cnt = min((uint32_t)kPerWave, n_blk - min(b0, n_blk));
  auto at = [&](uint32_t i) -> const char* {
    const uint32_t id = bits ? scramble(b0 + i, bits) : b0 + i;
    return src + (uint64_t)id * kBlockBytes + lane * 16;
  };
  uint32_t i = 0;
  for (; i + 4 <= cnt; i += 4) {
    u32x4 v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const char* p = at(i + u);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[u][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + k * 1024));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[u][k];
  }
  for (; i < cnt; ++i) {
    const char* p = at(i);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + k * 1024));
  }
  if (blockIdx.x == 0) {
    const u32x4* t = reinterpret_cast<const u32x4*>(src + (uint64_t)n_blk * kBlockBytes);
    for (uint32_t w = lane; w < tail_16; w += 64) acc ^= __builtin_nontemporal_load(t + w);
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= __shfl_xor(x, o, 64);
  if (lane == 0) sink[blockIdx.x] = __uint_as_float(x);
}

__global__ __launch_bounds__(kThreads) void probe_copy(const uint4* src, uint4* dst, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

int probe_blocks(uint64_t bytes) {
  const uint64_t n_blk = bytes / kBlockBytes;
  const uint64_t wgs = (n_blk + kPerWave - 1) / kPerWave;
  return (int)(wgs < 1 ? 1 : wgs);
}

hipError_t launch_probe(const void* src, void* dst, float* sink, uint64_t bytes, int mode,
                        hipStream_t s) {
  const uint64_t n = bytes / 16;
  if (mode == 1) {
    const uint64_t want = (n + kThreads - 1) / kThreads;
    const int blocks = (int)(want < 1 ? 1 : (want > kCopyBlocks ? kCopyBlocks : want));
    hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
    return hipGetLastError();
  }
  const uint64_t n_blk = bytes / kBlockBytes;
  int bits = 0;
  if (mode == 2)
    while ((1ull << bits) < n_blk) ++bits;
  const uint32_t tail = (uint32_t)((bytes - n_blk * kBlockBytes) / 16);
  hipLaunchKernelGGL(probe_read, dim3(probe_blocks(bytes)), dim3(64), 0, s,
                     static_cast<const char*>(src), (uint32_t)n_blk, bits, tail, sink);
  return hipGetLastError();
}

}  // namespace pkv
