// Device helpers shared by the kernels: bf16 bit conversions, wave
// reductions, status reporting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ void report(int32_t* status, uint32_t bit) {
  if (status) atomicOr(reinterpret_cast<unsigned int*>(status), bit);
}

__device__ __forceinline__ int clamp_len(int len, int max_len, int32_t* status, uint32_t bit) {
  if (len < 0 || len > max_len) {
    report(status, bit);
    len = len < 0 ? 0 : max_len;
  }
  return len;
}

}  // namespace pkv
