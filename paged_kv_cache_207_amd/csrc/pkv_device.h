// Device helpers shared by the kernels: bf16 bit conversions, wave
// reductions, status reporting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

// ---- K page layout -------------------------------------------------------
// A (page, KV head) slab of K holds page_size token rows of head_dim
// elements.  Rows of 64 or 128 bytes (bf16 head_dim 64, int8 head_dim 64 or
// 128) are stored piece-major: the first 64 bytes of every row, then the
// next 64 bytes of every row, with the rows of a piece in k_slot order, which
// places next to each other the rows one score tile of a 32-token step takes
// from a page (tokens 8i + 4t + 0..3 for tile t).  A K load of the
// matrix-core kernels (16 rows x 64 bytes per instruction) then reads runs
// of 512 bytes or more instead of 16 separate 64-byte pieces: on gfx950,
// reads of 4 KiB blocks as 16 pieces of 64 bytes per instruction stream at
// 5.9 TB/s, as runs of 512 bytes at 6.8 (in-order reads 6.85); the
// shared-prefix split launch (head_dim 64) went from 66.3 to 61.7 us, the
// int8 split pass from 88.8 to 87.3.  Other rows keep slot order, whole
// (bf16 head_dim 128 measured 1% slower piece-major).
__host__ __device__ constexpr bool k_pieced(int row_bytes) {
  return row_bytes == 64 || row_bytes == 128;
}
__host__ __device__ constexpr int k_slot(int t, int bs, int row_bytes) {
  return (!k_pieced(row_bytes) || (bs & 7)) ? t
                                            : ((t >> 2) & 1) * (bs >> 1) + (t >> 3) * 4 + (t & 3);
}
// Byte offset, within its slab, of byte b of token t's K row.
__host__ __device__ constexpr int k_byte(int t, int b, int bs, int row_bytes) {
  return k_pieced(row_bytes) ? ((b >> 6) * bs + k_slot(t, bs, row_bytes)) * 64 + (b & 63)
                             : t * row_bytes + b;
}

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

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two float32 -> packed bfloat16 (lo in bits 0-15), round to nearest even:
// one v_cvt_pk_bf16_f32 (a scalar cast compiles to a NaN-checking sequence).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// The larger of two floats as one v_maximum3_f32 (IEEE maximum: a NaN input
// gives NaN).  fmaxf must quiet signalling NaNs first, an extra move per
// operand that is not a known arithmetic result; the callers here never
// pass NaN (a score the column may not see is -inf).
__device__ __forceinline__ float fmax_fast(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one lane of each
// 16-lane row), without LDS: v_permlane16_swap leaves rows (0, 0, 2, 2) in
// one register and (1, 1, 3, 3) in the other, so combining the two pairs
// rows 0-1 and 2-3; v_permlane32_swap then does the same for the two halves.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmax_fast(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmax_fast(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane I of each 16-lane row, broadcast to the row (DPP row_newbcast).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + I, 0xf, 0xf,
                                                    false));
}

// DPP move of lane values within 16-lane rows (dpp_ctrl C: 0xB1 and 0x4E
// swap neighbours and pairs inside each group of 4, 0x141 mirrors each
// half-row of 8, 0x140 each row of 16).
template <int C>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xf, 0xf, false));
}

// Max / sum over the whole wave, in every lane, without LDS: within rows by
// DPP (pairs, quads, half-rows, rows), then across the four rows.
__device__ __forceinline__ float wave_max(float x) {
  x = fmax_fast(x, dpp_mov<0xB1>(x));
  x = fmax_fast(x, dpp_mov<0x4E>(x));
  x = fmax_fast(x, dpp_mov<0x141>(x));
  x = fmax_fast(x, dpp_mov<0x140>(x));
  return rows_max(x);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return rows_sum(x);
}

// Inclusive prefix sum over the wave's 64 lanes, without LDS: DPP row
// shifts by 1, 2, 4 and 8 inside each 16-lane row (lanes shifted in from
// outside the row read 0), then lane 15's sum added into rows 1 and 3 and
// lane 31's into rows 2 and 3 (row broadcasts).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, true);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = dpp_add<0x111, 0xf>(x);
  x = dpp_add<0x112, 0xf>(x);
  x = dpp_add<0x114, 0xf>(x);
  x = dpp_add<0x118, 0xf>(x);
  x = dpp_add<0x142, 0xa>(x);
  x = dpp_add<0x143, 0xc>(x);
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
