// Split-K combine: merge the per-split partials (m_s, l_s, o_s) of each
// (sequence, query head) into the attention output
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// over the splits that hold tokens (ceil(len / split_tokens) of them), then
// round to the output dtype.  A sequence with no tokens gives zeros.  This
// is the finalize step that follows the tile accumulation in
// metrale_storage high_speed_swap/impl_more.rs attend_layer.
//
// Also here: the block-table update kernel (tiny-llm paged_kv.py begin_step
// writes newly allocated blocks into the device table by index).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(64) void reduce_kernel(AttendArgs a) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;  // b * n_q_heads + h
  const int b = bh / a.n_q_heads;
  const int D = a.head_dim;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int n = (len + a.split_tokens - 1) / a.split_tokens;
  const int64_t row0 = (int64_t)bh * a.n_split;

  float M = -INFINITY;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, a.ws_ml[(row0 + s) * 2]);
  M = wave_max(M);
  float L = 0.f;
  for (int s = lane; s < n; s += 64) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (row0 + s) * 2);
    L += exp2f(ml.x - M) * ml.y;
  }
  L = wave_sum(L);
  const float inv = n > 0 ? 1.f / L : 0.f;

  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = exp2f(a.ws_ml[(row0 + s) * 2] - M);
      acc = fmaf(w, a.ws_o[(row0 + s) * D + d], acc);
    }
    const float r = acc * inv;
    const int64_t oi = (int64_t)bh * D + d;
    if (a.q_bf16)
      static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(r);
    else
      static_cast<float*>(a.out)[oi] = r;
  }
}

__global__ void table_apply_kernel(int32_t* table, int32_t stride, int32_t batch,
                                   const int32_t* upd, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int b = upd[3 * i], j = upd[3 * i + 1];
  if (b < 0 || b >= batch || j < 0 || j >= stride) return;
  table[(int64_t)b * stride + j] = upd[3 * i + 2];
}

}  // namespace

hipError_t launch_reduce(const AttendArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_kernel, dim3(a.batch * a.n_q_heads), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_table_apply(int32_t* table, int32_t stride, int32_t batch, const int32_t* upd,
                              int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_apply_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, stride,
                     batch, upd, n);
  return hipGetLastError();
}

}  // namespace pkv
