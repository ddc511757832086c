// Split-K combine: merge the per-split partials (m_s, l_s, o_s) of each
// (sequence, query head), and with a shared prefix the prefix pass's
// partials too, into the attention output
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// over the splits that hold tokens (ceil(len / split_tokens) of them, or,
// under the balanced schedule, the pieces the unit's first piece recorded),
// then round to the output dtype.  A sequence with no tokens gives zeros.  This
// is the finalize step that follows the tile accumulation in
// metrale_storage high_speed_swap/impl_more.rs attend_layer.
//
// Also here: the block-table update kernel (tiny-llm paged_kv.py begin_step
// writes newly allocated blocks into the device table by index).
#include <algorithm>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// One wave per (sequence, query head).  Up to 64 splits: one split per lane
// for the weights 2^(m_s - M), which stay in registers, and each lane owns
// every 64th pair of dims (one pair up to head_dim 128, two up to 256), the
// first 8 splits' partial outputs loaded together with the (m, l) pairs.  More splits: the weights go through LDS and each lane sums
// the splits' partial outputs with 8 loads in flight.
__global__ __launch_bounds__(64) void reduce_kernel(AttendArgs a) {
  extern __shared__ float wsplit[];  // [pieces] weights
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;  // b * n_q_heads + h
  const int b = bh / a.n_q_heads;
  const int D = a.head_dim;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int64_t oi0 = (int64_t)bh * D;
  // With a shared prefix every output is written here: the prefix pass left
  // n_pchunks partials per (sequence, query head), the split pass one per
  // piece of the private suffix (len - prefix_len tokens).
  const int npre = a.prefix_len > 0 ? a.n_pchunks : 0;
  if (npre > 0 && len == 0) {
    for (int d2 = lane; 2 * d2 < D; d2 += 64) {
      if (a.q_bf16)
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi0 + 2 * d2) = 0u;
      else
        *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi0 + 2 * d2) = float2{0.f, 0.f};
    }
    return;
  }
  const int slen = npre > 0 ? max(len - a.prefix_len, 0) : len;  // tokens of the split pass
  // suffix piece s of this (sequence, query head) sits in workspace row
  // row0 + s * rstep
  int n = 0;
  int64_t row0 = 0;
  int rstep = 1;
  if (a.bal_waves > 0 && *a.ws_sched) {
    // balanced schedule: the unit's pieces, as its first piece recorded them
    if (slen == 0 && npre == 0) return;  // the split pass wrote zeros
    if (slen > 0) {
      const int h = bh - b * a.n_q_heads;
      const int unit = b * a.n_kv_heads + h / a.group;
      const int2 d = *reinterpret_cast<const int2*>(a.ws_desc + 2 * unit);
      n = d.y;
      if (n <= 1 && npre == 0) return;  // one piece: the split pass wrote this output
      row0 = (int64_t)d.x * a.group + (h - (h / a.group) * a.group);
      rstep = a.group;
    }
  } else {
    n = (slen + a.split_tokens - 1) / a.split_tokens;
    if (a.single_done && n == 1) return;  // the split pass wrote this output
    row0 = (int64_t)bh * a.n_split;
    rstep = 1;
  }
  const float* ml = a.ws_ml + row0 * 2;
  const float* po = a.ws_o + row0 * D;
  const int64_t pstep = (int64_t)rstep * D;
  // pieces n .. n + npre - 1 are the prefix partials
  const float* pml = npre > 0 ? a.ws_pre_ml + (int64_t)bh * npre * 2 : nullptr;
  const float* ppo = npre > 0 ? a.ws_pre_o + (int64_t)bh * npre * D : nullptr;
  auto ml_of = [&](int p) -> const float* {
    return p < n ? ml + 2 * (int64_t)rstep * p : pml + 2 * (int64_t)(p - n);
  };
  auto o_of = [&](int p) -> const float* {
    return p < n ? po + p * pstep : ppo + (int64_t)(p - n) * D;
  };
  const int np = n + npre;

  if (np <= 64) {
    // one piece per lane: the weights stay in registers (read back per piece
    // with a lane read); each lane owns dims 2 d2, 2 d2 + 1 for d2 = lane,
    // lane + 64, ...  The first dim pair's partial outputs of the first 8
    // pieces are loaded together with the (m, l) pairs.
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = 2 * lane < D && u < np ? *reinterpret_cast<const float2*>(o_of(u) + 2 * lane)
                                    : float2{0.f, 0.f};
    const float2 mlv = lane < np ? *reinterpret_cast<const float2*>(ml_of(lane))
                                 : float2{-INFINITY, 0.f};
    const float M = wave_max(mlv.x);
    const float w = lane < np ? exp2f(mlv.x - M) : 0.f;
    const float L = wave_sum(w * mlv.y);
    const float inv = np > 0 ? 1.f / L : 0.f;
    for (int d2 = lane; 2 * (d2 - lane) < D; d2 += 64) {  // uniform trip count
      const bool has_d = 2 * d2 < D;
      if (d2 != lane) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = has_d && u < np ? *reinterpret_cast<const float2*>(o_of(u) + 2 * d2)
                                 : float2{0.f, 0.f};
      }
      float2 acc = {0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < np) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
          acc.x = fmaf(wu, x[u].x, acc.x);
          acc.y = fmaf(wu, x[u].y, acc.y);
        }
      }
      for (int s0 = 8; s0 < np; s0 += 8) {  // further pieces, 8 loads in flight
        float2 y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          y[u] = has_d && s0 + u < np
                     ? *reinterpret_cast<const float2*>(o_of(s0 + u) + 2 * d2)
                     : float2{0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u));
          acc.x = fmaf(ws, y[u].x, acc.x);
          acc.y = fmaf(ws, y[u].y, acc.y);
        }
      }
      if (has_d) {
        const float r0 = acc.x * inv, r1 = acc.y * inv;
        const int64_t oi = oi0 + 2 * d2;
        if (a.q_bf16)
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) =
              f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16);
        else
          *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi) = float2{r0, r1};
      }
    }
    return;
  }

  float M = -INFINITY;
  for (int s = lane; s < np; s += 64) M = fmaxf(M, ml_of(s)[0]);
  M = wave_max(M);
  float L = 0.f;
  for (int s = lane; s < np; s += 64) {
    const float2 x = *reinterpret_cast<const float2*>(ml_of(s));
    const float w = exp2f(x.x - M);
    wsplit[s] = w;
    L = fmaf(w, x.y, L);
  }
  L = wave_sum(L);
  __syncthreads();
  const float inv = np > 0 ? 1.f / L : 0.f;

  for (int d2 = lane; 2 * d2 < D; d2 += 64) {
    float2 acc = {0.f, 0.f};
    int s = 0;
    for (; s + 8 <= np; s += 8) {
      float2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const float2*>(o_of(s + u) + 2 * d2);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x = fmaf(wsplit[s + u], x[u].x, acc.x);
        acc.y = fmaf(wsplit[s + u], x[u].y, acc.y);
      }
    }
    for (; s < np; ++s) {
      const float2 x = *reinterpret_cast<const float2*>(o_of(s) + 2 * d2);
      acc.x = fmaf(wsplit[s], x.x, acc.x);
      acc.y = fmaf(wsplit[s], x.y, acc.y);
    }
    const float r0 = acc.x * inv, r1 = acc.y * inv;
    const int64_t oi = oi0 + 2 * d2;
    if (a.q_bf16)
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) =
          f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16);
    else
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi) = float2{r0, r1};
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

hipError_t launch_reduce(const AttendArgs& a, const Launch& l) {
  if (a.batch <= 0) return hipSuccess;
  const int max_n = (a.bal_waves > 0 ? std::max(a.n_split, a.bal_waves) : a.n_split) +
                    (a.prefix_len > 0 ? a.n_pchunks : 0);
  return launch1(reduce_kernel, dim3(a.batch * a.n_q_heads), dim3(64),
                 (size_t)max_n * sizeof(float), l, a);
}

hipError_t launch_table_apply(int32_t* table, int32_t stride, int32_t batch, const int32_t* upd,
                              int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_apply_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, stride,
                     batch, upd, n);
  return hipGetLastError();
}

}  // namespace pkv
