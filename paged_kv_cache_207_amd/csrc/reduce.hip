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

// One wave per (sequence, query head).  Up to 64 pieces: one piece per lane
// for the weights 2^(m_s - M), which stay in registers, and each lane owns a
// pair of dims (WIDE, head_dim above 128: every 64th pair), the first 8
// pieces' partial outputs loaded together with the (m, l) pairs.  More
// pieces: the weights go through LDS and each lane sums the partial outputs
// with 8 loads in flight.
//
// PRE (shared-prefix mode): the pieces are the prefix pass's n_pchunks
// partials of this (sequence, query head) first, then the split pass's
// pieces of the private suffix (len - prefix_len tokens), and every output
// is written here (zeros for an empty sequence).
template <bool WIDE, bool PRE>
__global__ __launch_bounds__(64) void reduce_kernel(AttendArgs a) {
  extern __shared__ float wsplit[];  // [pieces] weights
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;  // b * n_q_heads + h
  const int b = bh / a.n_q_heads;
  const int D = a.head_dim;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int64_t oi0 = (int64_t)bh * D;
  const int npre = PRE ? a.n_pchunks : 0;
  if (PRE && len == 0) {
    for (int d2 = lane; 2 * d2 < D; d2 += 64) {
      if (a.q_bf16)
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi0 + 2 * d2) = 0u;
      else
        *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi0 + 2 * d2) = float2{0.f, 0.f};
    }
    return;
  }
  const int slen = PRE ? max(len - a.prefix_len, 0) : len;  // tokens of the split pass
  // split piece s of this (sequence, query head) sits in workspace row
  // row0 + s * rstep
  int n = 0;
  int64_t row0 = 0;
  int rstep = 1;
  if (a.bal_waves > 0 && *a.ws_sched) {
    // balanced schedule: the unit's pieces, as its first piece recorded them
    if (!PRE && slen == 0) return;  // the split pass wrote zeros
    if (slen > 0) {
      const int h = bh - b * a.n_q_heads;
      const int unit = b * a.n_kv_heads + h / a.group;
      const int2 d = *reinterpret_cast<const int2*>(a.ws_desc + 2 * unit);
      n = d.y;
      if (!PRE && n <= 1) return;  // one piece: the split pass wrote this output
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
  const float* pml = PRE ? a.ws_pre_ml + (int64_t)bh * npre * 2 : nullptr;
  const float* ppo = PRE ? a.ws_pre_o + (int64_t)bh * npre * D : nullptr;
  const int np = npre + n;  // pieces: prefix partials, then split pieces
  // partial output of piece p (the branch is uniform)
  auto o_of = [&](int p) -> const float* {
    return PRE && p < npre ? ppo + (int64_t)p * D : po + (p - npre) * pstep;
  };
  auto ml_of = [&](int p) -> const float* {
    return PRE && p < npre ? pml + 2 * (int64_t)p : ml + 2 * (int64_t)rstep * (p - npre);
  };

  if (np <= 64) {
    int d2 = lane;  // dims 2 d2, 2 d2 + 1
    bool has_d = 2 * d2 < D;
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = has_d && u < np ? *reinterpret_cast<const float2*>(o_of(u) + 2 * d2)
                             : float2{0.f, 0.f};
    const float2 mlv = lane < np ? *reinterpret_cast<const float2*>(ml_of(lane))
                                 : float2{-INFINITY, 0.f};
    const float M = wave_max(mlv.x);
    const float w = lane < np ? exp2f(mlv.x - M) : 0.f;
    const float L = wave_sum(w * mlv.y);
    const float inv = np > 0 ? 1.f / L : 0.f;
    for (;;) {
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
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = has_d && s0 + u < np
                     ? *reinterpret_cast<const float2*>(o_of(s0 + u) + 2 * d2)
                     : float2{0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u));
          acc.x = fmaf(ws, x[u].x, acc.x);
          acc.y = fmaf(ws, x[u].y, acc.y);
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
      if (!WIDE) return;
      // head_dim above 128: the next 64 dim pairs
      d2 += 64;
      if (2 * (d2 - lane) >= D) return;
      has_d = 2 * d2 < D;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = has_d && u < np ? *reinterpret_cast<const float2*>(o_of(u) + 2 * d2)
                               : float2{0.f, 0.f};
    }
  }

  float M = -INFINITY;
  for (int s = lane; s < np; s += 64) M = fmaxf(M, ml_of(s)[0]);
  M = wave_max(M);
  float L = 0.f;
  for (int s = lane; s < np; s += 64) {
    const float2 y = *reinterpret_cast<const float2*>(ml_of(s));
    const float w = exp2f(y.x - M);
    wsplit[s] = w;
    L = fmaf(w, y.y, L);
  }
  L = wave_sum(L);
  __syncthreads();
  const float inv = np > 0 ? 1.f / L : 0.f;

  for (int d2 = lane; 2 * d2 < D; d2 += 64) {
    float2 acc = {0.f, 0.f};
    int s = 0;
    for (; s + 8 <= np; s += 8) {
      float2 y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = *reinterpret_cast<const float2*>(o_of(s + u) + 2 * d2);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x = fmaf(wsplit[s + u], y[u].x, acc.x);
        acc.y = fmaf(wsplit[s + u], y[u].y, acc.y);
      }
    }
    for (; s < np; ++s) {
      const float2 y = *reinterpret_cast<const float2*>(o_of(s) + 2 * d2);
      acc.x = fmaf(wsplit[s], y.x, acc.x);
      acc.y = fmaf(wsplit[s], y.y, acc.y);
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
  const bool pre = a.prefix_len > 0;
  const int max_n = (a.bal_waves > 0 ? std::max(a.n_split, a.bal_waves) : a.n_split) +
                    (pre ? a.n_pchunks : 0);
  const dim3 grid(a.batch * a.n_q_heads);
  const size_t lds = (size_t)max_n * sizeof(float);
  if (a.head_dim > 128)
    return pre ? launch1(reduce_kernel<true, true>, grid, dim3(64), lds, l, a)
               : launch1(reduce_kernel<true, false>, grid, dim3(64), lds, l, a);
  return pre ? launch1(reduce_kernel<false, true>, grid, dim3(64), lds, l, a)
             : launch1(reduce_kernel<false, false>, grid, dim3(64), lds, l, a);
}

hipError_t launch_table_apply(int32_t* table, int32_t stride, int32_t batch, const int32_t* upd,
                              int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_apply_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, stride,
                     batch, upd, n);
  return hipGetLastError();
}

}  // namespace pkv
