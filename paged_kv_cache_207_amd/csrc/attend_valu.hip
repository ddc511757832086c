// Paged decode attention, split-K partial pass, vector-ALU version.
//
// Reads K/V in place from the pages a sequence's block table lists (token t
// at page table[t / page_size], slot t % page_size: tiny-llm paged_kv.py,
// module docstring) instead of gathering them first.  Query head h uses KV
// head h / G.  Each workgroup covers one split of split_tokens tokens of one
// (sequence, KV head, group of up to 8 query heads) and produces, per query
// head, the running maximum m (log2 units), the running sum l of
// exp2(score - m) and the unnormalised sum o of exp2(score - m) * v over its
// tokens (an online softmax: the accumulate-then-finalize split of
// metrale_storage high_speed_swap/impl_more.rs attend_layer, whose tiles are
// combined here by a separate reduce kernel).  Tokens at or past lens[b] are
// never read.
//
// This kernel takes every page format (f32, bf16, int8 with per-token
// scales), any page size and head_dim <= 256.  Lanes hold tokens for the
// Q.K dot products (one token row per lane, query heads from LDS) and dims
// for the P.V products; it is the general path and the vector-ALU baseline
// of the matrix-core kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kHeads = 8;  // query heads per workgroup
constexpr int kTile = 64;  // tokens per tile (one per lane)
constexpr int kMaxD = 256;

template <int FMT>
__device__ __forceinline__ void load8(const void* base, int64_t e, float x[8]) {
  if (FMT == PKV_FMT_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + e);
    uint4 a = p[0], b = p[1];
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  } else if (FMT == PKV_FMT_BF16) {
    uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    uint2 a = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + e);
    uint32_t w[2] = {a.x, a.y};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] = (float)(int8_t)((w[i] >> (8 * j)) & 0xffu);
  }
}

template <int FMT>
__device__ __forceinline__ float load1(const void* base, int64_t e) {
  if (FMT == PKV_FMT_F32) return static_cast<const float*>(base)[e];
  if (FMT == PKV_FMT_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[e]);
  return (float)static_cast<const int8_t*>(base)[e];
}

template <int FMT>
__global__ __launch_bounds__(64) void attend_valu_kernel(AttendArgs a) {
  __shared__ float q_s[kHeads][kMaxD];
  __shared__ float p_s[kHeads][kTile];
  __shared__ int page_s[kTile];

  const int lane = threadIdx.x;
  const int D = a.head_dim, bs = a.page_size, G = a.group;
  constexpr int kEsz = FMT == PKV_FMT_F32 ? 4 : FMT == PKV_FMT_BF16 ? 2 : 1;
  const int nhc = (G + kHeads - 1) / kHeads;
  const int s = blockIdx.x;
  const int g = blockIdx.y / nhc, hc = blockIdx.y - g * nhc;
  const int b = blockIdx.z;
  const int h0 = g * G + hc * kHeads;
  const int gc = min(kHeads, G - hc * kHeads);

  const int len = clamp_len(a.lens[b], a.max_len, s == 0 && blockIdx.y == 0 ? a.status : nullptr,
                            PKV_DEV_LEN);
  const int t_begin = s * a.split_tokens;
  if (t_begin >= len) return;
  const int t_end = min(t_begin + a.split_tokens, len);

  for (int idx = lane; idx < gc * D; idx += 64) {
    const int hh = idx / D, d = idx - hh * D;
    const int64_t qi = ((int64_t)b * a.n_q_heads + h0 + hh) * D + d;
    const float qv = a.q_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qi])
                              : static_cast<const float*>(a.q)[qi];
    q_s[hh][d] = qv * a.qk_scale_log2;
  }
  __syncthreads();

  float m[kHeads], l[kHeads], o[kHeads][4];
#pragma unroll
  for (int hh = 0; hh < kHeads; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[hh][i] = 0.f;
  }
  const int64_t slab_elems = (int64_t)bs * D;

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    // ---- Q.K: one token per lane ----
    const int t = t0 + lane;
    int page = -1, slot = 0;
    if (t < t_end) {
      const int j = t / bs;
      page = a.table[(int64_t)b * a.table_stride + j];
      if (page < 0 || page >= a.n_pages) {
        report(a.status, PKV_DEV_READ_PAGE);
        page = -1;
      }
      slot = t - j * bs;
    }
    page_s[lane] = page;
    float acc[kHeads];
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh) acc[hh] = 0.f;
    const int64_t slab = (a.layer_page0 + (page < 0 ? 0 : page)) * a.n_kv_heads + g;
    if (page >= 0) {
      const int64_t kb = slab * slab_elems;
      for (int d0 = 0; d0 < D; d0 += 8) {
        float x[8];  // 8 elements: inside one 64-byte piece where rows are pieced
        load8<FMT>(a.k_pages, kb + k_byte(slot, d0 * kEsz, bs, D * kEsz) / kEsz, x);
#pragma unroll
        for (int hh = 0; hh < kHeads; ++hh) {
          if (hh < gc) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh] = fmaf(q_s[hh][d0 + e], x[e], acc[hh]);
          }
        }
      }
      if (FMT == PKV_FMT_INT8) {
        const float ks = a.k_scales[slab * bs + slot];
#pragma unroll
        for (int hh = 0; hh < kHeads; ++hh) acc[hh] *= ks;
      }
    }
    const float vscale = (FMT == PKV_FMT_INT8 && page >= 0) ? a.v_scales[slab * bs + slot] : 1.f;
    // ---- online softmax per query head ----
    float alpha[kHeads];
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh) {
      alpha[hh] = 1.f;
      if (hh < gc) {
        const float sc = page >= 0 ? acc[hh] : -INFINITY;
        const float m_new = fmaxf(m[hh], wave_max(sc));
        if (m_new != -INFINITY) alpha[hh] = exp2f(m[hh] - m_new);
        const float p = page >= 0 ? exp2f(sc - m_new) : 0.f;
        l[hh] = l[hh] * alpha[hh] + wave_sum(p);
        m[hh] = m_new;
        p_s[hh][lane] = p * vscale;
      }
    }
    __syncthreads();
    // ---- P.V: one dim per lane ----
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[hh][i] *= alpha[hh];
    const int ntile = min(kTile, t_end - t0);
    int tau = 0;
    if (bs % 8 == 0) {
      // 8 consecutive tokens share a page and sit in consecutive slots
      for (; tau + 8 <= ntile; tau += 8) {
        const int pg = page_s[tau];
        if (pg < 0) continue;
        const int tt = t0 + tau;
        const int64_t vb = ((a.layer_page0 + pg) * a.n_kv_heads + g) * slab_elems + (tt % bs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = lane + 64 * i;
          if (d < D) {
            float v[8];
            load8<FMT>(a.v_pages, vb + (int64_t)d * bs, v);
#pragma unroll
            for (int hh = 0; hh < kHeads; ++hh) {
              if (hh < gc) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][i] = fmaf(p_s[hh][tau + e], v[e], o[hh][i]);
              }
            }
          }
        }
      }
    }
    for (; tau < ntile; ++tau) {
      const int pg = page_s[tau];
      if (pg < 0) continue;
      const int tt = t0 + tau;
      const int64_t vb = ((a.layer_page0 + pg) * a.n_kv_heads + g) * slab_elems + (tt % bs);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) {
          const float v = load1<FMT>(a.v_pages, vb + (int64_t)d * bs);
#pragma unroll
          for (int hh = 0; hh < kHeads; ++hh)
            if (hh < gc) o[hh][i] = fmaf(p_s[hh][tau], v, o[hh][i]);
        }
      }
    }
    __syncthreads();
  }

  // ---- partial results ----
#pragma unroll
  for (int hh = 0; hh < kHeads; ++hh) {
    if (hh < gc) {
      const int64_t row = ((int64_t)b * a.n_q_heads + h0 + hh) * a.n_split + s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) a.ws_o[row * D + d] = o[hh][i];
      }
      if (lane == 0) {
        a.ws_ml[row * 2] = m[hh];
        a.ws_ml[row * 2 + 1] = l[hh];
      }
    }
  }
}

}  // namespace

hipError_t launch_attend_valu(const AttendArgs& a, int fmt, const Launch& l) {
  const int nhc = (a.group + kHeads - 1) / kHeads;
  dim3 grid(a.n_split, a.n_kv_heads * nhc, a.batch);
  if (fmt == PKV_FMT_F32) return launch1(attend_valu_kernel<PKV_FMT_F32>, grid, dim3(64), 0, l, a);
  if (fmt == PKV_FMT_BF16) return launch1(attend_valu_kernel<PKV_FMT_BF16>, grid, dim3(64), 0, l, a);
  return launch1(attend_valu_kernel<PKV_FMT_INT8>, grid, dim3(64), 0, l, a);
}

}  // namespace pkv
