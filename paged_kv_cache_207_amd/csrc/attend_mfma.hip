// Paged decode attention, split-K partial pass, matrix-core (MFMA) version
// for bf16 and int8 pages, head_dim 64 or 128, page sizes that are multiples
// of 16 and query groups of up to 16 heads.
//
// What it computes is the same as the vector-ALU kernel: per (sequence b, KV
// head g, split s) and per query head h of the group, the running maximum m
// (log2 units), the sum l of exp2(score - m) and the unnormalised sum of
// exp2(score - m) * v over the split's tokens, reading K/V in place through
// the block table (tiny-llm paged_kv.py docstring: token t at page
// table[t / page_size], slot t % page_size; query heads outnumber KV heads
// as in metrale_storage high_speed_swap/impl_more.rs attend_layer).
//
// How, on gfx950.  One wave owns one (b, g, s).  The query group is the N
// dimension of v_mfma_f32_16x16x32_bf16 (16 columns; columns >= G hold zeros),
// so every K/V element is loaded from HBM once, straight into registers, and
// used for all the group's heads without an LDS round trip.  The scores are
// computed transposed, S^T = K Q^T, whose accumulator layout (lane = head +
// 16 * token quad) is exactly the B-operand layout the P.V product needs, so
// the softmax weights never move between lanes.  P.V is computed as
// O^T = V^T P^T, with V read from the dim-major page slab (each lane loads 4
// consecutive slots of one dim).  The reduction order of the P.V k-slots is
// a fixed permutation of the 32 tokens of a step (tile 0 quad j, then tile 1
// quad j), applied identically to P and V.  A step covers 32 tokens (two
// 16-token tiles); the loads of step i+1 are issued before step i is
// computed.  int8 pages are converted to bf16 exactly (|code| <= 127); the
// per-token K scale multiplies the score and the V scale the weight.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int FMT, int D>
struct Step {
  static constexpr int NC = D / 32;  // 32-wide k chunks of the Q.K product
  static constexpr int ND = D / 16;  // 16-row dim tiles of the P.V product
  // bf16: 8 values per (tile, chunk); int8: 8 codes
  using KT = typename std::conditional<FMT == PKV_FMT_BF16, uint4, uint2>::type;
  // bf16: 4 values per (dim tile, tile); int8: 4 codes
  using VT = typename std::conditional<FMT == PKV_FMT_BF16, uint2, uint32_t>::type;
  // the same bytes as raw 32-bit vectors, for non-temporal loads
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  using NKT = typename std::conditional<sizeof(KT) == 16, u32x4, u32x2>::type;
  using NVT = typename std::conditional<sizeof(VT) == 8, u32x2, unsigned int>::type;
  KT k[2][NC];
  VT v[ND][2];
  f32x4 ks[2], vs[2];  // int8 only: scales of the lane's 4 tokens per tile
  bool live[2];        // tile has a valid page and at least one token
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Page reads are streamed once per call: non-temporal loads keep them from
// displacing other data in the caches (measured: +45% bandwidth on the
// 32k-token bf16 workload over plain loads).
template <typename T, typename R>
__device__ __forceinline__ T stream_load(const char* p) {
  return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const R*>(p)));
}

// 4 int8 codes -> 4 bf16 (exact: an integer of at most 7 bits plus sign)
__device__ __forceinline__ uint2 codes_to_bf16(uint32_t w) {
  float f0 = (float)(int8_t)(w & 0xffu), f1 = (float)(int8_t)((w >> 8) & 0xffu);
  float f2 = (float)(int8_t)((w >> 16) & 0xffu), f3 = (float)(int8_t)(w >> 24);
  uint2 r;
  r.x = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  r.y = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
  return r;
}

template <int FMT, int D, int BS>
__global__ __launch_bounds__(64) void attend_mfma_kernel(AttendArgs a) {
  using S = Step<FMT, D>;
  using KT = typename S::KT;
  using VT = typename S::VT;
  constexpr int NC = S::NC, ND = S::ND;
  constexpr int ESZ = FMT == PKV_FMT_BF16 ? 2 : 1;
  const int lane = threadIdx.x;
  const int n = lane & 15;  // head column (B/C operands), row (A operands)
  const int j = lane >> 4;  // k group (A/B operands), row quad (C operand)
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int bs = BS ? BS : a.page_size;

  const int len = clamp_len(a.lens[b], a.max_len, sp == 0 && g == 0 ? a.status : nullptr,
                            PKV_DEV_LEN);
  const int t_begin = sp * a.split_tokens;
  if (t_begin >= len) return;
  const int t_end = min(t_begin + a.split_tokens, len);

  // ---- query group as the B operand of S^T = K Q^T (zeros past the group) ----
  bf16x8 qf[NC];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        ((int64_t)b * a.n_q_heads + (int64_t)g * G + n) * D + 8 * j;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 x = {0, 0, 0, 0};
      if (n < G) x = *reinterpret_cast<const uint4*>(q + 32 * c);
      qf[c] = as_bf16x8(x);
    }
  }

  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const char* kp = static_cast<const char*>(a.k_pages);
  const char* vp = static_cast<const char*>(a.v_pages);
  const int32_t* trow = a.table + (int64_t)b * a.table_stride;
  const int pg_last = (t_end - 1) / bs;

  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float qs = a.qk_scale_log2;

  // The split is walked in windows of at most 64 logical pages: one table
  // entry per lane, picked out with a lane read (uniform) per tile.
  const int tokens_per_window = 64 * bs;
  for (int w0 = t_begin; w0 < t_end; w0 += tokens_per_window) {
    const int w_end = min(w0 + tokens_per_window, t_end);
    const int pg0 = w0 / bs;
    int vpage = -1;
    {
      const int lp = pg0 + lane;
      if (lp <= pg_last) {
        const int pg = trow[lp];
        if (pg < 0 || pg >= a.n_pages) report(a.status, PKV_DEV_READ_PAGE);
        else vpage = pg;
      }
    }

    // Loads are unconditional: a tile with no page (past the length or a bad
    // entry) reads page 0 of the array instead and is masked afterwards, so
    // the compiler can keep the next step's loads in flight.
    auto load_step = [&](int ts, S& r) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int tb = ts + 16 * tau;
        const int lp = tb / bs;
        const int page = tb < w_end ? __builtin_amdgcn_readlane(vpage, lp - pg0) : -1;
        r.live[tau] = page >= 0;
        const int slot0 = tb - lp * bs;
        const int64_t slab = (a.layer_page0 + (page >= 0 ? page : 0)) * a.n_kv_heads + g;
        const char* kslab = kp + slab * slab_bytes;  // uniform
        const char* vslab = vp + slab * slab_bytes;
        const int koff = ((slot0 + n) * D + 8 * j) * ESZ;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          r.k[tau][c] = stream_load<KT, typename S::NKT>(kslab + koff + 32 * c * ESZ);
        const int voff = (n * bs + slot0 + 4 * j) * ESZ;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
          r.v[dt][tau] = stream_load<VT, typename S::NVT>(vslab + voff + 16 * dt * bs * ESZ);
        if (FMT == PKV_FMT_INT8) {
          const float* kss = a.k_scales + slab * bs;
          const float* vss = a.v_scales + slab * bs;
          r.ks[tau] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kss + slot0 + 4 * j));
          r.vs[tau] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vss + slot0 + 4 * j));
        }
      }
    };

    auto compute_step = [&](int ts, S& r) {
      // S^T tiles: rows = tokens 16*tau + 4j + i, columns = heads
      f32x4 sacc[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bf16x8 ka;
          if constexpr (FMT == PKV_FMT_BF16) {
            ka = as_bf16x8(r.k[tau][c]);
          } else {
            const uint2 lo = codes_to_bf16(r.k[tau][c].x), hi = codes_to_bf16(r.k[tau][c].y);
            ka = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
          }
          sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[c], sacc[tau], 0, 0, 0);
        }
      }
      float sv[8];
      bool ok[8];
      float mx = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = ts + 16 * tau + 4 * j + i;
          ok[4 * tau + i] = r.live[tau] && t < w_end;
          float x = sacc[tau][i] * qs;
          if (FMT == PKV_FMT_INT8) x *= r.ks[tau][i];
          sv[4 * tau + i] = ok[4 * tau + i] ? x : -INFINITY;
          mx = fmaxf(mx, sv[4 * tau + i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = ok[i] ? __builtin_amdgcn_exp2f(sv[i] - m_use) : 0.f;
        psum += p;
        float pw = p;
        if (FMT == PKV_FMT_INT8) pw = ok[i] ? p * r.vs[i >> 2][i & 3] : 0.f;
        pb[i] = (__bf16)pw;
      }
      l = l * alpha + psum;
      m = m_new;
      // V^T A operands.  Where a slot of the step is dead (past the length or
      // on a missing page) zero its bf16 value: it may hold NaN, and 0 * NaN
      // would reach the sum.  int8 codes are finite and carry weight 0 there.
      const bool mask_v = FMT == PKV_FMT_BF16 && (ts + 32 > w_end || !r.live[0] || !r.live[1]);
      uint32_t keep[2][2] = {{~0u, ~0u}, {~0u, ~0u}};
      if (mask_v) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int w = 0; w < 2; ++w)
            keep[tau][w] = (ok[4 * tau + 2 * w] ? 0x0000ffffu : 0u) |
                           (ok[4 * tau + 2 * w + 1] ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        o[dt] *= alpha;
        uint4 va;
        if constexpr (FMT == PKV_FMT_BF16) {
          va = uint4{r.v[dt][0].x & keep[0][0], r.v[dt][0].y & keep[0][1],
                     r.v[dt][1].x & keep[1][0], r.v[dt][1].y & keep[1][1]};
        } else {
          const uint2 lo = codes_to_bf16(r.v[dt][0]), hi = codes_to_bf16(r.v[dt][1]);
          va = uint4{lo.x, lo.y, hi.x, hi.y};
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, o[dt], 0, 0, 0);
      }
    };

    // ---- two register sets, loads one step ahead ----
    const int n_steps = (w_end - w0 + 31) / 32;
    S r0, r1;
    load_step(w0, r0);
    for (int st = 0; st < n_steps; st += 2) {
      const int ts = w0 + 32 * st;
      if (st + 1 < n_steps) load_step(ts + 32, r1);
      compute_step(ts, r0);
      if (st + 1 < n_steps) {
        if (st + 2 < n_steps) load_step(ts + 64, r0);
        compute_step(ts + 32, r1);
      }
    }
  }

  // ---- partial results: O^T lane layout = dims 16*dt + 4j + i of head n ----
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n < G) {
    const int64_t row = ((int64_t)b * a.n_q_heads + (int64_t)g * G + n) * a.n_split + sp;
    float* wo = a.ws_o + row * D + 4 * j;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(wo + 16 * dt) = o[dt];
    if (j == 0) {
      a.ws_ml[row * 2] = m;
      a.ws_ml[row * 2 + 1] = l;
    }
  }
}

template <int FMT, int D>
hipError_t launch_d(const AttendArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.n_kv_heads, a.batch);
  if (a.page_size == 16)
    hipLaunchKernelGGL((attend_mfma_kernel<FMT, D, 16>), grid, dim3(64), 0, s, a);
  else if (a.page_size == 32)
    hipLaunchKernelGGL((attend_mfma_kernel<FMT, D, 32>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((attend_mfma_kernel<FMT, D, 0>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const AttendArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_d<FMT, 128>(a, s) : launch_d<FMT, 64>(a, s);
}

}  // namespace

bool mfma_supported(int fmt, int q_bf16, int head_dim, int page_size, int group) {
  return (fmt == PKV_FMT_BF16 || fmt == PKV_FMT_INT8) && q_bf16 &&
         (head_dim == 64 || head_dim == 128) && page_size % 16 == 0 && group >= 1 && group <= 16;
}

hipError_t launch_attend_mfma(const AttendArgs& a, int fmt, hipStream_t s) {
  if (!mfma_supported(fmt, a.q_bf16, a.head_dim, a.page_size, a.group))
    return hipErrorNotSupported;
  return fmt == PKV_FMT_BF16 ? launch_fmt<PKV_FMT_BF16>(a, s) : launch_fmt<PKV_FMT_INT8>(a, s);
}

}  // namespace pkv
