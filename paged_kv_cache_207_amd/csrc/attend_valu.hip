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
// Two kernels, both for every page format (f32, bf16, int8 with per-token
// scales) and any number of query heads per KV head: the row-tiled kernel
// further down for pages of a multiple of 8 tokens and head dims of 32, 64,
// 96, 128 or 256, and this one for any page size and head_dim <= 256.  Here
// lanes hold tokens for the Q.K dot products (one token row per lane, query
// heads from LDS) and dims for the P.V products.
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


// ---- The row-tiled vector kernel: pages of a multiple of 8 tokens and head
// dims of 32, 64, 96, 128 or 256 (DQ = D / 16 dims per lane).
//
// Lane 16 j + n works on tokens 8 j .. 8 j + 7 of each 32-token step (the
// matrix-core kernel's tile).  For Q.K it holds dims n DQ .. n DQ + DQ - 1 of
// KH query heads in registers, so one K load instruction reads whole token
// rows, and the 16 lanes of a row add their partial dot products by DPP;
// every lane of row j then holds the scores of its 8 tokens.  The softmax
// runs on those registers (row maxima by lane swaps), and for P.V the lane
// accumulates dims n + 16 i (one V load instruction reads 16 consecutive dim
// rows of 8 tokens) over its row's tokens; the four rows' partial sums are
// added once, when the split ends.  Loads run one step ahead (two register
// sets); the last step's loads are issued again past the end instead of
// under a condition.
template <int FMT>
__device__ __forceinline__ constexpr int esz_of() {
  return FMT == PKV_FMT_F32 ? 4 : FMT == PKV_FMT_BF16 ? 2 : 1;
}

// N consecutive page elements at p (aligned to N elements), as raw 32-bit
// words (the element bytes, packed), and element e of such words as a float.
template <int FMT, int N>
struct Raw {
  static constexpr int BYTES = N * esz_of<FMT>();
  static constexpr int WORDS = (BYTES + 3) / 4;
  uint32_t w[WORDS];
};

template <int FMT, int N>
__device__ __forceinline__ void load_raw(const char* p, Raw<FMT, N>& r) {
  constexpr int BYTES = Raw<FMT, N>::BYTES;
  constexpr int CH = BYTES % 16 == 0 ? 16 : BYTES % 8 == 0 ? 8 : BYTES % 4 == 0 ? 4 : 2;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int c = 0; c < BYTES / CH; ++c) {
    if constexpr (CH == 16) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + c);
      r.w[4 * c] = v.x; r.w[4 * c + 1] = v.y; r.w[4 * c + 2] = v.z; r.w[4 * c + 3] = v.w;
    } else if constexpr (CH == 8) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + c);
      r.w[2 * c] = v.x; r.w[2 * c + 1] = v.y;
    } else if constexpr (CH == 4) {
      r.w[c] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + c);
    } else {
      const uint32_t h = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p) + c);
      if (c & 1) r.w[c >> 1] |= h << 16;
      else r.w[c >> 1] = h;
    }
  }
}

template <int FMT, int N>
__device__ __forceinline__ float elem(const Raw<FMT, N>& r, int e) {
  if constexpr (FMT == PKV_FMT_F32) return __uint_as_float(r.w[e]);
  else if constexpr (FMT == PKV_FMT_BF16)
    return __uint_as_float(e & 1 ? r.w[e >> 1] & 0xffff0000u : r.w[e >> 1] << 16);
  else return (float)(int8_t)((r.w[e >> 2] >> (8 * (e & 3))) & 0xffu);
}

// Sum over the 16 lanes of a row, in every lane of it (DPP: pairs, quads,
// half-rows, rows).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

template <int DQ>
constexpr int rows_heads() {  // query heads per wave: their Q and outputs take 2 x 32 registers
  return 32 / DQ < 1 ? 1 : 32 / DQ > 8 ? 8 : 32 / DQ;
}

template <int FMT, int DQ>
struct RowStep {
  Raw<FMT, DQ> k[8];  // tokens 8j + x, dims n DQ + i
  Raw<FMT, 8> v[DQ];  // dims n + 16 i, tokens 8j + x
  float ks[8], vs[8];  // int8: the 8 tokens' K and V scales
  bool live;           // the lane's 8 tokens sit on a valid page
};

template <int FMT, int DQ>
__global__ __launch_bounds__(64, 2) void attend_rows_kernel(AttendArgs a) {
  constexpr int D = 16 * DQ;
  constexpr int KH = rows_heads<DQ>();
  constexpr int ESZ = esz_of<FMT>();
  const int lane = threadIdx.x;
  const int n = lane & 15, j = lane >> 4;
  const int bs = a.page_size, G = a.group;
  const int nhc = (G + KH - 1) / KH;
  const int s = blockIdx.x;
  const int g = blockIdx.y / nhc, hc = blockIdx.y - g * nhc;
  const int b = blockIdx.z;
  const int h0 = g * G + hc * KH;
  const int gc = min(KH, G - hc * KH);

  const int len = clamp_len(a.lens[b], a.max_len, s == 0 && blockIdx.y == 0 ? a.status : nullptr,
                            PKV_DEV_LEN);
  const int t_begin = s * a.split_tokens;
  // one output element of head h0 + hh, dim d (direct writes)
  auto put_out = [&](int hh, int d, float v) {
    const int64_t oi = ((int64_t)b * a.n_q_heads + h0 + hh) * D + d;
    if (a.q_bf16) static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(v);
    else static_cast<float*>(a.out)[oi] = v;
  };
  if (t_begin >= len) {
    if (a.direct_out) {  // an empty sequence's output is zero
      for (int hh = 0; hh < gc; ++hh)
        for (int d = lane; d < D; d += 64) put_out(hh, d, 0.f);
    }
    return;
  }
  const int t_end = min(t_begin + a.split_tokens, len);

  // the query group's dims n DQ .. + DQ - 1, in log2 units (zeros past gc)
  float q[KH][DQ];
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
      float qv = 0.f;
      if (hh < gc) {
        const int64_t qi = ((int64_t)b * a.n_q_heads + h0 + hh) * D + n * DQ + i;
        qv = a.q_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qi])
                      : static_cast<const float*>(a.q)[qi];
      }
      q[hh][i] = qv * a.qk_scale_log2;
    }
  float o[KH][DQ], m[KH], l[KH];
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[hh][i] = 0.f;
  }
  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const char* kp = static_cast<const char*>(a.k_pages);
  const char* vp = static_cast<const char*>(a.v_pages);
  const int32_t* trow = a.table + (int64_t)b * a.table_stride;
  using S = RowStep<FMT, DQ>;

  // windows of at most 64 pages: one table entry per lane
  for (int w0 = t_begin; w0 < t_end; w0 = (w0 / bs + 64) * bs) {
    const int pg0 = w0 / bs;
    const int w_end = min((pg0 + 64) * bs, t_end);
    int vpage = -1;
    if (pg0 + lane <= (w_end - 1) / bs) {
      const int pg = trow[pg0 + lane];
      if (pg < 0 || pg >= a.n_pages) report(a.status, PKV_DEV_READ_PAGE);
      else vpage = pg;
    }
    auto load = [&](int ts, S& r) {
      const int t8 = ts + 8 * j;  // the lane's first token (page-aligned chunk of 8)
      const int pidx = min(t8 / bs - pg0, 63);
      const int page = __shfl(vpage, pidx, 64);
      r.live = t8 < w_end && page >= 0;
      const int64_t slab = (a.layer_page0 + (page >= 0 ? page : 0)) * a.n_kv_heads + g;
      const int slot = t8 - (t8 / bs) * bs;
      const char* kb = kp + slab * slab_bytes;
#pragma unroll
      for (int x = 0; x < 8; ++x)
        load_raw<FMT, DQ>(kb + k_byte(slot + x, n * DQ * ESZ, bs, D * ESZ), r.k[x]);
      const char* vb = vp + slab * slab_bytes;
#pragma unroll
      for (int i = 0; i < DQ; ++i)
        load_raw<FMT, 8>(vb + ((int64_t)(n + 16 * i) * bs + slot) * ESZ, r.v[i]);
      if constexpr (FMT == PKV_FMT_INT8) {
        const float4* kq = reinterpret_cast<const float4*>(a.k_scales + slab * bs + slot);
        const float4* vq = reinterpret_cast<const float4*>(a.v_scales + slab * bs + slot);
        const float4 k0 = kq[0], k1 = kq[1], v0 = vq[0], v1 = vq[1];
        r.ks[0] = k0.x; r.ks[1] = k0.y; r.ks[2] = k0.z; r.ks[3] = k0.w;
        r.ks[4] = k1.x; r.ks[5] = k1.y; r.ks[6] = k1.z; r.ks[7] = k1.w;
        r.vs[0] = v0.x; r.vs[1] = v0.y; r.vs[2] = v0.z; r.vs[3] = v0.w;
        r.vs[4] = v1.x; r.vs[5] = v1.y; r.vs[6] = v1.z; r.vs[7] = v1.w;
      }
    };
    auto compute = [&](int ts, const S& r) {
      const int t8 = ts + 8 * j;
      // scores: each page value converted once, used for every head
      float sc[8][KH];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) sc[x][hh] = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) {
          const float kv = elem(r.k[x], i);
#pragma unroll
          for (int hh = 0; hh < KH; ++hh) sc[x][hh] = fmaf(q[hh][i], kv, sc[x][hh]);
        }
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) sc[x][hh] = row16_sum(sc[x][hh]);
        // one token at a time: unscheduled, the compiler converts every page
        // value of the step at once and runs out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
      // a token past the window (or the length), or on a missing page, gets
      // -inf: weight 0, and its page values (maybe NaN) are dropped below
      bool ok[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        ok[x] = r.live && t8 + x < w_end;
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
          float v = sc[x][hh];
          if (FMT == PKV_FMT_INT8) v *= r.ks[x];
          sc[x][hh] = ok[x] ? v : -INFINITY;
        }
      }
      // online softmax: sc becomes the weights (int8: times the V scale)
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        float mx = sc[0][hh];
#pragma unroll
        for (int x = 1; x < 8; ++x) mx = fmaxf(mx, sc[x][hh]);
        const float m_new = fmaxf(m[hh], rows_max(mx));
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[hh] - m_use);
        m[hh] = m_new;
        float ps = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p = __builtin_amdgcn_exp2f(sc[x][hh] - m_use);
          ps += p;
          // int8: a dead token's scale may be any bits (NaN too), so its
          // weight is 0 outright rather than 0 times the scale
          sc[x][hh] = FMT == PKV_FMT_INT8 ? (ok[x] ? p * r.vs[x] : 0.f) : p;
        }
        l[hh] = fmaf(l[hh], alpha, ps);
#pragma unroll
        for (int i = 0; i < DQ; ++i) o[hh][i] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
      // P.V: each V value converted once (0 for a dead token: its weight is
      // 0, but the value may be NaN)
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float vv = ok[x] ? elem(r.v[i], x) : 0.f;
#pragma unroll
          for (int hh = 0; hh < KH; ++hh) o[hh][i] = fmaf(sc[x][hh], vv, o[hh][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int ts = w0; ts < w_end; ts += 32) {
      S r;
      load(ts, r);
      compute(ts, r);
    }
  }

  // ---- the four rows' partial sums, then the partial results ----
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) {
    l[hh] = rows_sum(l[hh]);
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[hh][i] = rows_sum(o[hh][i]);
  }
  if (a.direct_out) {  // the only split: normalise and write the outputs
#pragma unroll
    for (int hh = 0; hh < KH; ++hh) {
      if (hh < gc && j == 0) {
        const float inv = 1.f / l[hh];
#pragma unroll
        for (int i = 0; i < DQ; ++i) put_out(hh, n + 16 * i, o[hh][i] * inv);
      }
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) {
    if (hh < gc) {
      const int64_t row = ((int64_t)b * a.n_q_heads + h0 + hh) * a.n_split + s;
      if (j == 0) {
#pragma unroll
        for (int i = 0; i < DQ; ++i) a.ws_o[row * D + n + 16 * i] = o[hh][i];
      }
      if (lane == 0) {
        a.ws_ml[row * 2] = m[hh];
        a.ws_ml[row * 2 + 1] = l[hh];
      }
    }
  }
}

template <int FMT>
hipError_t launch_rows(const AttendArgs& a, const Launch& l) {
  auto go = [&](auto kernel, int kh) {
    const int nhc = (a.group + kh - 1) / kh;
    return launch1(kernel, dim3(a.n_split, a.n_kv_heads * nhc, a.batch), dim3(64), 0, l, a);
  };
  switch (a.head_dim) {
    case 32: return go(attend_rows_kernel<FMT, 2>, rows_heads<2>());
    case 64: return go(attend_rows_kernel<FMT, 4>, rows_heads<4>());
    case 96: return go(attend_rows_kernel<FMT, 6>, rows_heads<6>());
    case 128: return go(attend_rows_kernel<FMT, 8>, rows_heads<8>());
    default: return go(attend_rows_kernel<FMT, 16>, rows_heads<16>());
  }
}

bool rows_supported(const AttendArgs& a) { return valu_rows_supported(a.page_size, a.head_dim); }

}  // namespace

bool valu_rows_supported(int page_size, int head_dim) {
  const int d = head_dim;
  return page_size % 8 == 0 && (d == 32 || d == 64 || d == 96 || d == 128 || d == 256);
}

hipError_t launch_attend_valu(const AttendArgs& a, int fmt, const Launch& l) {
  if (rows_supported(a)) {
    if (fmt == PKV_FMT_F32) return launch_rows<PKV_FMT_F32>(a, l);
    if (fmt == PKV_FMT_BF16) return launch_rows<PKV_FMT_BF16>(a, l);
    return launch_rows<PKV_FMT_INT8>(a, l);
  }
  const int nhc = (a.group + kHeads - 1) / kHeads;
  dim3 grid(a.n_split, a.n_kv_heads * nhc, a.batch);
  if (fmt == PKV_FMT_F32) return launch1(attend_valu_kernel<PKV_FMT_F32>, grid, dim3(64), 0, l, a);
  if (fmt == PKV_FMT_BF16) return launch1(attend_valu_kernel<PKV_FMT_BF16>, grid, dim3(64), 0, l, a);
  return launch1(attend_valu_kernel<PKV_FMT_INT8>, grid, dim3(64), 0, l, a);
}

}  // namespace pkv
