// Paged attention for several queries per sequence (a chunk of new tokens,
// as in chunked prefill), matrix-core version for bf16 and int8 pages.
//
// What it computes: sequence b's T_b = cu_q[b+1] - cu_q[b] query rows stand
// for its last T_b tokens (the rows a chunked page write just stored, as in
// AstrAI cache.py PagedCache.write with seq_len > 1), row i at position
// pos = lens[b] - T_b + i.  Each query head attends with its KV head to the
// tokens t <= pos, read in place through the block table: the valid-slot
// rule of metrale_storage high_speed_swap/impl_more.rs (a query at q_pos
// sees the first q_pos % page_size + 1 slots of its own block), which is the
// decode rule of tiny-llm paged_kv.py when T_b = 1.  A position below 0 sees
// nothing and gives zeros.
//
// How, on gfx950.  The 16 columns of the matrix-core tiles (mfma_step.h)
// are (query position, head) pairs of one KV head's group: n_pos = 16 / G
// consecutive positions times the G heads, so every K/V byte a wave loads
// serves all of them; each column keeps its own causal bound, its own
// running maximum and sum.  One wave owns one (sequence, KV head, group of
// n_pos positions) and walks the tokens up to its last position in 32-token
// steps, loads one step ahead (two register sets, peeled tail, as the decode
// kernel), and writes normalised outputs; there is no split of the token
// range, the parallelism comes from the queries.
//
// Launch order is XCD-aware: workgroups are handed to the 8 XCDs in turn, so
// block x runs on XCD x % 8; the items of one (sequence, KV head) are given
// consecutive blocks of one XCD, where they run together and share that
// XCD's L2 copy of the sequence's pages.
#include <algorithm>

#include "mfma_step.h"

namespace pkv {
namespace {

constexpr int kXcds = 8;

template <int FMT, int D, int BS>
__global__ __launch_bounds__(64, 2) void attend_multi_kernel(MultiArgs a) {
  using S = Step<FMT, D>;
  constexpr int NC = S::NC, ND = S::ND;
  constexpr int ESZ = FMT == PKV_FMT_BF16 ? 2 : 1;
  const int lane = threadIdx.x;
  const int n = lane & 15;  // column (B/C operands)
  const int j = lane >> 4;  // k group (A/B operands), row quad (C operand)
  const int G = a.group;
  const int P = a.n_pos;
  const int bs = BS ? BS : a.page_size;

  // ---- the item: (sequence, KV head) pair and group of positions
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int pair = (k / a.n_qgroups) * kXcds + xcd;
  const int qg = k % a.n_qgroups;
  if (pair >= a.batch * a.n_kv_heads) return;
  const int b = pair / a.n_kv_heads;
  const int g = pair - b * a.n_kv_heads;
  const bool reporter = qg == 0 && g == 0 && lane == 0;
  int q0 = a.cu_q[b];
  int T = a.cu_q[b + 1] - q0;
  if (q0 < 0 || T < 0 || q0 + T > a.total_q) {
    if (reporter) report(a.status, PKV_DEV_QROWS);
    return;  // malformed rows: none is read or written
  }
  const int len = clamp_len(a.lens[b], a.max_len, reporter ? a.status : nullptr, PKV_DEV_LEN);
  if (reporter && (T > len || T > a.max_q)) report(a.status, PKV_DEV_QROWS);
  const int p0 = qg * P;
  if (p0 >= T) return;

  // ---- this lane's column: position p0 + p of the chunk, head g * G + h
  const int p = n / G;
  const int h = n - p * G;
  const bool col = n < P * G && p0 + p < T;
  const int pos = len - T + p0 + p;  // below 0: sees nothing
  const int last = min(p0 + P, T) - 1;
  const int t_end = min(max(len - T + last + 1, 0), len);  // tokens the item reads

  bf16x8 qf[NC];
  const int64_t qrow = col ? (int64_t)(q0 + p0 + p) * a.n_q_heads + (int64_t)g * G + h : 0;
  load_q<FMT, D>(qf, static_cast<const uint16_t*>(a.q) + qrow * D, col && pos >= 0, j);

  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const PageSrc src{static_cast<const char*>(a.k_pages), static_cast<const char*>(a.v_pages),
                    a.k_scales, a.v_scales, a.layer_page0, slab_bytes, a.n_kv_heads, bs};
  const int32_t* trow = a.table + (int64_t)b * a.table_stride;
  const int pg_last = (t_end - 1) / bs;

  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float qs = a.qk_scale_log2;

  // windows of at most 64 logical pages: one table entry per lane
  const int tokens_per_window = 64 * bs;
  for (int w0 = 0; w0 < t_end; w0 += tokens_per_window) {
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

    auto load_step_at = [&](int ts, S& r) {
      const int lp = ts / bs;
      const int page_a = ts < w_end ? __builtin_amdgcn_readlane(vpage, lp - pg0) : -1;
      int page_b = page_a;
      if (BS == 16) page_b = ts + 16 < w_end ? __builtin_amdgcn_readlane(vpage, lp + 1 - pg0) : -1;
      load_step<FMT, D, BS>(r, src, page_a, page_b, ts - lp * bs, g, lane);
    };

    auto compute_step = [&](int ts, S& r) {
      f32x4 sacc[2];
      step_scores<FMT, D>(r, qf, sacc);
      const bool lane_live = BS == 16 && j >= 2 ? r.live_b : r.live_a;
      float ksc[8], vsc[8];
      if constexpr (FMT == PKV_FMT_INT8) step_scales<FMT, D>(r, j, ksc, vsc);
      float sv[8];
      bool readable[8], ok[8];  // token 8j + x: stored on a valid page / seen by the column
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int t = ts + 8 * j + x;
        readable[x] = lane_live && t < w_end;
        ok[x] = readable[x] && t <= pos;
        float y = sacc[x >> 2][x & 3] * qs;
        if (FMT == PKV_FMT_INT8) y *= ksc[x];
        sv[x] = ok[x] ? y : -INFINITY;
        mx = fmaxf(mx, sv[x]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float pr = ok[x] ? __builtin_amdgcn_exp2f(sv[x] - m_use) : 0.f;
        psum += pr;
        float pw = pr;
        if (FMT == PKV_FMT_INT8) pw = ok[x] ? pr * vsc[x] : 0.f;
        pb[x] = (__bf16)pw;
      }
      l = l * alpha + psum;
      m = m_new;
      // every stored slot is finite; only slots past the item's range (or
      // on a missing page) may hold NaN and are zeroed
      uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
      if (FMT == PKV_FMT_BF16 && (ts + 32 > w_end || !r.live_a || !r.live_b))
        v_keep_masks(readable, keep);
      step_pv<FMT, D>(r, pb, keep, alpha, o);
    };

    // ---- two register sets, loads one step ahead, prefetches unconditional
    // in the loop body and the last one or two steps peeled
    const int n_steps = (w_end - w0 + 31) / 32;
    auto T32 = [&](int i) { return w0 + 32 * i; };
    S r0, r1;
    load_step_at(T32(0), r0);
    int st = 0;
    for (; st + 2 < n_steps; st += 2) {
      load_step_at(T32(st + 1), r1);
      compute_step(T32(st), r0);
      load_step_at(T32(st + 2), r0);
      compute_step(T32(st + 1), r1);
    }
    if (st + 1 < n_steps) {
      load_step_at(T32(st + 1), r1);
      compute_step(T32(st), r0);
      compute_step(T32(st + 1), r1);
    } else {
      compute_step(T32(st), r0);
    }
  }

  // ---- results: O^T lane layout = dims 16 dt + 4j + i of column n
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (col) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      store_out4(a.out, 1, qrow * D + 16 * dt + 4 * j, o[dt] * inv);
  }
}

template <int FMT, int D, int BS>
hipError_t launch_bs(const MultiArgs& a, const Launch& l) {
  const int64_t pairs = (int64_t)a.batch * a.n_kv_heads;
  const int64_t grid = (pairs + kXcds - 1) / kXcds * kXcds * a.n_qgroups;
  return launch1(attend_multi_kernel<FMT, D, BS>, dim3((unsigned)grid), dim3(64), 0, l, a);
}

template <int FMT, int D>
hipError_t launch_d(const MultiArgs& a, const Launch& l) {
  if (a.page_size == 16) return launch_bs<FMT, D, 16>(a, l);
  if (a.page_size == 32) return launch_bs<FMT, D, 32>(a, l);
  return launch_bs<FMT, D, 0>(a, l);
}

template <int FMT>
hipError_t launch_fmt(const MultiArgs& a, const Launch& l) {
  return a.head_dim == 128 ? launch_d<FMT, 128>(a, l) : launch_d<FMT, 64>(a, l);
}

}  // namespace

int64_t multi_grid(int batch, int n_kv_heads, int n_qgroups) {
  const int64_t pairs = (int64_t)batch * n_kv_heads;
  return (pairs + kXcds - 1) / kXcds * kXcds * n_qgroups;
}

hipError_t launch_attend_multi(const MultiArgs& a, int fmt, const Launch& l) {
  if (!mfma_supported(fmt, 1, a.head_dim, a.page_size, a.group, 1, a.n_kv_heads))
    return hipErrorNotSupported;
  return fmt == PKV_FMT_BF16 ? launch_fmt<PKV_FMT_BF16>(a, l) : launch_fmt<PKV_FMT_INT8>(a, l);
}

}  // namespace pkv
