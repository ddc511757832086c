// The shared-prefix pass: attention of every sequence's decode queries over
// the tokens its block table shares with all the others, reading those
// pages once for many sequences instead of once per sequence.
//
// Pages shared by reference count (libmir-metal src/engine/kv/paged/mod.rs,
// PagedStore::snapshot; tiny-llm paged_kv.py: one block serves every reader
// of it) hold the same K/V for every sequence that lists them, so the scores
// of all those sequences' queries against one shared token can come from one
// read of it.  Here the columns of the matrix-core tiles are (sequence, query
// head) pairs of one KV head: a wave holds one or two tiles of 16 columns
// (the G heads of consecutive sequences), walks one chunk of the shared
// tokens in 32-token steps (the step machinery of mfma_step.h, with cached
// loads, since every such wave reads the same pages), and leaves per column
// the running maximum m (log2 units), the sum l and the unnormalised weighted
// V sum of that chunk: the tile accumulation of metrale_storage
// high_speed_swap/impl_more.rs attend_layer, finalised by the combine kernel
// together with the pieces of the private suffix.
//
// Column (b, h) sees the shared tokens t < min(lens[b], prefix_len), the
// decode length rule of tiny-llm paged_kv.py begin_step.  Each wave also
// checks that its sequences' table rows list the shared pages it read, and
// reports PKV_DEV_PREFIX otherwise.
//
// These waves are extra workgroups of the split pass's launch (see
// attend_mfma.hip): they run beside its memory-bound waves on the same
// SIMDs, so their vector work hides under the streaming of the private
// suffixes instead of taking a launch of its own.
#pragma once

#include "mfma_step.h"

namespace pkv {

// One step of cached (not streamed) loads: the same pages serve every prefix wave.
template <int FMT, int D, int BS>
__device__ __forceinline__ void load_step_cached(Step<FMT, D>& r, const PageSrc& s, int page_a,
                                                 int page_b, int slot0, int g, int lane) {
  using S = Step<FMT, D>;
  constexpr int ESZ = FMT == PKV_FMT_BF16 ? 2 : 1;
  const int n = lane & 15, j = lane >> 4;
  const int bs = BS ? BS : s.bs;
  r.live_a = page_a >= 0;
  r.live_b = page_b >= 0;
  const int64_t slab_a = (s.layer_page0 + (page_a >= 0 ? page_a : 0)) * s.n_kv_heads + g;
  const int64_t slab_b = (s.layer_page0 + (page_b >= 0 ? page_b : 0)) * s.n_kv_heads + g;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int tok = 8 * (n >> 2) + 4 * tau + (n & 3);
    const bool on_b = BS == 16 && tok >= 16;
    const char* kb = s.k + (on_b ? slab_b : slab_a) * s.slab_bytes;
    const int row = BS == 16 ? (tok & 15) : slot0 + tok;
#pragma unroll
    for (int c = 0; c < S::NK; ++c)
      r.k[tau][c] = *reinterpret_cast<const typename S::KT*>(
          kb + k_byte(row, kdim_of<FMT>(S::KPL * c, j) * ESZ, bs, D * ESZ));
  }
  const bool v_on_b = BS == 16 && j >= 2;
  const char* vb = s.v + (v_on_b ? slab_b : slab_a) * s.slab_bytes;
  const int col = BS == 16 ? 8 * (j & 1) : slot0 + 8 * j;
  const int voff = (n * bs + col) * ESZ;
#pragma unroll
  for (int dt = 0; dt < S::ND; ++dt)
    r.v[dt] = *reinterpret_cast<const typename S::VT*>(vb + voff + 16 * dt * bs * ESZ);
  if (FMT == PKV_FMT_INT8) {
    const int x = 8 * j + (n & 7);
    const bool s_on_b = BS == 16 && x >= 16;
    const int slot = BS == 16 ? (x & 15) : slot0 + x;
    const float* sb = n < 8 ? s.ks : s.vs;
    r.sc = sb[(s_on_b ? slab_b : slab_a) * bs + slot];
  }
}

// Online-softmax state of one 16-column tile: the reference maximum m (log2
// units), the sums ls (taken by the matrix cores: every entry of a lane holds
// its column's whole sum) and the unnormalised outputs o.
template <int ND>
struct Tile {
  float m;
  f32x4 ls;
  f32x4 o[ND];
};

// 16-column tiles per prefix wave: two at head_dim 64 (every K/V operand
// serves both), one at 128 (within the registers of the decode path).
template <int D>
__host__ __device__ constexpr int prefix_tiles() {
  return D == 64 ? 2 : 1;
}

// Prefix work items: (column block of 16 TT columns, KV head, chunk), column
// blocks fastest.
template <int TT>
__host__ __device__ inline int64_t prefix_col_blocks(int batch, int group) {
  return ((int64_t)batch * group + 16 * TT - 1) / (16 * TT);
}

// One prefix work item, done by one wave: TT tiles of 16 columns (TT = 2
// shares every K/V operand between two tiles; TT = 1 keeps the registers of
// the head_dim 128 decode path).  RAW (a positive scale): scores stay in raw
// units (int8: times the K scale) until the exponential, whose one fma
// applies the scale, and the maximum is taken over raw scores and scaled
// once.
template <int FMT, int D, int BS, int TT, bool RAW>
__device__ __forceinline__ void prefix_wave(const AttendArgs& a, int wid) {
  using S = Step<FMT, D>;
  constexpr int NC = S::NC, ND = S::ND;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int G = a.group;
  const int nb = (int)prefix_col_blocks<TT>(a.batch, G);
  const int cb = wid % nb, rest = wid / nb;
  const int g = rest % a.n_kv_heads, chunk = rest / a.n_kv_heads;
  const int bs = BS ? BS : a.page_size;
  const int ncols = a.batch * G;
  const int c0 = cb * 16 * TT;
  const int P0 = a.prefix_len;

  // the two tiles' columns: (sequence, head in group) of column c0 + 16 t + n,
  // and how many shared tokens each may see
  int bcol[TT], hcol[TT], bound[TT];
  bf16x8 qf[TT][NC];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int c = c0 + 16 * t + n;
    const bool used = c < ncols;
    const int b = used ? c / G : 0;
    bcol[t] = b;
    hcol[t] = c - b * G;
    int len = used ? a.lens[b] : 0;
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);  // reported by the split pass
    bound[t] = used ? min(len, P0) : 0;
    load_q<FMT, D>(qf[t], static_cast<const uint16_t*>(a.q) +
                             ((int64_t)b * a.n_q_heads + (int64_t)g * G + hcol[t]) * D,
                   used, j);
  }
  const int t_begin = chunk * a.pchunk;
  const int t_end = min(t_begin + a.pchunk, P0);
  // steps past every column's bound are skipped; slots at or past the wave's
  // largest bound may never have been written (NaN), so their V is zeroed
  int bmax = bound[0];
#pragma unroll
  for (int t = 1; t < TT; ++t) bmax = max(bmax, bound[t]);
#pragma unroll
  for (int o1 = 1; o1 < 64; o1 <<= 1) bmax = max(bmax, __shfl_xor(bmax, o1, 64));
  bmax = __builtin_amdgcn_readfirstlane(bmax);
  const int t_stop = min(t_end, bmax);
  // per tile, the smallest bound of its used columns (uniform): a step that
  // ends by then is seen whole by every column of the tile; lim: this
  // lane's column sees tokens t < lim
  int bmin[TT], lim[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    int v = c0 + 16 * t + n < ncols ? bound[t] : 0x7fffffff;
#pragma unroll
    for (int o1 = 1; o1 < 64; o1 <<= 1) v = min(v, __shfl_xor(v, o1, 64));
    bmin[t] = __builtin_amdgcn_readfirstlane(v);
    lim[t] = min(bound[t], t_stop);
  }

  Tile<ND> st[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    st[t].m = -INFINITY;
    st[t].ls = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) st[t].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float qs = a.qk_scale_log2;
  const int64_t slab_bytes = (int64_t)bs * D * (FMT == PKV_FMT_BF16 ? 2 : 1);
  const PageSrc src{static_cast<const char*>(a.k_pages), static_cast<const char*>(a.v_pages),
                    a.k_scales, a.v_scales, a.layer_page0, slab_bytes, a.n_kv_heads, bs};

  // the chunk's page ids, one per lane (a chunk spans at most 64 pages), read
  // once: a step picks its pages with a lane read, so no step waits on a
  // table load
  const int pg0 = t_begin / bs;
  const int pg_end = (t_end + bs - 1) / bs;  // this chunk's pages: [pg0, pg_end)
  int vpage = -1;
  if (pg0 + lane < pg_end) {
    const int pg = a.prefix_pages[pg0 + lane];
    if (pg < 0 || pg >= a.n_pages) report(a.status, PKV_DEV_READ_PAGE);
    else vpage = pg;
  }
  auto load_at = [&](int ts, S& r) {
    const int lp = ts / bs;
    const int pa = __builtin_amdgcn_readlane(vpage, lp - pg0);
    int pb = pa;
    if (BS == 16) pb = ts + 16 < t_stop ? __builtin_amdgcn_readlane(vpage, lp + 1 - pg0) : -1;
    load_step_cached<FMT, D, BS>(r, src, pa, pb, ts - lp * bs, g, lane);
  };
  const bf16x8 ones = as_bf16x8(uint4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  auto compute = [&](int ts, S& r) {
    // uniform: every slot of the step is on a page and inside the range some
    // column of the wave sees (the common case: nothing to mask)
    const bool whole = ts + 32 <= t_stop && r.live_a && r.live_b;
    const bool lane_live = BS == 16 && j >= 2 ? r.live_b : r.live_a;
    float ksc[8], vsc[8];
    if constexpr (FMT == PKV_FMT_INT8) step_scales<FMT, D>(r, ksc, vsc);
    if (!whole) {
      // V slots no column may see are zeroed (they may hold NaN); int8:
      // their V scales, so that a zero weight stays zero
      bool vok[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) vok[x] = lane_live && ts + 8 * j + x < t_stop;
      if constexpr (FMT == PKV_FMT_BF16) {
        uint32_t keep[4];
        v_keep_masks(vok, keep);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          r.v[dt].x &= keep[0];
          r.v[dt].y &= keep[1];
          r.v[dt].z &= keep[2];
          r.v[dt].w &= keep[3];
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) vsc[x] = vok[x] ? vsc[x] : 0.f;
      }
    }
    // the P.V operand of every tile: V^T rows (int8 codes converted once)
    bf16x8 va[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      if constexpr (FMT == PKV_FMT_BF16) {
        va[dt] = as_bf16x8(r.v[dt]);
      } else {
        const uint2 lo = codes_to_bf16(r.v[dt].x), hi = codes_to_bf16(r.v[dt].y);
        va[dt] = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      f32x4 sacc[2];
      step_scores<FMT, D>(r, qf[t], sacc);
      // scores (RAW: unscaled; int8: times the K scale); a token the column
      // may not see gets -inf, and so a weight of exactly 0 below
      // (exp2(-inf) = 0: no select on the weights)
      float sv[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        sv[x] = RAW ? sacc[x >> 2][x & 3] : sacc[x >> 2][x & 3] * qs;
        if (FMT == PKV_FMT_INT8) sv[x] *= ksc[x];
      }
      if (!(whole && ts + 32 <= bmin[t])) {  // uniform: some column sees part of the step
#pragma unroll
        for (int x = 0; x < 8; ++x)
          sv[x] = lane_live && ts + 8 * j + x < lim[t] ? sv[x] : -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int x = 1; x < 8; ++x) mx = fmax_fast(mx, sv[x]);
      mx = rows_max(mx);
      if (RAW) mx *= qs;  // a positive scale keeps the maximum where it is
      const float m_new = fmax_fast(st[t].m, mx);
      // the reference maximum moves only when some column's maximum passes
      // it by more than kRescaleSlack (-inf + slack: any finite maximum), so
      // weights stay below 2^kRescaleSlack and the outputs and sums are
      // rescaled on few steps; the combine weighs each partial by its own
      // reference
      const bool grow = __builtin_amdgcn_ballot_w64(m_new > st[t].m + kRescaleSlack) != 0;
      const float m_ref = grow ? m_new : st[t].m;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float p[8], pw[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        p[x] = __builtin_amdgcn_exp2f(RAW ? __builtin_fmaf(sv[x], qs, -m_use) : sv[x] - m_use);
        pw[x] = FMT == PKV_FMT_INT8 ? p[x] * vsc[x] : p[x];
      }
      const bf16x8 pb = as_bf16x8(uint4{pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                        pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7])});
      // the sums' operand: the weights themselves (int8: before the V scale)
      const bf16x8 ps = FMT == PKV_FMT_INT8
                            ? as_bf16x8(uint4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                              pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])})
                            : pb;
      if (grow) {
        const float alpha = __builtin_amdgcn_exp2f(st[t].m - m_use);
        st[t].ls *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) st[t].o[dt] *= alpha;
        st[t].m = m_ref;
      }
      st[t].ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ps, st[t].ls, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        st[t].o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pb, st[t].o[dt], 0, 0, 0);
    }
  };

  // NS register sets, loads NS steps ahead (all of a chunk's steps are in
  // flight from the start when NS covers them).  Every wave of the launch
  // asks the caches for the same shared lines at about the same time, so a
  // step costs a full memory round trip: depth, not bandwidth, sets the pace
  // here.  Loads are unconditional (a step past the chunk reloads the last
  // one and is not computed), so no load sits under a condition and the
  // compiler counts outstanding loads exactly.
  // The waves of one (KV head, chunk) read the same lines; each starts at a
  // different step of the chunk (the softmax merge does not depend on the
  // order), so at any moment their requests spread over the chunk's pages.
  // Two register sets, loads one step ahead; the last steps are peeled so no
  // load sits under a condition.
  const int n_steps = t_stop > t_begin ? (t_stop - t_begin + 31) / 32 : 0;
  if (n_steps > 0) {
    const int rot = cb % n_steps;
    auto T = [&](int i) {
      int k = i + rot;
      k -= k >= n_steps ? n_steps : 0;
      return t_begin + 32 * k;
    };
    S r0, r1;
    load_at(T(0), r0);
    int s = 0;
    for (; s + 2 < n_steps; s += 2) {
      load_at(T(s + 1), r1);
      compute(T(s), r0);
      load_at(T(s + 2), r0);
      compute(T(s + 1), r1);
    }
    if (s + 1 < n_steps) {
      load_at(T(s + 1), r1);
      compute(T(s), r0);
      compute(T(s + 1), r1);
    } else {
      compute(T(s), r0);
    }
  }

  // ---- partials of this chunk: O^T lane layout = dims 16 dt + 4 j + i of column n ----
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float l = st[t].ls[0];  // the column's whole sum, in every lane of the column
    if (c0 + 16 * t + n < ncols) {
      const int64_t row =
          (((int64_t)bcol[t] * a.n_q_heads + (int64_t)g * G + hcol[t]) * a.n_pchunks + chunk);
      float* wo = a.ws_pre_o + row * D + 4 * j;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(wo + 16 * dt) = st[t].o[dt];
      if (j == 0) *reinterpret_cast<float2*>(a.ws_pre_ml + row * 2) = float2{st[t].m, l};
    }
  }

  // ---- the promise behind this pass: every sequence read here lists this
  // chunk's shared pages in its own table row, for the tokens it sees.  One
  // (sequence, page) pair per lane, the table entry, the length and the
  // shared id loaded together ----
  const int b_first = c0 / G;
  const int b_last = min(c0 + 16 * TT - 1, ncols - 1) / G;
  const int per = pg_end - pg0;  // at most 64 pages
  const int pairs = (b_last - b_first + 1) * per;
  bool bad = false;
  for (int p0 = 0; p0 < pairs; p0 += 256) {
    int ent[4], len4[4], want[4], lpv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = min(p0 + 64 * u + lane, pairs - 1);  // in bounds; repeats are harmless
      const int bb = b_first + p / per, lp = pg0 + p % per;
      lpv[u] = lp;
      ent[u] = a.table_full[(int64_t)bb * a.table_stride + lp];
      len4[u] = a.lens[bb];
      want[u] = __shfl(vpage, lp - pg0, 64);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int L = len4[u] < 0 ? 0 : (len4[u] > a.max_len ? a.max_len : len4[u]);
      bad |= (int64_t)lpv[u] * bs < min(L, P0) && ent[u] != want[u];
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) report(a.status, PKV_DEV_PREFIX);
}

}  // namespace pkv
