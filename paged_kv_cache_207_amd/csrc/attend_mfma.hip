// Paged decode attention, split-K partial pass, matrix-core (MFMA) version
// for bf16 and int8 pages, head_dim 64 or 128, page size 16 or a multiple of
// 32, and query groups of up to 16 heads.
//
// What it computes is the same as the vector-ALU kernel: per (sequence b, KV
// head g, split s) and per query head h of the group, the running maximum m
// (log2 units), the sum l of exp2(score - m) and the unnormalised sum of
// exp2(score - m) * v over the split's tokens, reading K/V in place through
// the block table (tiny-llm paged_kv.py docstring: token t at page
// table[t / page_size], slot t % page_size; query heads outnumber KV heads
// as in metrale_storage high_speed_swap/impl_more.rs attend_layer).
//
// How, on gfx950 (the step machinery is in mfma_step.h).  One wave works on
// one piece (b, g, token range) at a time; the query group is the N
// dimension of the matrix-core tiles (16 columns; columns >= G hold zeros).  The loads of step i+1 are issued
// before step i is computed.  int8 pages are converted to bf16 exactly
// (|code| <= 127); the per-token K scale multiplies the score and the V
// scale the weight.
//
// Work distribution: a persistent grid of single-wave workgroups, under one
// of two schedules built in LDS from the lengths.
//   Fixed splits: a work list of (split, KV head) items, full splits first.
//   A sequence that fits in one split gets its output written directly.  For
//   longer sequences either the combine kernel merges the partials
//   afterwards (the default), or, when the caller asks for it
//   (fuse_combine), the workgroup that finishes a (sequence, KV head)'s last
//   split merges them in the same launch.
//   Balanced (BAL): each wave takes an equal share of the flat space of all
//   (sequence, KV head) units' 32-token steps, every unit charged a set-up
//   cost on top, and walks the pieces of units its share covers.  A unit
//   covered by one piece gets its output written directly; otherwise its
//   first piece records where the partials sit and the combine kernel merges
//   them.  Waves then finish together however uneven the lengths are.  When
//   every non-empty sequence has the same length the BAL kernel takes the
//   fixed splits instead (they are balanced already).
#include <algorithm>
#include <climits>

#include "mfma_step.h"
#include "prefix_wave.h"

namespace pkv {
namespace {

// Balanced schedule: at least this many steps per wave (fewer waves for
// small calls, so their partials stay few).
constexpr int kMinWaveSteps = 8;

// Most waves per workgroup.  Each wave takes its own work; the workgroup's
// first wave builds the schedule in LDS for all of them.  The dispatcher
// hands workgroups to the XCDs in turn, and with one-wave workgroups the
// last XCDs received theirs 2.5-4 us after the first (per-wave start stamps
// of a 1024-wave launch): several waves a workgroup shorten that stagger.
// A launch with fewer waves than four per compute unit takes narrower
// workgroups, so that its waves still spread over every compute unit.
constexpr int kGroupWaves = 4;


// Partials are exchanged between workgroups, which may sit on different XCDs
// with separate L2 caches.  Writers store them as agent-scope relaxed atomics
// (sc1 stores, written through to the coherence point) and wait for those
// stores to complete before counting their split in; the one workgroup that
// combines a (sequence, KV head) invalidates its caches once (an agent-scope
// acquire) and then reads the partials with ordinary vector loads.  No
// L2 write-back is needed: measured, a release/acquire pair per work item
// doubled the 32k-token split pass.
__device__ __forceinline__ void put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Combine the n split partials (m_s, l_s, o_s) of every query head of KV
// group g of sequence b: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// merged split by split with a running maximum.  One lane per (head, 4 dims);
// 16 splits' loads in flight per lane.
template <int D>
__device__ __forceinline__ void combine_group(const AttendArgs& a, int b, int g, int n, int lane) {
  constexpr int Q4 = D / 4;
  constexpr int U = 16;
  for (int idx = lane; idx < a.group * Q4; idx += 64) {
    const int hh = idx / Q4, d4 = idx - hh * Q4;
    const int64_t hrow = (int64_t)b * a.n_q_heads + (int64_t)g * a.group + hh;
    const float* ml = a.ws_ml + hrow * a.n_split * 2;
    const float* po = a.ws_o + hrow * a.n_split * D + 4 * d4;
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += U) {
      float2 x[U];
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = min(s0 + u, n - 1);  // in bounds; repeats are given weight 0 below
        x[u] = *reinterpret_cast<const float2*>(ml + 2 * s);
        v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)s * D);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u < n) {
          const float Mn = fmaxf(M, x[u].x);
          const float al = __builtin_amdgcn_exp2f(M - Mn), w = __builtin_amdgcn_exp2f(x[u].x - Mn);
          acc = acc * al + v[u] * w;
          L = L * al + x[u].y * w;
          M = Mn;
        }
      }
    }
    store_out4(a.out, a.q_bf16, hrow * D + 4 * d4, acc * (1.f / L));
  }
}

// The piece loop of the split pass under one schedule (SB: balanced), after
// the kernel has built the schedule's prefix sums and lengths in LDS.  Each
// schedule gets its own copy, so the fixed-split copy carries none of the
// balanced schedule's loop state.
template <int FMT, int D, int BS, bool SB>
__device__ __forceinline__ void run_pieces(const AttendArgs& a, const int32_t* fpre,
                                           const int32_t* qpre, const int32_t* lens, int vb) {
  using S = Step<FMT, D>;
  using KT = typename S::KT;
  constexpr int NC = S::NC, ND = S::ND;
  constexpr int ESZ = FMT == PKV_FMT_BF16 ? 2 : 1;
  constexpr int KPL = S::KPL;
  auto kdim = [](int c, int jj) { return kdim_of<FMT>(c, jj); };
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;  // head column (B/C operands), row (A operands)
  const int j = lane >> 4;  // k group (A/B operands), row quad (C operand)
  const int G = a.group;
  const int bs = BS ? BS : a.page_size;
  const int C = a.split_tokens;
  const int B = a.batch;
  const int n_full = fpre[B];
  const int n_items = (n_full + qpre[B]) * a.n_kv_heads;

  // sequences with no tokens have no work item: their output is zero (with a
  // shared prefix the combine writes every output)
  const int nblk = a.split_waves;  // split-pass waves; this one is wave vb
  for (int b = vb; b < (a.prefix_len > 0 ? 0 : B); b += nblk) {
    if (lens[b] != 0) continue;
    for (int i = lane; i < a.n_q_heads * D / 4; i += 64)
      store_out4(a.out, a.q_bf16, (int64_t)b * a.n_q_heads * D + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
  }

  // balanced schedule: this wave's slots [F, F1) of the T-slot flat space
  int64_t T = 0, F = 0, F1 = 0;
  int n_waves = 1;
  if constexpr (SB) {
    T = __builtin_amdgcn_readfirstlane(fpre[B]);
    const int64_t want = std::max<int64_t>(1, (T + kMinWaveSteps - 1) / kMinWaveSteps);
    n_waves = (int)std::min<int64_t>(nblk, want);
    if (vb < n_waves) {
      F = (int64_t)vb * T / n_waves;
      F1 = ((int64_t)vb + 1) * T / n_waves;
    }
  }
  int item = vb;

  for (;;) {
  // ---- the next piece: tokens [t_begin, t_end) of unit (b, g); `direct`
  // when it is the unit's only piece (normalised output written here), else
  // its partial goes to workspace rows row_base + n * row_step (n < G)
  int b, g, t_begin, t_end, sp = 0, n_splits_b = 1;
  bool direct, owns_new;
  int64_t row_base;
  int row_step;
  if constexpr (SB) {
    if (F >= F1) break;
    int lo = 0, hi = B - 1;  // the sequence owning slot F (never an empty one)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (fpre[mid] <= F) lo = mid;
      else hi = mid - 1;
    }
    b = __builtin_amdgcn_readfirstlane(lo);
    const int len_b = __builtin_amdgcn_readfirstlane(lens[b]);
    const int pre_b = __builtin_amdgcn_readfirstlane(fpre[b]);
    const int steps = (len_b + 31) >> 5;
    const int cu = steps + a.unit_cost;
    g = (int)((F - pre_b) / cu);
    const int64_t s_first = pre_b + (int64_t)g * cu + a.unit_cost;  // slot of step 0
    const int64_t u_end = s_first + steps;
    const int64_t p_lo = std::max(F, s_first), p_hi = std::min(F1, u_end);
    F = u_end;
    if (p_lo >= p_hi) continue;  // only set-up slots of this unit fall here
    t_begin = (int)(p_lo - s_first) * 32;
    t_end = std::min((int)(p_hi - s_first) * 32, len_b);
    direct = p_lo == s_first && p_hi == u_end && a.prefix_len == 0;
    owns_new = a.k_new != nullptr && p_hi == u_end;
    const int unit = b * a.n_kv_heads + g;
    const int slot = unit + vb;  // strictly increasing along the flat space
    row_base = (int64_t)slot * G;
    row_step = 1;
    if (p_lo == s_first && lane == 0) {
      // the unit's first piece records where its pieces' partials sit: the
      // waves from this one to the one holding the unit's last step (one
      // piece: the output is written here and the combine skips the unit)
      const int w_last = (int)((u_end * n_waves - 1) / T);
      *reinterpret_cast<int2*>(a.ws_desc + 2 * unit) = int2{slot, w_last - vb + 1};
    }
  } else {
    if (item >= n_items) break;
    const int pair = item / a.n_kv_heads;
    g = item - pair * a.n_kv_heads;
    item += nblk;
    // largest b whose prefix is <= the index: that sequence owns it
    const int32_t* pre = pair < n_full ? fpre : qpre;
    const int idx = pair < n_full ? pair : pair - n_full;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= idx) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    sp = pair < n_full ? idx - fpre[b] : fpre[b + 1] - fpre[b];
    n_splits_b = (lens[b] + C - 1) / C;
    t_begin = sp * C;
    t_end = min(t_begin + C, lens[b]);
    direct = n_splits_b == 1 && a.prefix_len == 0;
    // decode step: the sequence's new row sits at position len - 1, in the
    // last step of its last split (see substitute_new below)
    owns_new = a.k_new != nullptr && sp == n_splits_b - 1;
    row_base = ((int64_t)b * a.n_q_heads + (int64_t)g * G) * a.n_split + sp;
    row_step = a.n_split;
  }
  const int len = lens[b];

  // ---- query group as the B operand of S^T = K Q^T (zeros past the group) ----
  bf16x8 qf[NC];
  load_q<FMT, D>(qf, static_cast<const uint16_t*>(a.q) +
                         ((int64_t)b * a.n_q_heads + (int64_t)g * G + n) * D,
                 n < G, j);

  // the pages' KV head: with more than 16 query heads per KV head, each
  // KV head stands as kv_rep groups of `group` query heads (g counts those)
  const int gp = g / a.kv_rep, hkv = a.n_kv_heads / a.kv_rep;
  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const PageSrc src{static_cast<const char*>(a.k_pages), static_cast<const char*>(a.v_pages),
                    a.k_scales, a.v_scales, a.layer_page0, slab_bytes, hkv, bs};
  const int32_t* trow = a.table + (int64_t)b * a.table_stride;
  const int pg_last = (t_end - 1) / bs;

  const int t_new = len - 1;  // decode step: the position of the new row

  // A decode step's new row (its K chunks as the A operand lays them out, one
  // V value per dim lane), the page it goes to, and whether the length was
  // in range (a clamped length writes nothing).  At head_dim 64 the row is
  // fetched when the piece starts, so the loads are long done when its last
  // step needs them; at 128 the registers are not there, and the row is
  // fetched in the last step.
  constexpr bool kEarlyRow = D == 64;
  struct NewRow {
    uint4 kb4[NC];
    uint32_t vnew[ND];
    int page;
    bool ok;
  };
  auto fetch_new = [&](NewRow& nr) {
    nr.ok = a.lens[b] - a.prefix_len == len;
    const int64_t row = ((int64_t)b * hkv + gp) * D;
    const uint16_t* kr = static_cast<const uint16_t*>(a.k_new) + row;
    const uint16_t* vr = static_cast<const uint16_t*>(a.v_new) + row;
#pragma unroll
    for (int c = 0; c < NC; ++c) nr.kb4[c] = *reinterpret_cast<const uint4*>(kr + kdim(c, j));
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) nr.vnew[dt] = vr[16 * dt + n];
    nr.page = trow[t_new / bs];
  };
  NewRow early;
  if constexpr (kEarlyRow) {
    if (owns_new) fetch_new(early);
  }

  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float qs = a.qk_scale_log2;

  // The split is walked in windows of at most 64 logical pages: one table
  // entry per lane, picked out with a lane read (uniform) per tile.
  for (int w0 = t_begin; w0 < t_end; w0 = (w0 / bs + 64) * bs) {
    const int pg0 = w0 / bs;
    const int w_end = min((pg0 + 64) * bs, t_end);  // at most 64 pages, even from inside a page
    int vpage = -1;
    {
      const int lp = pg0 + lane;
      if (lp <= pg_last) {
        const int pg = trow[lp];
        if (pg < 0 || pg >= a.n_pages) report(a.status, PKV_DEV_READ_PAGE);
        else vpage = pg;
      }
    }

    // With 16-token pages a step spans pages A (tokens 0-15) and B (16-31);
    // with larger pages both halves sit on page A.
    auto load_step_at = [&](int ts, S& r) {
      const int lp = ts / bs;
      const int page_a = ts < w_end ? __builtin_amdgcn_readlane(vpage, lp - pg0) : -1;
      int page_b = page_a;
      if (BS == 16) page_b = ts + 16 < w_end ? __builtin_amdgcn_readlane(vpage, lp + 1 - pg0) : -1;
      load_step<FMT, D, BS>(r, src, page_a, page_b, ts - lp * bs, gp, lane);
    };

    auto compute_step = [&](int ts, S& r) {
      f32x4 sacc[2];
      step_scores<FMT, D>(r, qf, sacc);
      const bool lane_live = BS == 16 && j >= 2 ? r.live_b : r.live_a;
      float ksc[8], vsc[8];  // int8: scales of tokens 8j .. 8j+7
      if constexpr (FMT == PKV_FMT_INT8) step_scales<FMT, D>(r, ksc, vsc);
      float sv[8];
      bool ok[8];  // token 8j + x of the step is real
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        ok[x] = lane_live && ts + 8 * j + x < w_end;
        float y = sacc[x >> 2][x & 3] * qs;
        if (FMT == PKV_FMT_INT8) y *= ksc[x];
        sv[x] = ok[x] ? y : -INFINITY;
        mx = fmax_fast(mx, sv[x]);
      }
      mx = rows_max(mx);
      const float m_new = fmax_fast(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float psum = 0.f;
      float pw[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float p = ok[x] ? __builtin_amdgcn_exp2f(sv[x] - m_use) : 0.f;
        psum += p;
        pw[x] = p;
        // int8: a dead token's scale may be any bits (NaN too), so its
        // weight is zeroed rather than multiplied
        if (FMT == PKV_FMT_INT8) pw[x] = ok[x] ? p * vsc[x] : 0.f;
      }
      const bf16x8 pb = as_bf16x8(uint4{pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                        pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7])});
      l = l * alpha + psum;
      m = m_new;
      uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
      if (FMT == PKV_FMT_BF16 && (ts + 32 > w_end || !r.live_a || !r.live_b)) v_keep_masks(ok, keep);
      // the running outputs are rescaled only when some column's maximum
      // grew (alpha = 1 leaves them as they are, bit for bit)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
      }
      step_pv<FMT, D>(r, pb, keep, o);
    };

    // A fused decode step: the item that owns the sequence's last split loads
    // its head's new row, quantizes it for int8 pages (the page write's own
    // operations), stores it in its page, and puts it in place of the slot's
    // old contents in the registers of the step that holds it.  That step is
    // the item's last, handled after the pipelined loop with no load in
    // flight behind it, so the row costs no registers during the loop.
    auto substitute_new = [&](int ts, S& r) {
      if (!owns_new || t_new < ts || t_new >= ts + 32) return;
      NewRow late;
      if constexpr (!kEarlyRow) fetch_new(late);
      const NewRow& nr = kEarlyRow ? early : late;
      if (!nr.ok) return;  // an out-of-range length (reported, clamped): no write
      const int x_new = t_new - ts;                          // slot of the token in the step
      const int tau_new = (x_new >> 2) & 1;                  // score tile holding it
      const int n_new = ((x_new >> 3) << 2) | (x_new & 3);  // its K row lane
      const int j_new = x_new >> 3;                          // its V k-group
      uint4 kb4[NC];
      uint32_t vnew[ND];
#pragma unroll
      for (int c = 0; c < NC; ++c) kb4[c] = nr.kb4[c];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) vnew[dt] = nr.vnew[dt];
      KT knew[S::NK];
      float ks_new = 0.f, vs_new = 0.f;
      if constexpr (FMT == PKV_FMT_BF16) {
#pragma unroll
        for (int c = 0; c < NC; ++c) knew[c] = kb4[c];
      } else {
        // scale = max|x| / 127 over the row, code = clamp(rint(x / scale), +-127)
        float mk = 0.f, mv = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t w4[4] = {kb4[c].x, kb4[c].y, kb4[c].z, kb4[c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mk = fmaxf(mk, fmaxf(fabsf(bf16_bits_to_f32(w4[i] & 0xffffu)),
                                 fabsf(bf16_bits_to_f32(w4[i] >> 16))));
        }
        mk = fmaxf(mk, __shfl_xor(mk, 16, 64));
        mk = fmaxf(mk, __shfl_xor(mk, 32, 64));
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) mv = fmaxf(mv, fabsf(bf16_bits_to_f32(vnew[dt])));
#pragma unroll
        for (int o1 = 1; o1 < 16; o1 <<= 1) mv = fmaxf(mv, __shfl_xor(mv, o1, 64));
        ks_new = __fdiv_rn(mk, 127.0f);
        vs_new = __fdiv_rn(mv, 127.0f);
        auto code = [](float x, float sc) -> uint32_t {
          if (sc == 0.f) return 0u;
          const float q = fminf(fmaxf(rintf(__fdiv_rn(x, sc)), -127.f), 127.f);
          return (uint32_t)(int32_t)q & 0xffu;
        };
#pragma unroll
        for (int p = 0; p < S::NK; ++p) {
          uint32_t cw[4] = {0u, 0u, 0u, 0u};  // codes of chunks 2p (cw 0-1) and 2p + 1 (cw 2-3)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 kb = kb4[2 * p + h];
            const uint32_t w4[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t lo = code(bf16_bits_to_f32(w4[i] & 0xffffu), ks_new);
              const uint32_t hi = code(bf16_bits_to_f32(w4[i] >> 16), ks_new);
              cw[2 * h + (i >> 1)] |= (lo | (hi << 8)) << (16 * (i & 1));
            }
          }
          knew[p] = KT{cw[0], cw[1], cw[2], cw[3]};
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vnew[dt] = code(bf16_bits_to_f32(vnew[dt]), vs_new);
      }
      // the page write
      const int jp = t_new / bs;
      const int page = nr.page;
      if (g % a.kv_rep != 0) {
        // the KV head's row is written by its first group's piece
      } else if (page < 0 || page >= a.n_pages) {
        report(a.status, PKV_DEV_WRITE_PAGE);
      } else {
        const int slot = t_new - jp * bs;
        const int64_t slab = (a.layer_page0 + page) * hkv + gp;
        char* kw = static_cast<char*>(const_cast<void*>(a.k_pages)) + slab * slab_bytes;
        char* vw = static_cast<char*>(const_cast<void*>(a.v_pages)) + slab * slab_bytes;
        if (n == 0) {  // lanes j = 0..3 of one row hold the whole K row
#pragma unroll
          for (int c = 0; c < S::NK; ++c)
            *reinterpret_cast<KT*>(kw + k_byte(slot, kdim(KPL * c, j) * ESZ, bs, D * ESZ)) =
                knew[c];
        }
        if (j == 0) {  // lanes n = 0..15 hold every dim of the V row
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const int64_t e = (int64_t)(16 * dt + n) * bs + slot;
            if (FMT == PKV_FMT_BF16) reinterpret_cast<uint16_t*>(vw)[e] = (uint16_t)vnew[dt];
            else reinterpret_cast<uint8_t*>(vw)[e] = (uint8_t)vnew[dt];
          }
        }
        if (FMT == PKV_FMT_INT8 && lane == 0) {
          const_cast<float*>(a.k_scales)[slab * bs + slot] = ks_new;
          const_cast<float*>(a.v_scales)[slab * bs + slot] = vs_new;
        }
      }
      // the registers of this step
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int c = 0; c < S::NK; ++c)
          if (tau == tau_new && n == n_new) r.k[tau][c] = knew[c];
      if (j == j_new) {
        const int e = x_new & 7;  // element of this lane's 8-token V operand
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          if constexpr (FMT == PKV_FMT_BF16) {
            uint32_t w[4] = {r.v[dt].x, r.v[dt].y, r.v[dt].z, r.v[dt].w};
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
              if (q2 == (e >> 1))
                w[q2] = e & 1 ? (w[q2] & 0x0000ffffu) | (vnew[dt] << 16)
                              : (w[q2] & 0xffff0000u) | vnew[dt];
            r.v[dt] = uint4{w[0], w[1], w[2], w[3]};
          } else {
            uint32_t w[2] = {r.v[dt].x, r.v[dt].y};
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
              if (q2 == (e >> 2))
                w[q2] = (w[q2] & ~(0xffu << (8 * (e & 3)))) | (vnew[dt] << (8 * (e & 3)));
            r.v[dt] = uint2{w[0], w[1]};
          }
        }
      }
      if (FMT == PKV_FMT_INT8) {  // scale lanes: see Step::sc
        if (lane == 16 * j_new + (x_new & 7)) r.sc = ks_new;
        if (lane == 16 * j_new + 8 + (x_new & 7)) r.sc = vs_new;
      }
    };

    // ---- two register sets, loads one step ahead.  The loop body issues its
    // prefetches unconditionally and the last one or two steps are peeled:
    // a load under a condition would make the compiler wait for every
    // outstanding load (the prefetch included) before each step.  (Three
    // sets, two steps ahead, would keep more int8 bytes in flight, but do
    // not fit the 256 registers a wave has at two waves per SIMD.)
    const int n_steps = (w_end - w0 + 31) / 32;
    auto T = [&](int i) { return w0 + 32 * i; };
    S r0, r1;
    load_step_at(T(0), r0);
    int st = 0;
    for (; st + 2 < n_steps; st += 2) {
      load_step_at(T(st + 1), r1);
      compute_step(T(st), r0);
      load_step_at(T(st + 2), r0);
      compute_step(T(st + 1), r1);
    }
    if (st + 1 < n_steps) {
      load_step_at(T(st + 1), r1);
      compute_step(T(st), r0);
      substitute_new(T(st + 1), r1);
      compute_step(T(st + 1), r1);
    } else {
      substitute_new(T(st), r0);
      compute_step(T(st), r0);
    }
  }

  // ---- results: O^T lane layout = dims 16*dt + 4j + i of head n ----
  l = rows_sum(l);
  const int64_t hrow = (int64_t)b * a.n_q_heads + (int64_t)g * G + n;  // (b, h) row
  if (direct) {
    // the unit's only piece: normalise and write the output here
    if (n < G) {
      const float inv = 1.f / l;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        store_out4(a.out, a.q_bf16, hrow * D + 16 * dt + 4 * j, o[dt] * inv);
    }
  } else if (!a.fuse_combine) {
    // one of several pieces: leave the partial for the combine kernel
    if (n < G) {
      const int64_t row = row_base + (int64_t)n * row_step;
      float* wo = a.ws_o + row * D + 4 * j;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(wo + 16 * dt) = o[dt];
      if (j == 0) *reinterpret_cast<float2*>(a.ws_ml + row * 2) = float2{m, l};
    }
  } else {
    if (n < G) {
      const int64_t row = hrow * a.n_split + sp;
      float* wo = a.ws_o + row * D + 4 * j;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) put(wo + 16 * dt + i, o[dt][i]);
      if (j == 0) {
        put(a.ws_ml + row * 2, m);
        put(a.ws_ml + row * 2 + 1, l);
      }
    }
    // count this split in once its partial stores have completed; the
    // workgroup that brings the count to the sequence's number of splits
    // combines the group's partials and resets the counter for the next call
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t* counter = a.counters + (int64_t)b * a.n_kv_heads + g;
    unsigned old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old == (unsigned)(n_splits_b - 1)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      combine_group<D>(a, b, g, n_splits_b, lane);
      if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  }  // pieces
}

template <int FMT, int D, int BS, bool BAL, bool PRE>
__global__ __launch_bounds__(64 * kGroupWaves, 2) void attend_mfma_kernel(AttendArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int G = a.group;
  const int bs = BS ? BS : a.page_size;
  const int C = a.split_tokens;
  const int B = a.batch;

  // shared-prefix mode: the workgroups past the split pass's are the prefix
  // pass's waves (two column tiles per wave at head_dim 64; one at 128,
  // within this kernel's registers)
  if constexpr (PRE) {
    // the next step's table updates, spread over the launch's workgroups;
    // each names an entry no wave of this launch reads (checked: a row past
    // the length), so writing it here races with nothing
    for (int u = (int)(blockIdx.x * blockDim.x + threadIdx.x); u < a.n_next_upd;
         u += (int)(gridDim.x * blockDim.x)) {
      const int ub = a.next_upd[3 * u], blk = a.next_upd[3 * u + 1], pg = a.next_upd[3 * u + 2];
      if (ub < 0 || ub >= B || blk < 0 || blk >= a.table_stride) continue;
      int len = a.lens[ub];
      len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
      if ((int64_t)blk * bs < len) {
        report(a.status, PKV_DEV_TABLE_NEXT);
        continue;
      }
      a.upd_table[(int64_t)ub * a.table_stride + blk] = pg;
    }
    if ((int)blockIdx.x >= a.split_blocks) {  // a workgroup of prefix waves only
      constexpr int TT = prefix_tiles<D>();
      const int wid = ((int)blockIdx.x - a.split_blocks) * a.pre_group_waves + wave;
      const int n_pre = (int)prefix_col_blocks<TT>(B, G) * a.n_kv_heads * a.n_pchunks;
      if (wave < a.pre_group_waves && wid < n_pre) {
        if (a.qk_scale_log2 > 0.f)
          prefix_wave<FMT, D, BS, TT, true>(a, wid);
        else
          prefix_wave<FMT, D, BS, TT, false>(a, wid);
      }
      return;
    }
  }

  // ---- work list (LDS), one of two schedules.
  // Fixed splits: exclusive prefix sums over the sequences of their full
  // splits and of their partial last splits, and the clamped lengths.  Work
  // items are (split, KV head) pairs, full splits first, so the longest items
  // are handed out first; split wave v takes items v, v + split_waves, ...
  // Balanced (BAL): every (sequence, KV head) unit is a run of 32-token steps
  // preceded by unit_cost set-up slots (its query, table and first loads
  // start cold); fpre holds the exclusive prefix of the sequences' costs
  // n_kv_heads * (steps + unit_cost).  Wave w takes the slots
  // [w T / Wn, (w + 1) T / Wn) of that flat space, so every wave gets the
  // same share of steps plus set-ups, whatever the spread of lengths.  A
  // batch whose non-empty sequences all have one length is already balanced
  // by fixed splits, which cut it along KV heads and split boundaries (the
  // balanced cut measured slower there), so the BAL kernel takes the fixed
  // schedule for it and records the choice for the combine kernel.
  extern __shared__ int32_t wl[];
  int32_t* fpre = wl;              // [B + 1]
  int32_t* qpre = wl + B + 1;      // [B + 1]
  int32_t* lens = wl + 2 * B + 2;  // [B]
  int32_t* sched = wl + 3 * B + 2;  // [1]: the balanced schedule is taken
  // the workgroup's first wave builds the schedule for all of its waves
  if (wave == 0) {
    // clamped lengths into LDS (one load round trip), with the shortest and
    // longest non-empty ones
    int lmin = INT_MAX, lmax = 0;
    for (int b0 = 0; b0 < B; b0 += 256) {
      int lv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int bb = b0 + 64 * u + lane;
        lv[u] = bb < B ? a.lens[bb] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int bb = b0 + 64 * u + lane;
        int len = clamp_len(lv[u], a.max_len, blockIdx.x == 0 ? a.status : nullptr,
                            PKV_DEV_LEN);
        if (a.prefix_len > 0) {
          // the private suffix past the shared prefix; a decode step's new row
          // must land in it
          if (a.k_new && bb < B && len > 0 && len <= a.prefix_len && blockIdx.x == 0)
            report(a.status, PKV_DEV_PREFIX);
          len = max(len - a.prefix_len, 0);
        }
        if (bb < B) {
          lens[bb] = len;
          if (len > 0) {
            lmin = min(lmin, len);
            lmax = max(lmax, len);
          }
        }
      }
    }
    bool balanced = false;
    if constexpr (BAL) {
      // uneven lengths: some lane's non-empty ones differ from the first
      // non-empty lane's (two ballots and a lane read, no shuffles)
      const uint64_t busy = __builtin_amdgcn_ballot_w64(lmax > 0);
      if (busy) {
        const int l0 = __builtin_amdgcn_readlane(lmax, (int)__builtin_ctzll(busy));
        balanced = __builtin_amdgcn_ballot_w64(lmax > 0 && (lmin != l0 || lmax != l0)) != 0;
      }
      if (blockIdx.x == 0 && lane == 0) *a.ws_sched = balanced ? 1 : 0;
    }
    if (lane == 0) *sched = balanced ? 1 : 0;
    // exclusive prefix sums of the schedule's counts: lane l sums its run of
    // E = ceil(B / 64) consecutive sequences from the LDS lengths, one wave
    // scan gives the runs' offsets, then each lane writes its run.  (One
    // scan per 64 sequences, each a chain of lane shuffles, took 1.5-1.9 us
    // of the launch's start.)
    __builtin_amdgcn_wave_barrier();  // the lengths above, written by other lanes
    auto counts = [&](int len, int& f, int& q) {
      if (balanced) {
        const int steps = (len + 31) >> 5;
        f = steps > 0 ? a.n_kv_heads * (steps + a.unit_cost) : 0;
        q = 0;
      } else {
        f = len / C;
        q = len % C != 0 ? 1 : 0;
      }
    };
    const int E = (B + 63) >> 6;
    const int s0 = min(lane * E, B), s1 = min(s0 + E, B);
    int tf = 0, tq = 0;
    for (int bb = s0; bb < s1; ++bb) {
      int f, q;
      counts(lens[bb], f, q);
      tf += f;
      tq += q;
    }
    const int sf = wave_incl_scan(tf), sq = wave_incl_scan(tq);  // inclusive, over the lanes
    int cf = sf - tf, cq = sq - tq;
    for (int bb = s0; bb < s1; ++bb) {
      int f, q;
      counts(lens[bb], f, q);
      fpre[bb] = cf;
      qpre[bb] = cq;
      cf += f;
      cq += q;
    }
    if (lane == 63) {
      fpre[B] = sf;
      qpre[B] = sq;
    }
  }  // wave 0
  __syncthreads();
  // this wave's rank among the split waves, numbered across the workgroups
  // first: when only the first ranks find work, they still sit in different
  // workgroups, spread over every compute unit
  const int vb = wave * a.split_blocks + (int)blockIdx.x;
  if (vb >= a.split_waves) return;  // ranks past the last (a short launch's spare waves)
  if constexpr (BAL) {
    if (__builtin_amdgcn_readfirstlane(*sched) != 0) {
      run_pieces<FMT, D, BS, true>(a, fpre, qpre, lens, vb);
      return;
    }
  }
  run_pieces<FMT, D, BS, false>(a, fpre, qpre, lens, vb);
}

// Persistent launch: as many waves as the chip holds at once for this
// kernel (occupancy x compute units), capped by the number of work items
// the host can bound (every sequence at max_len).
int compute_units() {
  static thread_local int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

template <typename K>
int resident_waves(K kernel, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kGroupWaves, lds) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu * kGroupWaves * compute_units();
}

// Waves per workgroup for a launch of `waves` waves: the widest of 4, 2, 1
// that still gives every compute unit a workgroup.
inline int group_width(int64_t waves) {
  const int64_t cus = compute_units();
  return waves >= 4 * cus ? 4 : waves >= 2 * cus ? 2 : 1;
}

template <int FMT, int D, int BS, bool BAL, bool PRE>
hipError_t launch_sched(const AttendArgs& a, const Launch& l) {
  auto kernel = attend_mfma_kernel<FMT, D, BS, BAL, PRE>;
  const size_t lds = (size_t)(3 * a.batch + 3) * sizeof(int32_t);
  const int64_t bound = BAL ? a.bal_waves : (int64_t)a.n_kv_heads * a.batch * a.n_split;
  const int64_t resident = resident_waves(kernel, lds);
  AttendArgs b = a;
  if (a.prefix_len <= 0) {
    const int64_t waves = std::max<int64_t>(1, std::min<int64_t>(bound, resident));
    const int gw = group_width(waves);
    b.split_waves = (int32_t)waves;
    b.split_blocks = (int32_t)((waves + gw - 1) / gw);
    return launch1(kernel, dim3((unsigned)b.split_blocks), dim3(64 * gw), lds, l, b);
  }
  // shared-prefix mode: split workgroups first, then workgroups of prefix
  // waves, all resident together when they fit (the split pass leaves room)
  const int64_t pre = prefix_col_blocks<prefix_tiles<D>()>(a.batch, a.group) * a.n_kv_heads *
                      a.n_pchunks;
  int64_t split = a.split_wanted ? std::min<int64_t>(bound, resident) : 0;
  if (split > 0)
    split = std::max<int64_t>(1, std::min(split, std::max(resident - pre, resident / 2)));
  // The workgroup width follows the split pass's waves; prefix workgroups
  // use as many of their waves as spreads them over every compute unit (512
  // prefix waves in 4-wave groups sat on half the units).
  const int gw = group_width(std::max(split, pre));
  const int64_t cus = compute_units();
  const int wp = (int)std::max<int64_t>(1, std::min<int64_t>(gw, pre / cus));
  const int64_t split_groups = (split + gw - 1) / gw, groups = split_groups + (pre + wp - 1) / wp;
  if (groups > 0x7fffffff || split > 0x7fffffff) return hipErrorInvalidValue;
  b.split_waves = (int32_t)split;
  b.split_blocks = (int32_t)split_groups;
  b.pre_group_waves = wp;
  return launch1(kernel, dim3((unsigned)groups), dim3(64 * gw), lds, l, b);
}

template <int FMT, int D, int BS>
hipError_t launch_bs(const AttendArgs& a, const Launch& l) {
  if (a.prefix_len > 0)
    return a.bal_waves > 0 ? launch_sched<FMT, D, BS, true, true>(a, l)
                           : launch_sched<FMT, D, BS, false, true>(a, l);
  return a.bal_waves > 0 ? launch_sched<FMT, D, BS, true, false>(a, l)
                         : launch_sched<FMT, D, BS, false, false>(a, l);
}

template <int FMT, int D>
hipError_t launch_d(const AttendArgs& a, const Launch& l) {
  if (a.page_size == 16) return launch_bs<FMT, D, 16>(a, l);
  if (a.page_size == 32) return launch_bs<FMT, D, 32>(a, l);
  return launch_bs<FMT, D, 0>(a, l);
}

template <int FMT>
hipError_t launch_fmt(const AttendArgs& a, const Launch& l) {
  return a.head_dim == 128 ? launch_d<FMT, 128>(a, l) : launch_d<FMT, 64>(a, l);
}

}  // namespace

bool mfma_supported(int fmt, int q_bf16, int head_dim, int page_size, int group, int batch,
                    int n_kv_heads) {
  return (fmt == PKV_FMT_BF16 || fmt == PKV_FMT_INT8) && q_bf16 &&
         (head_dim == 64 || head_dim == 128) && (page_size == 16 || page_size % 32 == 0) &&
         group >= 1 && group <= 16 && batch >= 1 && batch <= kMaxMfmaBatch &&
         n_kv_heads <= kMaxMfmaKvHeads;
}

hipError_t launch_attend_mfma(const AttendArgs& a, int fmt, const Launch& l) {
  if (!mfma_supported(fmt, a.q_bf16, a.head_dim, a.page_size, a.group, a.batch, a.n_kv_heads))
    return hipErrorNotSupported;
  return fmt == PKV_FMT_BF16 ? launch_fmt<PKV_FMT_BF16>(a, l) : launch_fmt<PKV_FMT_INT8>(a, l);
}

}  // namespace pkv
