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
// How, on gfx950.  A workgroup of 8 waves (one per compute unit) owns one
// (sequence, KV head) and 16 * n_pos consecutive positions of its chunk;
// each wave holds two tiles of 16 matrix-core columns, each tile n_pos =
// 16 / G positions times the G heads (mfma_step.h gives the tile layouts),
// every column with its own causal bound, running maximum and sum.  Both
// tiles use the same K/V operand registers, so each LDS read feeds two
// matrix-core operations.  The workgroup walks the tokens up to its last
// position in blocks of four 32-token steps: all 512 threads load the next
// block's K/V (and int8 scales) from the pages into registers while the
// waves compute the current block's steps from LDS, then store it into the
// other set of LDS buffers (one barrier per 128 tokens).
// int8 codes are converted to bf16 once, on the way into LDS, and slots past
// the range or on a missing page are stored as zeros, so every wave reads
// plain bf16 operands.  Each byte read from the pages thus serves 256 query
// columns; there is no split of the token range, the parallelism comes from
// the queries.  Steps that every column of a wave sees whole skip the
// per-token masks, and the output is rescaled only when some column's
// running maximum grew.
//
// LDS holds K as [32 tokens][head_dim] (tokens in score-tile order, see
// k_row), rows padded by 32 bytes, and V as [head_dim][32 tokens], bf16, with
// the four 16-byte token chunks of a row permuted (v_chunk), so the rows one
// read instruction touches fall on different banks.  Measured on gfx950 for
// 16-byte reads: rows padded by 16 bytes (or 48, 64) conflict 2-way, by 32
// bytes not at all; unpadded V rows with the chunk index XOR-ed with bits 1-2
// of the row do not conflict either (V padded by 32 bytes would not fit the
// eight step buffers in LDS).
//
// Launch order is XCD-aware: workgroups are handed to the 8 XCDs in turn, so
// block x runs on XCD x % 8; the blocks of one (sequence, KV head) are given
// consecutive blocks of one XCD, where they run together and share that
// XCD's L2 copy of the sequence's pages.
#include <algorithm>

#include "mfma_step.h"

namespace pkv {
namespace {

constexpr int kXcds = 8;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTiles = 2;  // 16-column tiles per wave: both use the same K/V operands
constexpr int kPageWin = 512;  // page ids staged in LDS at a time
constexpr int kHalves = 4;     // 32-token steps per staged block (one barrier each)

template <int D>
struct MultiLds {
  static constexpr int KP = 2 * D + 32;  // K row pitch in bytes (one token)
  static constexpr int VP = 2 * 32;      // V row pitch in bytes (one dim), chunks permuted
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 32 * KP;
  static constexpr int S_OFF = V_OFF + D * VP;  // int8: 32 K scales, then 32 V scales
  static constexpr int BUF = S_OFF + 64 * 4;
};

// Position of 16-byte chunk c (tokens 8c .. 8c+7) in the LDS row of dim d.
__device__ __forceinline__ int v_chunk(int d, int c) { return c ^ ((d >> 1) & 3); }

// LDS row of token r of a step: the 16 tokens of score tile t (token
// 8 (n / 4) + 4t + n % 4 for row n) are stored in rows 16t .. 16t+15, so the
// lanes of one read instruction touch consecutive rows, whose 16-byte-padded
// pitch spreads them over distinct banks.
__device__ __forceinline__ int k_row(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// 16 int8 codes -> 16 bf16 (two 16-byte words)
__device__ __forceinline__ void codes16_to_bf16(uint4 w, uint4& lo, uint4& hi) {
  const uint2 a = codes_to_bf16(w.x), b = codes_to_bf16(w.y);
  const uint2 c = codes_to_bf16(w.z), d = codes_to_bf16(w.w);
  lo = uint4{a.x, a.y, b.x, b.y};
  hi = uint4{c.x, c.y, d.x, d.y};
}

// zero the bf16 elements e (0..7) of a 16-byte word with dead[e]
__device__ __forceinline__ uint4 zero_dead(uint4 v, uint32_t dead_bits) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = ((dead_bits >> (2 * i)) & 1u ? 0x0000ffffu : 0u) |
                       ((dead_bits >> (2 * i + 1)) & 1u ? 0xffff0000u : 0u);
    w[i] &= ~m;
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// RAW (a positive scale): scores stay in raw units (int8: times the token's
// K scale) until the exponential, whose one fma applies the scale; the
// running maximum is taken over raw scores and scaled once.
template <int FMT, int D, int BS, bool RAW>
__global__ __launch_bounds__(kThreads, 1) void attend_multi_kernel(MultiArgs a) {
  using L = MultiLds<D>;
  constexpr int NC = D / 32, ND = D / 16;
  constexpr int ESZ = FMT == PKV_FMT_BF16 ? 2 : 1;  // page element bytes
  constexpr int E = 16 / ESZ;                        // elements per 16-byte chunk
  constexpr int CK = D / E;                          // K chunks per token row
  constexpr int NKC = 32 * CK;                       // K chunks per step
  constexpr int CV = 32 / E;                         // V chunks per dim row
  constexpr int NVC = D * CV;                        // V chunks per step
  constexpr int KL = (NKC + kThreads - 1) / kThreads;
  constexpr int VL = (NVC + kThreads - 1) / kThreads;
  __shared__ __align__(16) char lds[2 * kHalves * L::BUF];

  const int tid = threadIdx.x;
  // wave-uniform values are made scalar so that branches on them are
  // scalar branches, not per-lane masks
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15;  // column (B/C operands)
  const int j = lane >> 4;  // k group (A/B operands), row quad (C operand)
  const int G = a.group;
  const int P = a.n_pos;
  const int bs = BS ? BS : a.page_size;

  // ---- the item: (sequence, KV head) pair and block of 4 * P positions
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int pair = (k / a.n_qgroups) * kXcds + xcd;
  const int qb = k % a.n_qgroups;
  if (pair >= a.batch * a.n_kv_heads) return;  // whole workgroup: uniform
  const int b = pair / a.n_kv_heads;
  const int g = pair - b * a.n_kv_heads;
  const bool reporter = qb == 0 && g == 0 && tid == 0;
  const int q0 = __builtin_amdgcn_readfirstlane(a.cu_q[b]);
  const int T = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]) - q0;
  if (q0 < 0 || T < 0 || q0 + T > a.total_q) {
    if (reporter) report(a.status, PKV_DEV_QROWS);
    return;  // malformed rows: none is read or written
  }
  const int len = clamp_len(__builtin_amdgcn_readfirstlane(a.lens[b]), a.max_len,
                            reporter ? a.status : nullptr, PKV_DEV_LEN);
  if (reporter && (T > len || T > a.max_q)) report(a.status, PKV_DEV_QROWS);
  const int pb0 = qb * kWaves * kTiles * P;  // the block's first position
  if (pb0 >= T) return;
  const int last_blk = min(pb0 + kWaves * kTiles * P, T) - 1;
  const int t_end = min(max(len - T + last_blk + 1, 0), len);  // tokens the block reads

  // ---- this wave's positions (kTiles tiles of P) and this lane's columns
  const int p0 = pb0 + wave * kTiles * P;
  const int p = n / G;
  const int h = n - p * G;
  bool col[kTiles];
  int pos[kTiles];  // below 0: sees nothing
  int64_t qrow[kTiles];
  bf16x8 qf[kTiles][NC];
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const int pu = p0 + u * P + p;
    col[u] = n < P * G && pu < T;
    pos[u] = len - T + pu;
    qrow[u] = col[u] ? (int64_t)(q0 + pu) * a.n_q_heads + (int64_t)g * G + h : 0;
    load_q<PKV_FMT_BF16, D>(qf[u], static_cast<const uint16_t*>(a.q) + qrow[u] * D,
                            col[u] && pos[u] >= 0, j);
  }
  const int w_last = p0 < T ? len - T + min(p0 + kTiles * P, T) - 1 : -1;  // wave's last

  const char* kp = static_cast<const char*>(a.k_pages);
  const char* vp = static_cast<const char*>(a.v_pages);
  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const int32_t* trow = a.table + (int64_t)b * a.table_stride;
  const int pg_last = t_end > 0 ? (t_end - 1) / bs : -1;

  // Page ids of a window of kPageWin logical pages, staged in LDS by the
  // whole workgroup (bad entries stored as -1 and reported), so a step's page
  // lookups are LDS reads and the step loads never wait on a table load.
  __shared__ int32_t pids[kPageWin];
  int win0 = 0;  // first logical page held in pids
  auto stage_pages = [&](int lp0) {  // all threads; ends with a barrier
    win0 = lp0;
    for (int e = tid; e < kPageWin; e += kThreads) {
      const int lp = lp0 + e;
      int v = -1;
      if (lp <= pg_last) {
        const int pg = trow[lp];
        if (pg < 0 || pg >= a.n_pages) report(a.status, PKV_DEV_READ_PAGE);
        else v = pg;
      }
      pids[e] = v;
    }
    __syncthreads();
  };
  // whether the window must move before the pages of a staged block
  // (logical pages lp .. lp + 2 kHalves at most) can be looked up
  auto window_misses = [&](int lp) {
    return lp < win0 || lp + 2 * kHalves + 1 >= win0 + kPageWin;
  };

  // ---- cooperative step load: registers, then LDS
  struct Stage {
    uint4 kc[KL], vc[VL];
    float sc;
    int page_a, page_b, slot0;
  };
  auto page_of = [&](int lp) {  // uniform; -1 past the range or on a bad entry
    return lp > pg_last ? -1 : __builtin_amdgcn_readfirstlane(pids[lp - win0]);
  };
  auto load_stage = [&](int ts, Stage& st) {
    const int lp = ts / bs;
    st.page_a = page_of(lp);
    st.page_b = BS == 16 ? (ts + 16 < t_end ? page_of(lp + 1) : -1) : st.page_a;
    st.slot0 = ts - lp * bs;
    const int64_t sa = (a.layer_page0 + max(st.page_a, 0)) * a.n_kv_heads + g;
    const int64_t sb = (a.layer_page0 + max(st.page_b, 0)) * a.n_kv_heads + g;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int q = tid + i * kThreads;
      st.kc[i] = uint4{0, 0, 0, 0};
      if (NKC % kThreads == 0 || q < NKC) {
        const int r = q / CK, c = q - r * CK;  // token row, chunk
        const bool on_b = BS == 16 && r >= 16;
        const int slot = BS == 16 ? (r & 15) : st.slot0 + r;
        st.kc[i] = stream_load<uint4, typename Step<FMT, D>::u32x4>(
            kp + (on_b ? sb : sa) * slab_bytes + k_byte(slot, c * 16, bs, D * ESZ));
      }
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int q = tid + i * kThreads;
      st.vc[i] = uint4{0, 0, 0, 0};
      if (NVC % kThreads == 0 || q < NVC) {
        const int d = q / CV, kk = q - d * CV;  // dim row, token group
        const int t0 = kk * E;
        const bool on_b = BS == 16 && t0 >= 16;
        const int slot = BS == 16 ? (t0 & 15) : st.slot0 + t0;
        st.vc[i] = stream_load<uint4, typename Step<FMT, D>::u32x4>(
            vp + (on_b ? sb : sa) * slab_bytes + ((int64_t)d * bs + slot) * ESZ);
      }
    }
    st.sc = 0.f;
    if (FMT == PKV_FMT_INT8 && tid < 64) {
      const int x = tid & 31;
      const bool on_b = BS == 16 && x >= 16;
      const int slot = BS == 16 ? (x & 15) : st.slot0 + x;
      const float* sp = tid < 32 ? a.k_scales : a.v_scales;
      st.sc = __builtin_nontemporal_load(sp + (on_b ? sb : sa) * bs + slot);
    }
  };
  auto store_stage = [&](int ts, const Stage& st, char* buf) {
    // token r of the step is dead past the block's range or on a missing
    // page; a whole step (the common case) is stored as it came
    const bool whole = ts + 32 <= t_end && st.page_a >= 0 && st.page_b >= 0;  // uniform
    const int live_n = t_end - ts;  // tokens r < live_n are inside the range
    auto page_dead = [&](int r) { return (BS == 16 && r >= 16 ? st.page_b : st.page_a) < 0; };
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int q = tid + i * kThreads;
      if (NKC % kThreads == 0 || q < NKC) {
        const int r = q / CK, c = q - r * CK;
        char* dst = buf + L::K_OFF + k_row(r) * L::KP + c * E * 2;
        const bool z = !whole && (r >= live_n || page_dead(r));
        if constexpr (FMT == PKV_FMT_BF16) {
          *reinterpret_cast<uint4*>(dst) = z ? uint4{0, 0, 0, 0} : st.kc[i];
        } else {
          uint4 lo, hi;
          codes16_to_bf16(st.kc[i], lo, hi);
          if (z) lo = hi = uint4{0, 0, 0, 0};
          *reinterpret_cast<uint4*>(dst) = lo;
          *reinterpret_cast<uint4*>(dst + 16) = hi;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int q = tid + i * kThreads;
      if (NVC % kThreads == 0 || q < NVC) {
        const int d = q / CV, kk = q - d * CV;
        const int t0 = kk * E;
        char* row = buf + L::V_OFF + d * L::VP;  // the chunks of tokens t0 ..
        // one bit per token of the chunk (its E tokens share one page half):
        // all on a missing page, else those at or past the range's end
        uint32_t dbits = 0;
        if (!whole) {
          const int keep = min(max(live_n - t0, 0), E);
          dbits = page_dead(t0) ? (1u << E) - 1u : ((1u << E) - 1u) & ~((1u << keep) - 1u);
        }
        if constexpr (FMT == PKV_FMT_BF16) {  // one chunk of 8 tokens
          *reinterpret_cast<uint4*>(row + 16 * v_chunk(d, kk)) =
              whole ? st.vc[i] : zero_dead(st.vc[i], dbits);
        } else {  // 16 codes: two chunks of bf16
          uint4 lo, hi;
          codes16_to_bf16(st.vc[i], lo, hi);
          *reinterpret_cast<uint4*>(row + 16 * v_chunk(d, 2 * kk)) =
              whole ? lo : zero_dead(lo, dbits & 0xffu);
          *reinterpret_cast<uint4*>(row + 16 * v_chunk(d, 2 * kk + 1)) =
              whole ? hi : zero_dead(hi, dbits >> 8);
        }
      }
    }
    if (FMT == PKV_FMT_INT8 && tid < 64) {
      const int r = tid & 31;
      reinterpret_cast<float*>(buf + L::S_OFF)[tid] =
          !whole && (r >= live_n || page_dead(r)) ? 0.f : st.sc;
    }
  };

  // o: the unnormalised outputs; ls: the softmax sums, taken by one more
  // matrix-core product per tile and step with an all-ones A operand (every
  // row of the result is the column's sum over the step's 32 weights, in
  // every lane of the column), which replaces per-lane adds and the final
  // cross-lane reduction; m: the reference maximum the weights are taken
  // against.
  f32x4 o[kTiles][ND], ls[kTiles];
  float m[kTiles];
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    ls[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[u] = -INFINITY;
  }
  const bf16x8 ones = as_bf16x8(uint4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const float qs = a.qk_scale_log2;

  // The wave's smallest position: every column of the wave sees a step whole
  // when the step lies below it (and inside the block's range, on live pages).
  const int pos_min = len - T + p0;

  auto compute_step = [&](int ts, const char* buf, bool live_a, bool live_b) {
    f32x4 sacc[kTiles][2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int u = 0; u < kTiles; ++u) sacc[u][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * tau + n;  // LDS row of token 8 (n / 4) + 4 tau + n % 4
      // all of the tile's K chunks in one batch of reads, then the products
      uint4 kw[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kw[c] = *reinterpret_cast<const uint4*>(buf + L::K_OFF + row * L::KP +
                                                kdim_of<PKV_FMT_BF16>(c, j) * 2);
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < kTiles; ++u)
          sacc[u][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw[c]), qf[u][c],
                                                                 sacc[u][tau], 0, 0, 0);
    }
    float ksc[8], vsc[8];
    if constexpr (FMT == PKV_FMT_INT8) {
      const float4* sp = reinterpret_cast<const float4*>(buf + L::S_OFF);
      const float4 k0 = sp[2 * j], k1 = sp[2 * j + 1], v0 = sp[8 + 2 * j], v1 = sp[8 + 2 * j + 1];
      const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        ksc[x] = kk[x];
        vsc[x] = vv[x];
      }
    }
    // the step's V operands, read now so the reads are in flight during the
    // softmax
    uint4 vw[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      vw[dt] = *reinterpret_cast<const uint4*>(buf + L::V_OFF + (16 * dt + n) * L::VP +
                                               16 * v_chunk(16 * dt + n, j));
    // wave-uniform: every token of the step is seen by every column
    const bool open = live_a && live_b && ts + 31 <= pos_min && ts + 32 <= t_end;
    const bool lane_live = BS == 16 && j >= 2 ? live_b : live_a;
    // Phase 1, per tile: scores, maxima, the reference maximum and the rescale
    // (rare); phase 2 then holds no branch, so the exponentials of one tile
    // and the P.V products of the other can interleave.
    float sv[kTiles][8], m_use[kTiles];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      // scores: raw sums (int8: times the token's K scale), in log2 units
      // unless RAW.  A token the column may not see gets -inf, in place, and
      // so a weight of exactly 0 (exp2(-inf) = 0): both paths share the
      // exponentials below.
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        sv[u][x] = sacc[u][x >> 2][x & 3];
        if (FMT == PKV_FMT_INT8) sv[u][x] *= ksc[x];
        if (!RAW) sv[u][x] *= qs;
      }
      if (!open) {
        const int lim = min(pos[u], t_end - 1) - ts - 8 * j;  // token 8j + x seen iff x <= lim
#pragma unroll
        for (int x = 0; x < 8; ++x) sv[u][x] = lane_live && x <= lim ? sv[u][x] : -INFINITY;
      }
      float mx = sv[u][0];
#pragma unroll
      for (int x = 1; x < 8; ++x) mx = fmax_fast(mx, sv[u][x]);
      mx = rows_max(mx);
      if (RAW) mx *= qs;  // a positive scale keeps the maximum where it is
      const float m_new = fmax_fast(m[u], mx);
      // Lazy rescale: the weights are taken against a reference maximum that
      // moves only when some column's maximum passed it by more than
      // kRescaleSlack (log2 units), so weights stay below 2^kRescaleSlack and
      // the outputs and sums are rescaled on few steps.
      const bool grow = __any(m_new > m[u] + kRescaleSlack);  // -inf + slack: any finite max
      const float m_ref = grow ? m_new : m[u];
      m_use[u] = m_ref == -INFINITY ? 0.f : m_ref;
      if (grow) {
        const float alpha = __builtin_amdgcn_exp2f(m[u] - m_use[u]);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[u][dt] *= alpha;
        ls[u] *= alpha;
        m[u] = m_ref;
      }
    }
    // Phase 2: weights, P.V and the sums
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      float pw[8];
      float pv[8];  // the weights of the sums (int8: before the V scale)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float pr = __builtin_amdgcn_exp2f(RAW ? fmaf(sv[u][x], qs, -m_use[u])
                                                    : sv[u][x] - m_use[u]);
        pv[x] = pr;
        pw[x] = FMT == PKV_FMT_INT8 ? pr * vsc[x] : pr;
      }
      const bf16x8 pb = as_bf16x8(uint4{pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                        pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7])});
      const bf16x8 ps = FMT == PKV_FMT_INT8
                            ? as_bf16x8(uint4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                              pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])})
                            : pb;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw[dt]), pb, o[u][dt], 0, 0, 0);
      ls[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ps, ls[u], 0, 0, 0);
    }
  };

  // ---- the step loop: the loads of step i+1 are in flight while step i is
  // computed from LDS; then step i+1 goes into the other LDS buffer (one
  // barrier per step).  The prefetch is issued every iteration (past the
  // last step it reloads the last step, unused): a load under a condition
  // would make every step wait for all outstanding loads.
  const int n_steps = (t_end + 31) / 32;
  if (n_steps > 0) {
    // Blocks of kHalves 32-token steps are staged at a time, so one barrier,
    // one round of page lookups and one load/store round serve 64 tokens.
    // Halves past the last step load the last step again and are stored as
    // dead slots (zeros) that no wave computes.
    const int ts_last = 32 * (n_steps - 1);
    const int n_blocks = (n_steps + kHalves - 1) / kHalves;
    auto at = [&](int ts) { return min(ts, ts_last); };
    stage_pages(0);
    Stage st[kHalves];
    bool la[kHalves], lb[kHalves];
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      load_stage(at(32 * hf), st[hf]);
      store_stage(32 * hf, st[hf], lds + hf * L::BUF);
      la[hf] = st[hf].page_a >= 0;
      lb[hf] = st[hf].page_b >= 0;
    }
    __syncthreads();
    for (int i = 0; i < n_blocks; ++i) {
      const int ts = 32 * kHalves * i;
      const int ts1 = ts + 32 * kHalves;  // the next block
      if (window_misses(at(ts1) / bs)) stage_pages(at(ts1) / bs);  // uniform, rare
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) load_stage(at(ts1 + 32 * hf), st[hf]);
      char* cur = lds + (i & 1) * kHalves * L::BUF;
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf)
        if (ts + 32 * hf <= w_last) compute_step(ts + 32 * hf, cur + hf * L::BUF, la[hf], lb[hf]);
      if (i + 1 < n_blocks) {
        char* nxt = lds + ((i + 1) & 1) * kHalves * L::BUF;
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) {
          store_stage(ts1 + 32 * hf, st[hf], nxt + hf * L::BUF);
          la[hf] = st[hf].page_a >= 0;
          lb[hf] = st[hf].page_b >= 0;
        }
      }
      __syncthreads();
    }
  }

  // ---- results: O^T lane layout = dims 16 dt + 4j + i of column n
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const float lu = ls[u][0];  // the column's whole sum, in every lane of the column
    if (col[u]) {
      const float inv = lu > 0.f ? 1.f / lu : 0.f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        store_out4(a.out, 1, qrow[u] * D + 16 * dt + 4 * j, o[u][dt] * inv);
    }
  }
}

template <int FMT, int D, int BS>
hipError_t launch_bs(const MultiArgs& a, const Launch& l) {
  const int64_t grid = multi_grid(a.batch, a.n_kv_heads, a.n_qgroups);
  if (a.qk_scale_log2 > 0.f)
    return launch1(attend_multi_kernel<FMT, D, BS, true>, dim3((unsigned)grid), dim3(kThreads), 0,
                   l, a);
  return launch1(attend_multi_kernel<FMT, D, BS, false>, dim3((unsigned)grid), dim3(kThreads), 0,
                 l, a);
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

int multi_positions_per_block(int group) { return kWaves * kTiles * (16 / group); }

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
