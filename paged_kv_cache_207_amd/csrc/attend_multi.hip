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
// (sequence, KV head) and 16 * n_pos positions of its chunk; each wave holds
// two tiles of 16 matrix-core columns, each tile n_pos = 16 / G consecutive
// positions times the G heads (mfma_step.h gives the tile layouts), every
// column with its own causal bound, running maximum and sum.  The waves'
// runs of 2 n_pos positions are dealt to the sequence's workgroups in turn,
// so that each workgroup reads about as many tokens as the others.  Both
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
// k_row) and V as [head_dim][32 tokens], bf16, unpadded, with the 16-byte
// chunks of a row permuted by bits of the row (k_pos, v_chunk), so the rows
// one read instruction touches fall on different banks.  bf16 pages are
// copied into LDS by the memory unit itself (global_load_lds, 16 bytes a
// lane): no registers hold the next block and no LDS stores are issued, so
// the waves' instruction streams carry only the address arithmetic; each
// wave's 64 chunks of a load land side by side, which the unpadded layout
// allows.  Dead slots of a partial step are zeroed after the copy lands.
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
constexpr int kHalves = 4;
constexpr int kCopyWaves = 4;  // waves that copy bf16 steps into LDS (one per SIMD)     // 32-token steps per staged block (one barrier each)

template <int D>
struct MultiLds {
  static constexpr int KP = 2 * D;   // K row pitch in bytes (one token), chunks swizzled
  static constexpr int VP = 2 * 32;  // V row pitch in bytes (one dim), chunks permuted
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 32 * KP;
  static constexpr int S_OFF = V_OFF + D * VP;  // int8: 32 K scales, then 32 V scales
  static constexpr int BUF = S_OFF + 64 * 4;
};

// Position of 16-byte chunk c (tokens 8c .. 8c+7) in the LDS row of dim d.
__device__ __forceinline__ int v_chunk(int d, int c) { return c ^ ((d >> 1) & 3); }

// LDS row of token r of a step: the 16 tokens of score tile t (token
// 8 (n / 4) + 4t + n % 4 for row n) are stored in rows 16t .. 16t+15, so the
// lanes of one read instruction touch consecutive rows.
__device__ __forceinline__ int k_row(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}
// The token stored in LDS row `row` (k_row inverted).
__device__ __forceinline__ int k_tok(int row) {
  const int n = row & 15;
  return 8 * (n >> 2) + 4 * (row >> 4) + (n & 3);
}
// Byte offset of 16-byte chunk c (dims 8c .. 8c+7) of K row `row`: the chunk
// index is XOR-ed with bits of the row, so the rows one read instruction
// touches (same c, consecutive rows) fall on distinct banks: 256-byte rows
// take bits 0-3 (16 chunk positions over 16 rows); 128-byte rows take bits
// 1-3, row parity giving the other half of the banks.
template <int D>
__device__ __forceinline__ int k_pos(int row, int c) {
  const int swz = D == 128 ? (row & 15) : ((row >> 1) & 7);
  return row * 2 * D + 16 * (c ^ swz);
}

// A wave-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The column maxima of two tiles at once (each over the four 16-lane rows,
// in every lane of the column): the first row swap pairs rows 0-1 and 2-3 of
// x in one register with those of y in the other, so one maximum serves
// both; x's pair maxima then sit in rows 0 and 2, y's in 1 and 3.  A half
// swap and a maximum give x's column maxima in rows 0 and 2 and y's in 1
// and 3, and a last row swap hands each to all four rows.  Three swaps and
// two maxima instead of four and four.
__device__ __forceinline__ void rows_max2(float& x, float& y) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  const float z = fmax_fast(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false,
                                                  false);
  const float w = fmax_fast(__uint_as_float(b[0]), __uint_as_float(b[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false,
                                                  false);
  x = __uint_as_float(c[0]);
  y = __uint_as_float(c[1]);
}

// 16 bytes per lane from global memory straight into LDS: the wave's 64
// chunks land side by side from lds_wave (wave-uniform), lane l's at
// lds_wave + 16 l.  Completion counts on the vector-memory counter.
__device__ __forceinline__ void lds_dma16(const char* src, char* lds_wave) {
  __builtin_amdgcn_global_load_lds(
      (__attribute__((address_space(1))) void*)(const_cast<char*>(src)),
      (__attribute__((address_space(3))) void*)(lds_wave), 16, 0, 0);
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
  // two sets of kHalves step buffers, used in turn
  __shared__ __align__(16) char lds0[kHalves * L::BUF];
  __shared__ __align__(16) char lds1[kHalves * L::BUF];
  __shared__ int32_t live_bits[2];  // bf16: liveness of the next block's pages, by block parity

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
  // The chunk's positions go to waves in runs of WP; run r belongs to
  // workgroup r % nq, so each of the sequence's nq workgroups holds runs from
  // the start to the end of the chunk and reads about as many tokens as the
  // others (the last positions see the most tokens).
  const int WP = kTiles * P;                        // positions per wave
  const int n_runs = (T + WP - 1) / WP;             // runs holding positions
  const int nq = min((T + kWaves * WP - 1) / (kWaves * WP), a.n_qgroups);
  if (qb >= nq) return;  // T = 0 too
  const int top = min((n_runs - 1 - qb) / nq, kWaves - 1);  // the workgroup's last run
  const int last_blk = min((qb + nq * top) * WP + WP, T) - 1;
  const int t_end = min(max(len - T + last_blk + 1, 0), len);  // tokens the block reads

  // ---- this wave's positions (kTiles tiles of P) and this lane's columns
  const int p0 = (qb + nq * wave) * WP;  // at or past T: no positions
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

  // this KV head's slab of logical page 0 of the layer, and the distance
  // between the slabs of consecutive page ids
  const int64_t slab0 = a.layer_page0 * a.n_kv_heads + g;
  const int64_t slab_bytes = (int64_t)bs * D * ESZ;
  const char* kp = static_cast<const char*>(a.k_pages) + slab0 * slab_bytes;
  const char* vp = static_cast<const char*>(a.v_pages) + slab0 * slab_bytes;
  const int64_t page_bytes = slab_bytes * a.n_kv_heads;
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

  // ---- step staging.  The pages of a step: page_a holds its first slot
  // (slot0) and, with pages of 16, page_b its last 16 tokens.
  struct Pages {
    int page_a, page_b, slot0;
  };
  // The page ids of logical pages lp0 .. lp0 + kBlockPages - 1 (the most a
  // staged block starting in page lp0 touches), one per lane, from one LDS
  // read: the block's uniform lookups then read lanes of it instead of
  // waiting on an LDS round trip each.  -1 past the range or on a bad entry.
  constexpr int kBlockPages = 2 * kHalves + 2;
  auto block_pages = [&](int lp0) {
    const int e = min(lane, kBlockPages - 1);  // inside the window (window_misses)
    const int v = pids[lp0 - win0 + e];
    return lane < kBlockPages && lp0 + lane <= pg_last ? v : -1;
  };
  auto step_pages = [&](int ts, int pl, int lp0) {
    Pages s;
    const int lp = ts / bs;
    s.page_a = __builtin_amdgcn_readlane(pl, lp - lp0);
    s.page_b = BS == 16 ? (ts + 16 < t_end ? __builtin_amdgcn_readlane(pl, lp + 1 - lp0) : -1)
                        : s.page_a;
    s.slot0 = ts - lp * bs;
    return s;
  };
  // a step whose 32 slots are all inside the range on live pages
  auto step_whole = [&](int ts, const Pages& s) {
    return ts + 32 <= t_end && s.page_a >= 0 && s.page_b >= 0;
  };

  // bf16: the step's 16-byte LDS chunks, K rows first, then V rows; chunk q
  // comes from one 16-byte piece of a page
  constexpr int KCB = D / 8;                // chunks per K row
  constexpr int NKB = 32 * KCB;             // K chunks per step
  constexpr int NCH = NKB + D * 4;          // all chunks of a step
  constexpr int CL = NCH / kThreads;        // chunks per thread
  static_assert(NCH % kThreads == 0 && NKB % 64 == 0, "a wave's chunks are all K or all V");
  // Chunk i of a thread (q = tid + i kThreads) is a K chunk for the first
  // NKB (whole waves).  Its source, for a step whose pages are at byte
  // offsets 0 and whose first slot is 0, and the page it lies on (page_b:
  // the second 16 tokens with pages of 16) are the same for every step; a
  // step adds its page's offset and, for pages of more than 32 tokens, its
  // first slot's (slot0, a multiple of 32, moves every K byte of a slab by
  // k_byte(slot0, 0) and every V byte by 2 slot0).
  // Only the first kCopyWaves waves issue the copies (each thread CW
  // chunks): the two waves of a SIMD would otherwise both spend the start of
  // every block issuing them, with no compute to overlap; this way the
  // other wave of each SIMD computes meanwhile.
  constexpr int kCopyThreads = 64 * kCopyWaves;
  constexpr int CW = NCH / kCopyThreads;
  static_assert(NCH % kCopyThreads == 0 && NKB % kCopyThreads == 0 || NKB < kCopyThreads,
                "a copy wave's chunks are all K or all V");
  auto is_k = [&](int i) {
    return NKB >= kCopyThreads ? i < NKB / kCopyThreads : wave < NKB / 64;  // uniform
  };
  const char* csrc[CW];
  bool con_b[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int q = tid + i * kCopyThreads;
    if (is_k(i)) {
      const int row = q / KCB, c = (q % KCB) ^ ((k_pos<D>(row, 0) / 16) & (KCB - 1));
      const int r = k_tok(row);
      con_b[i] = BS == 16 && r >= 16;
      csrc[i] = kp + k_byte(BS == 16 ? (r & 15) : r, c * 16, bs, D * 2);
    } else {
      const int d = (q - NKB) >> 2, c = v_chunk(d, (q - NKB) & 3);
      con_b[i] = BS == 16 && c >= 2;
      csrc[i] = vp + ((int64_t)d * bs + (BS == 16 ? (8 * c) & 15 : 8 * c)) * 2;
    }
  }
  auto copy_step = [&](const Pages& s, char* buf) {
    // (scalar offsets, selected per lane: without the read-first-lane the
    // compiler selects the page per lane and multiplies per lane)
    const int64_t oa = uniform64(max(s.page_a, 0) * page_bytes);
    const int64_t ob = uniform64(max(s.page_b, 0) * page_bytes);
    const int64_t kd = BS == 0 ? k_byte(s.slot0, 0, bs, D * 2) : 0;
    const int64_t vd = BS == 0 ? 2 * s.slot0 : 0;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int64_t off = (con_b[i] ? ob : oa) + (is_k(i) ? kd : vd);
      lds_dma16(csrc[i] + off, buf + 16 * (wave * 64 + i * kCopyThreads));
    }
  };
  // after the copy landed: zero the K rows and V slots of tokens past the
  // range or on a missing page (each chunk is one thread's)
  auto zero_dead_slots = [&](int ts, const Pages& s, char* buf) {
    const int live_n = t_end - ts;
    auto page_dead = [&](int r) { return (BS == 16 && r >= 16 ? s.page_b : s.page_a) < 0; };
#pragma unroll
    for (int i = 0; i < CL; ++i) {
      const int q = tid + i * kThreads;
      uint4* p = reinterpret_cast<uint4*>(buf + 16 * q);
      if (q < NKB) {
        const int r = k_tok(q / KCB);
        if (r >= live_n || page_dead(r)) *p = uint4{0, 0, 0, 0};
      } else {
        const int t0 = 8 * v_chunk((q - NKB) >> 2, (q - NKB) & 3);
        const int keep = min(max(live_n - t0, 0), 8);
        const uint32_t dbits = page_dead(t0) ? 0xffu : 0xffu & ~((1u << keep) - 1u);
        if (dbits) *p = zero_dead(*p, dbits);
      }
    }
  };

  // int8: codes through registers, converted to bf16 on the way into LDS
  struct Stage {
    uint4 kc[KL], vc[VL];
    float sc;
  };
  auto load_stage = [&](const Pages& pg, Stage& st) {
    const int64_t oa = uniform64(max(pg.page_a, 0) * page_bytes);
    const int64_t ob = uniform64(max(pg.page_b, 0) * page_bytes);
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int q = tid + i * kThreads;
      st.kc[i] = uint4{0, 0, 0, 0};
      if (NKC % kThreads == 0 || q < NKC) {
        const int r = q / CK, c = q - r * CK;  // token row, chunk
        const bool on_b = BS == 16 && r >= 16;
        const int slot = BS == 16 ? (r & 15) : pg.slot0 + r;
        st.kc[i] = stream_load<uint4, typename Step<FMT, D>::u32x4>(
            kp + (on_b ? ob : oa) + k_byte(slot, c * 16, bs, D * ESZ));
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
        const int slot = BS == 16 ? (t0 & 15) : pg.slot0 + t0;
        st.vc[i] = stream_load<uint4, typename Step<FMT, D>::u32x4>(
            vp + (on_b ? ob : oa) + ((int64_t)d * bs + slot) * ESZ);
      }
    }
    st.sc = 0.f;
    if (FMT == PKV_FMT_INT8 && tid < 64) {
      const int x = tid & 31;
      const bool on_b = BS == 16 && x >= 16;
      const int slot = BS == 16 ? (x & 15) : pg.slot0 + x;
      const float* sp = tid < 32 ? a.k_scales : a.v_scales;
      const int64_t sl = slab0 + (int64_t)max(on_b ? pg.page_b : pg.page_a, 0) * a.n_kv_heads;
      st.sc = __builtin_nontemporal_load(sp + sl * bs + slot);
    }
  };
  auto store_stage = [&](int ts, const Pages& pg, const Stage& st, char* buf) {
    // token r of the step is dead past the block's range or on a missing
    // page; a whole step (the common case) is stored as it came
    const bool whole = step_whole(ts, pg);  // uniform
    const int live_n = t_end - ts;  // tokens r < live_n are inside the range
    auto page_dead = [&](int r) { return (BS == 16 && r >= 16 ? pg.page_b : pg.page_a) < 0; };
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int q = tid + i * kThreads;
      if (NKC % kThreads == 0 || q < NKC) {
        const int r = q / CK, c = q - r * CK;  // 16 codes: bf16 chunks 2c, 2c + 1
        const bool z = !whole && (r >= live_n || page_dead(r));
        uint4 lo, hi;
        codes16_to_bf16(st.kc[i], lo, hi);
        if (z) lo = hi = uint4{0, 0, 0, 0};
        *reinterpret_cast<uint4*>(buf + L::K_OFF + k_pos<D>(k_row(r), 2 * c)) = lo;
        *reinterpret_cast<uint4*>(buf + L::K_OFF + k_pos<D>(k_row(r), 2 * c + 1)) = hi;
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
        uint4 lo, hi;  // 16 codes: two chunks of bf16
        codes16_to_bf16(st.vc[i], lo, hi);
        *reinterpret_cast<uint4*>(row + 16 * v_chunk(d, 2 * kk)) =
            whole ? lo : zero_dead(lo, dbits & 0xffu);
        *reinterpret_cast<uint4*>(row + 16 * v_chunk(d, 2 * kk + 1)) =
            whole ? hi : zero_dead(hi, dbits >> 8);
      }
    }
    if (tid < 64) {
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
  // against, and m_use the same with 0 in place of -inf (no token seen yet),
  // so that the weights' exponent never takes -inf - -inf.
  f32x4 o[kTiles][ND], ls[kTiles];
  float m[kTiles], m_use[kTiles];
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    ls[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[u] = -INFINITY;
    m_use[u] = 0.f;
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
        kw[c] = *reinterpret_cast<const uint4*>(
            buf + L::K_OFF + k_pos<D>(row, kdim_of<PKV_FMT_BF16>(c, j) / 8));
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
    float sv[kTiles][8], mxs[kTiles];
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
      mxs[u] = sv[u][0];
#pragma unroll
      for (int x = 1; x < 8; ++x) mxs[u] = fmax_fast(mxs[u], sv[u][x]);
    }
    static_assert(kTiles == 2, "the column maxima of two tiles are taken together");
    rows_max2(mxs[0], mxs[1]);
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      float mx = mxs[u];
      if (RAW) mx *= qs;  // a positive scale keeps the maximum where it is
      const float m_new = fmax_fast(m[u], mx);
      // Lazy rescale: the weights are taken against a reference maximum that
      // moves only when some column's maximum passed it by more than
      // kRescaleSlack (log2 units), so weights stay below 2^kRescaleSlack and
      // the outputs and sums are rescaled on few steps.
      const bool grow = __any(m_new > m[u] + kRescaleSlack);  // -inf + slack: any finite max
      if (grow) {  // (rare) the reference moves to m_new
        const float mu = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[u] - mu);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[u][dt] *= alpha;
        ls[u] *= alpha;
        m[u] = m_new;
        m_use[u] = mu;
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

  // ---- the step loop, in blocks of kHalves 32-token steps: the next
  // block's copy is in flight while the waves compute the current one from
  // the other set of LDS buffers; one barrier per block (two where a step of
  // the next block has dead slots to zero).  The two buffer sets are
  // distinct arrays, used in turn by a loop unrolled twice, so the compiler
  // sees that the copy into one never overlaps the reads of the other and
  // does not wait for it before them.  Halves past the last step take the
  // last step's pages and are never computed.
  const int n_steps = (t_end + 31) / 32;
  if (n_steps > 0) {
    const int ts_last = 32 * (n_steps - 1);
    const int n_blocks = (n_steps + kHalves - 1) / kHalves;
    auto at = [&](int ts) { return min(ts, ts_last); };
    // whether step ts of a block just copied has dead slots that a wave reads
    auto needs_zeros = [&](int ts, const Pages& pg) { return ts < t_end && !step_whole(ts, pg); };
    stage_pages(0);
    Pages pg[kHalves];
    Stage st[kHalves];
    int pa[kHalves], pb[kHalves];  // the computed block's page ids (uniform: scalar registers)
    {
      const int pl0 = block_pages(0);
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        pg[hf] = step_pages(at(32 * hf), pl0, 0);
        if constexpr (FMT == PKV_FMT_BF16) {
          if (wave < kCopyWaves) copy_step(pg[hf], lds0 + hf * L::BUF);
        } else {
          load_stage(pg[hf], st[hf]);
          store_stage(32 * hf, pg[hf], st[hf], lds0 + hf * L::BUF);
        }
        pa[hf] = pg[hf].page_a;
        pb[hf] = pg[hf].page_b;
      }
      __syncthreads();
      if constexpr (FMT == PKV_FMT_BF16) {
        bool z = false;
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) z = z || needs_zeros(32 * hf, pg[hf]);
        if (z) {
#pragma unroll
          for (int hf = 0; hf < kHalves; ++hf)
            if (needs_zeros(32 * hf, pg[hf])) zero_dead_slots(32 * hf, pg[hf], lds0 + hf * L::BUF);
          __syncthreads();
        }
      }
    }
    auto block = [&](int i, char* cur, char* nxt) __attribute__((always_inline)) {
      const int ts = 32 * kHalves * i;
      const int ts1 = ts + 32 * kHalves;  // the next block
      const bool more = i + 1 < n_blocks;
      const int lp1 = at(ts1) / bs;
      if (window_misses(lp1)) stage_pages(lp1);  // uniform, rare
      if constexpr (FMT == PKV_FMT_BF16) {
        // bf16: the copy waves look the next block's pages up, copy it and
        // publish which of its pages are live; the other waves read that
        // after the barrier instead of looking the pages up themselves
        if (wave < kCopyWaves) {
          const int pl = block_pages(lp1);
          int bits = 0;
#pragma unroll
          for (int hf = 0; hf < kHalves; ++hf) {
            pg[hf] = step_pages(at(ts1 + 32 * hf), pl, lp1);
            bits |= (pg[hf].page_a >= 0 ? 1 : 0) << (2 * hf);
            bits |= (pg[hf].page_b >= 0 ? 2 : 0) << (2 * hf);
          }
          if (more) {
#pragma unroll
            for (int hf = 0; hf < kHalves; ++hf) copy_step(pg[hf], nxt + hf * L::BUF);
          }
          if (tid == 0) live_bits[(i + 1) & 1] = bits;
        }
      } else {
        const int pl = block_pages(lp1);
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) pg[hf] = step_pages(at(ts1 + 32 * hf), pl, lp1);
        // issued every block (past the last, the last step again): a load
        // under a condition would make every step wait for all loads
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) load_stage(pg[hf], st[hf]);
      }
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf)
        if (ts + 32 * hf <= w_last) compute_step(ts + 32 * hf, cur + hf * L::BUF, pa[hf] >= 0, pb[hf] >= 0);
      if constexpr (FMT != PKV_FMT_BF16) {
        if (more) {
#pragma unroll
          for (int hf = 0; hf < kHalves; ++hf)
            store_stage(ts1 + 32 * hf, pg[hf], st[hf], nxt + hf * L::BUF);
        }
      }
      __syncthreads();  // its fence waits for this thread's copies too
      if constexpr (FMT == PKV_FMT_BF16) {
        // the next block's page liveness (only the signs of the ids matter
        // from here on)
        const int bits = __builtin_amdgcn_readfirstlane(live_bits[(i + 1) & 1]);
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) {
          pg[hf].page_a = (bits >> (2 * hf)) & 1 ? 0 : -1;
          pg[hf].page_b = (bits >> (2 * hf)) & 2 ? 0 : -1;
        }
        bool z = false;
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) z = z || needs_zeros(ts1 + 32 * hf, pg[hf]);
        if (more && z) {
#pragma unroll
          for (int hf = 0; hf < kHalves; ++hf)
            if (needs_zeros(ts1 + 32 * hf, pg[hf]))
              zero_dead_slots(ts1 + 32 * hf, pg[hf], nxt + hf * L::BUF);
          __syncthreads();
        }
      }
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        pa[hf] = pg[hf].page_a;
        pb[hf] = pg[hf].page_b;
      }
    };
    for (int i = 0; i < n_blocks; i += 2) {
      block(i, lds0, lds1);
      if (i + 1 < n_blocks) block(i + 1, lds1, lds0);
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
