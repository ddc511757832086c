// Matrix-core building blocks of the paged attention kernels: one 32-token
// step of K/V read in place from the pages into registers, the score tiles
// S^T = K Q^T and the accumulation O^T += V^T P^T, on
// v_mfma_f32_16x16x32_bf16.
//
// Operand layouts (checked on the hardware): A lane l holds row l % 16 and k
// slots 8 (l / 16) .. +7; B lane l holds column l % 16 and the same k slots;
// C lane l holds column l % 16 and rows 4 (l / 16) .. +3.  Below, n = l % 16
// and j = l / 16.  The 16 columns are query rows (heads of the GQA group, or
// (query position, head) pairs), so every K/V byte loaded serves all of them.
//
// Row r of score tile t (t = 0, 1) holds token 8 (r / 4) + 4t + r % 4 of the
// step: the accumulator lanes of k group j then hold tokens 8j .. 8j+7 in
// order, which are exactly the k slots their P.V B operand needs, so the
// softmax weights never move between lanes, and each lane's V operand is 8
// consecutive slots of one dim of the dim-major V slab (one 16-byte load, 8
// bytes for int8).
//
// Page reads are streamed once per call: non-temporal loads keep them from
// displacing other data in the caches (measured: +45% bandwidth on the
// 32k-token bf16 workload over plain loads).  Memory instructions, not only
// bytes, set the pace: every K load covers 64 contiguous bytes of each row it
// touches (int8 lanes load 16 codes at once, see kdim_of), and a step's 64
// per-token int8 scales arrive in one 4-byte load per lane and are handed to
// the lanes that need them by DPP row broadcasts.
#pragma once

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// log2 units a column's maximum may pass its reference maximum by before the
// reference moves and the running outputs are rescaled: weights taken against
// the reference stay below 2^8, and most steps skip the rescale.
constexpr float kRescaleSlack = 8.f;

template <int FMT, int D>
struct Step {
  static constexpr int NC = D / 32;  // 32-wide k chunks of the Q.K product
  static constexpr int ND = D / 16;  // 16-row dim tiles of the P.V product
  // K: one 16-byte load per (tile, load) = 8 bf16 values (one k chunk) or
  // 16 int8 codes (two k chunks); V: 8 tokens per dim tile
  static constexpr int NK = FMT == PKV_FMT_BF16 ? NC : D / 64;
  static constexpr int KPL = NC / NK;  // k chunks per K load
  using KT = uint4;
  using VT = typename std::conditional<FMT == PKV_FMT_BF16, uint4, uint2>::type;
  // the same bytes as raw 32-bit vectors, for non-temporal loads
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  using NKT = u32x4;
  using NVT = typename std::conditional<sizeof(VT) == 16, u32x4, u32x2>::type;
  KT k[2][NK];
  VT v[ND];
  // int8 only: lane 16j + x holds the K scale (x < 8) or V scale (x >= 8) of
  // token 8j + x % 8 of the step, so the 16-lane row j holds the scales of
  // the tokens its k group uses; step_scales broadcasts them along the row
  float sc;
  bool live_a, live_b;  // the step's first / second 16 tokens sit on a valid page
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

template <typename T, typename R>
__device__ __forceinline__ T stream_load(const char* p) {
  return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const R*>(p)));
}

// 4 int8 codes -> 4 bf16 (exact: an integer of at most 7 bits plus sign, so
// its bf16 is the upper half of its float).  One byte permute packs the
// upper halves of two floats (bytes 2-3 of the first, then of the second).
__device__ __forceinline__ uint2 codes_to_bf16(uint32_t w) {
  float f0 = (float)(int8_t)(w & 0xffu), f1 = (float)(int8_t)((w >> 8) & 0xffu);
  float f2 = (float)(int8_t)((w >> 16) & 0xffu), f3 = (float)(int8_t)(w >> 24);
  uint2 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  return r;
}

// The head dims that k slots 8j .. 8j+7 of Q.K chunk c stand for (the
// contraction may take the dims in any order, as long as K and Q agree).
// bf16: dims 32c + 8j .. +7, one 16-byte load of a K row per chunk.  int8:
// lane j's 16 consecutive codes 64 (c / 2) + 16j .. +15 come in one 16-byte
// load and serve chunks c and c + 1 (codes 0-7, then 8-15), so a K load
// instruction covers 64 contiguous bytes of each row it reads, as in bf16.
template <int FMT>
__device__ __forceinline__ int kdim_of(int c, int j) {
  return FMT == PKV_FMT_BF16 ? 32 * c + 8 * j : 64 * (c >> 1) + 16 * j + 8 * (c & 1);
}

// Write 4 consecutive outputs (bf16 rounded to nearest even, or f32).
__device__ __forceinline__ void store_out4(void* out, int q_bf16, int64_t oi, f32x4 r) {
  if (q_bf16) {
    const uint2 w = {f32_to_bf16_bits(r[0]) | (f32_to_bf16_bits(r[1]) << 16),
                     f32_to_bf16_bits(r[2]) | (f32_to_bf16_bits(r[3]) << 16)};
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + oi) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oi) = r;
  }
}

// Where one layer's pages of one KV head live.
struct PageSrc {
  const char* k;
  const char* v;
  const float* ks;  // int8 scales (null otherwise)
  const float* vs;
  int64_t layer_page0;
  int64_t slab_bytes;  // bytes of one (page, KV head) slab of K (or V)
  int n_kv_heads;
  int bs;
};

// The query group as the B operand of S^T = K Q^T: column n's query row
// (zeros where the column is unused), dims as kdim_of lays them out.
template <int FMT, int D>
__device__ __forceinline__ void load_q(bf16x8* qf, const uint16_t* qrow, bool used, int j) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    uint4 x = {0, 0, 0, 0};
    if (used) x = *reinterpret_cast<const uint4*>(qrow + kdim_of<FMT>(c, j));
    qf[c] = as_bf16x8(x);
  }
}

// Load one step.  page_a / page_b are the pages of the step's first and
// second 16 tokens (equal for pages of 32 tokens or more; slot0 is the
// step's first slot in page_a then); -1 = none.  Loads are unconditional: a
// half with no page reads page 0 of the layer instead and is masked by its
// live flag afterwards, so the compiler can keep the next step's loads in
// flight.
template <int FMT, int D, int BS>
__device__ __forceinline__ void load_step(Step<FMT, D>& r, const PageSrc& s, int page_a,
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
    // this lane's K row: token 8 * (n / 4) + 4 * tau + n % 4 of the step
    const int tok = 8 * (n >> 2) + 4 * tau + (n & 3);
    const bool on_b = BS == 16 && tok >= 16;
    const char* kb = s.k + (on_b ? slab_b : slab_a) * s.slab_bytes;
    const int row = BS == 16 ? (tok & 15) : slot0 + tok;
    // a load of 16 bytes stays inside one piece of the K layout (64 bytes
    // or more for these rows)
#pragma unroll
    for (int c = 0; c < S::NK; ++c)
      r.k[tau][c] = stream_load<typename S::KT, typename S::NKT>(
          kb + k_byte(row, kdim_of<FMT>(S::KPL * c, j) * ESZ, bs, D * ESZ));
  }
  // V operand: tokens 8j .. 8j+7 of dim 16 * dt + n
  const bool v_on_b = BS == 16 && j >= 2;
  const char* vb = s.v + (v_on_b ? slab_b : slab_a) * s.slab_bytes;
  const int col = BS == 16 ? 8 * (j & 1) : slot0 + 8 * j;
  const int voff = (n * bs + col) * ESZ;
#pragma unroll
  for (int dt = 0; dt < S::ND; ++dt)
    r.v[dt] = stream_load<typename S::VT, typename S::NVT>(vb + voff + 16 * dt * bs * ESZ);
  if (FMT == PKV_FMT_INT8) {
    const int x = 8 * j + (n & 7);  // token of this lane's scale
    const bool s_on_b = BS == 16 && x >= 16;
    const int slot = BS == 16 ? (x & 15) : slot0 + x;
    const float* sb = n < 8 ? s.ks : s.vs;
    r.sc = __builtin_nontemporal_load(sb + (s_on_b ? slab_b : slab_a) * bs + slot);
  }
}

// S^T tiles of a step: sacc[tau] row 4j + i = token 8j + 4 tau + i.
template <int FMT, int D>
__device__ __forceinline__ void step_scores(const Step<FMT, D>& r, const bf16x8* qf,
                                            f32x4 sacc[2]) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      bf16x8 ka;
      if constexpr (FMT == PKV_FMT_BF16) {
        ka = as_bf16x8(r.k[tau][c]);
      } else {
        // chunk c: codes 8 (c % 2) .. +7 of the lane's 16-code load c / 2
        const uint4& w = r.k[tau][c >> 1];
        const uint2 lo = codes_to_bf16(c & 1 ? w.z : w.x), hi = codes_to_bf16(c & 1 ? w.w : w.y);
        ka = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
      }
      sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[c], sacc[tau], 0, 0, 0);
    }
  }
}

// int8: the K and V scales of this lane's tokens 8j .. 8j+7, broadcast
// along the lane's 16-lane row (no LDS round trip).
template <int FMT, int D>
__device__ __forceinline__ void step_scales(const Step<FMT, D>& r, float ksc[8], float vsc[8]) {
  ksc[0] = row_bcast<0>(r.sc);
  ksc[1] = row_bcast<1>(r.sc);
  ksc[2] = row_bcast<2>(r.sc);
  ksc[3] = row_bcast<3>(r.sc);
  ksc[4] = row_bcast<4>(r.sc);
  ksc[5] = row_bcast<5>(r.sc);
  ksc[6] = row_bcast<6>(r.sc);
  ksc[7] = row_bcast<7>(r.sc);
  vsc[0] = row_bcast<8>(r.sc);
  vsc[1] = row_bcast<9>(r.sc);
  vsc[2] = row_bcast<10>(r.sc);
  vsc[3] = row_bcast<11>(r.sc);
  vsc[4] = row_bcast<12>(r.sc);
  vsc[5] = row_bcast<13>(r.sc);
  vsc[6] = row_bcast<14>(r.sc);
  vsc[7] = row_bcast<15>(r.sc);
}

// O^T += V^T P^T over the step (the caller rescales O^T first when a
// column's running maximum grew).  pb holds the weights of this lane's tokens
// 8j .. 8j+7 for its column.  With bf16 pages, dead slots
// (past the readable range or on a missing page) are zeroed through `keep`
// (one mask per 32-bit word of the V operand) when mask_v is set: they may
// hold NaN, and 0 * NaN would reach the sum.  int8 codes are finite and
// carry weight 0 there.
template <int FMT, int D>
__device__ __forceinline__ void step_pv(const Step<FMT, D>& r, bf16x8 pb, const uint32_t keep[4],
                                        f32x4* o) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    uint4 va;
    if constexpr (FMT == PKV_FMT_BF16) {
      va = uint4{r.v[dt].x & keep[0], r.v[dt].y & keep[1], r.v[dt].z & keep[2],
                 r.v[dt].w & keep[3]};
    } else {
      const uint2 lo = codes_to_bf16(r.v[dt].x), hi = codes_to_bf16(r.v[dt].y);
      va = uint4{lo.x, lo.y, hi.x, hi.y};
    }
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, o[dt], 0, 0, 0);
  }
}

// Word masks that zero the bf16 V slots of tokens 8j + x with ok[x] false.
__device__ __forceinline__ void v_keep_masks(const bool ok[8], uint32_t keep[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w)
    keep[w] = (ok[2 * w] ? 0x0000ffffu : 0u) | (ok[2 * w + 1] ? 0xffff0000u : 0u);
}

}  // namespace pkv
