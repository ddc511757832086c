// Gather: copy one sequence's first `len` rows out of its pages into a
// contiguous token-major [len][n_kv_heads][head_dim] buffer (AstrAI
// inference/cache.py PagedCache.gather truncated by CacheView.gather;
// libmir-metal src/engine/kv/paged/mod.rs PagedStore::context).  It exists to
// compare the in-place attention read against a gather-first one.  int8
// pages give their raw codes and per-(token, KV head) scales.
//
// One workgroup (one wave) copies 16 tokens of one KV head: K rows with
// 16-byte vectors, V by reading the dim-major slab (consecutive lanes read
// consecutive slots) through an LDS transpose.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kTok = 16;

template <int ESZ>
__global__ __launch_bounds__(64) void gather_kernel(GatherArgs a) {
  extern __shared__ uint32_t sv[];  // [kTok][D + 1] words
  __shared__ int64_t slab_off[kTok];  // element offset of the slot's (page, head) slab, -1 = none
  __shared__ int slot_of[kTok];
  const int D = a.head_dim, ld = D + 1;
  const int lane = threadIdx.x, h = blockIdx.y;
  const int t0 = blockIdx.x * kTok;
  if (lane < kTok) {
    int64_t off = -1;
    int slot = 0;
    const int t = t0 + lane;
    if (t < a.len) {
      const int j = t / a.page_size;
      const int page = a.table_row[j];
      if (page < 0 || page >= a.n_pages) {
        report(a.status, PKV_DEV_READ_PAGE);
      } else {
        slot = t - j * a.page_size;
        off = ((a.layer_page0 + page) * a.n_kv_heads + h) * a.page_size * D;
      }
    }
    slab_off[lane] = off;
    slot_of[lane] = slot;
  }
  __syncthreads();

  // K: slot row -> output row, 16-byte vectors (zeros for a skipped page)
  {
    constexpr int EPV = 16 / ESZ;
    const int vpr = D / EPV;
    for (int vi = lane; vi < kTok * vpr; vi += 64) {
      const int r = vi / vpr, d0 = (vi - r * vpr) * EPV;
      const int t = t0 + r;
      if (t >= a.len) continue;
      uint4 x = {0, 0, 0, 0};
      if (slab_off[r] >= 0) {
        const int64_t e = slab_off[r] + (int64_t)slot_of[r] * D + d0;
        x = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_pages) + e * ESZ);
      }
      const int64_t o = ((int64_t)t * a.n_kv_heads + h) * D + d0;
      *reinterpret_cast<uint4*>(static_cast<char*>(a.k_out) + o * ESZ) = x;
    }
  }
  // V: dim-major slab -> LDS [token][dim] -> output rows
  {
    const int r = lane & (kTok - 1);
    for (int d = lane >> 4; d < D; d += 4) {
      uint32_t w = 0;
      if (t0 + r < a.len && slab_off[r] >= 0) {
        const int64_t e = slab_off[r] + (int64_t)d * a.page_size + slot_of[r];
        if (ESZ == 4) w = static_cast<const uint32_t*>(a.v_pages)[e];
        else if (ESZ == 2) w = static_cast<const uint16_t*>(a.v_pages)[e];
        else w = static_cast<const uint8_t*>(a.v_pages)[e];
      }
      sv[r * ld + d] = w;
    }
  }
  __syncthreads();
  {
    constexpr int EPW = 4 / ESZ;  // elements per 32-bit output word
    const int wpr = D / EPW;
    for (int wi = lane; wi < kTok * wpr; wi += 64) {
      const int r = wi / wpr, d0 = (wi - r * wpr) * EPW;
      const int t = t0 + r;
      if (t >= a.len) continue;
      const uint32_t* s = sv + r * ld + d0;
      uint32_t w;
      if (ESZ == 4) w = s[0];
      else if (ESZ == 2) w = s[0] | (s[1] << 16);
      else w = s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24);
      const int64_t o = ((int64_t)t * a.n_kv_heads + h) * D + d0;
      *reinterpret_cast<uint32_t*>(static_cast<char*>(a.v_out) + o * ESZ) = w;
    }
  }
  // int8 scales
  if (ESZ == 1 && lane < kTok) {
    const int t = t0 + lane;
    if (t < a.len) {
      float ks = 0.f, vs = 0.f;
      if (slab_off[lane] >= 0) {
        const int64_t si = slab_off[lane] / D + slot_of[lane];
        ks = a.k_scales[si];
        vs = a.v_scales[si];
      }
      a.ks_out[(int64_t)t * a.n_kv_heads + h] = ks;
      a.vs_out[(int64_t)t * a.n_kv_heads + h] = vs;
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int fmt, const Launch& l) {
  if (a.len <= 0) return hipSuccess;
  dim3 grid((a.len + kTok - 1) / kTok, a.n_kv_heads);
  const size_t shm = kTok * (a.head_dim + 1) * sizeof(uint32_t);
  if (fmt == PKV_FMT_F32) return launch1(gather_kernel<4>, grid, dim3(64), shm, l, a);
  if (fmt == PKV_FMT_BF16) return launch1(gather_kernel<2>, grid, dim3(64), shm, l, a);
  return launch1(gather_kernel<1>, grid, dim3(64), shm, l, a);
}

}  // namespace pkv
