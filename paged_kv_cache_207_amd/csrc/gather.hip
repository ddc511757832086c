// Gather: copy one sequence's first `len` rows out of its pages into a
// contiguous token-major [len][n_kv_heads][head_dim] buffer (AstrAI
// inference/cache.py PagedCache.gather truncated by CacheView.gather;
// libmir-metal src/engine/kv/paged/mod.rs PagedStore::context).  It exists to
// compare the in-place attention read against a gather-first one.  int8
// pages give their raw codes and per-(token, KV head) scales.
//
// One workgroup (one wave) copies 16 tokens of one KV head: K rows with
// 16-byte vectors; V through an LDS transpose.  When the 16 tokens are 16
// consecutive slots of one page (page sizes that are multiples of 16, the
// usual case), each dim's run of slots is read as 16-byte vectors and
// scattered into token rows in LDS, which then go out as 16-byte vectors;
// otherwise each slot's element is read on its own.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kTok = 16;

template <int ESZ>
__global__ __launch_bounds__(64) void gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) char srow[];  // [kTok][D * ESZ + 16] bytes: token rows of V
  __shared__ int64_t slab_off[kTok];  // element offset of the slot's (page, head) slab, -1 = none
  __shared__ int slot_of[kTok];
  const int D = a.head_dim;
  const int pitch = D * ESZ + 16;
  const int lane = threadIdx.x, h = blockIdx.y;
  const int t0 = blockIdx.x * kTok;
  const int n_tok = min(kTok, a.len - t0);
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
      if (slab_off[r] >= 0) {  // 16 bytes: inside one 64-byte piece where rows are pieced
        const int64_t byte = slab_off[r] * ESZ + k_byte(slot_of[r], d0 * ESZ, a.page_size,
                                                        D * ESZ);
        x = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_pages) + byte);
      }
      const int64_t o = ((int64_t)t * a.n_kv_heads + h) * D + d0;
      *reinterpret_cast<uint4*>(static_cast<char*>(a.k_out) + o * ESZ) = x;
    }
  }
  // V: dim-major slab -> LDS token rows -> output rows
  const bool run = n_tok == kTok && a.page_size % kTok == 0 && slab_off[0] >= 0 &&
                   slab_off[kTok - 1] == slab_off[0] && slot_of[0] % kTok == 0;  // uniform
  if (run) {
    constexpr int GS = 16 / ESZ;       // slots per 16-byte vector
    constexpr int NGS = kTok / GS;     // vectors per dim
    const char* vb = static_cast<const char*>(a.v_pages) +
                     (slab_off[0] + slot_of[0]) * ESZ;
    for (int task = lane; task < D * NGS; task += 64) {
      const int d = task / NGS, g = task - d * NGS;
      const uint4 x = *reinterpret_cast<const uint4*>(vb + ((int64_t)d * a.page_size + g * GS) * ESZ);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        char* dst = srow + (g * GS + i) * pitch + d * ESZ;
        const uint32_t word = w[(i * ESZ) >> 2];
        if (ESZ == 4) *reinterpret_cast<uint32_t*>(dst) = word;
        else if (ESZ == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(word >> (16 * (i & 1)));
        else *reinterpret_cast<uint8_t*>(dst) = (uint8_t)(word >> (8 * (i & 3)));
      }
    }
  } else {
    for (int task = lane; task < kTok * D; task += 64) {
      const int r = task & (kTok - 1), d = task / kTok;
      uint32_t w = 0;
      if (t0 + r < a.len && slab_off[r] >= 0) {
        const int64_t e = slab_off[r] + (int64_t)d * a.page_size + slot_of[r];
        if (ESZ == 4) w = static_cast<const uint32_t*>(a.v_pages)[e];
        else if (ESZ == 2) w = static_cast<const uint16_t*>(a.v_pages)[e];
        else w = static_cast<const uint8_t*>(a.v_pages)[e];
      }
      char* dst = srow + r * pitch + d * ESZ;
      if (ESZ == 4) *reinterpret_cast<uint32_t*>(dst) = w;
      else if (ESZ == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
      else *reinterpret_cast<uint8_t*>(dst) = (uint8_t)w;
    }
  }
  __syncthreads();
  {
    const int vpr = D * ESZ / 16;  // 16-byte vectors per token row
    for (int vi = lane; vi < n_tok * vpr; vi += 64) {
      const int r = vi / vpr, c = vi - r * vpr;
      const uint4 x = *reinterpret_cast<const uint4*>(srow + r * pitch + 16 * c);
      const int64_t o = ((int64_t)(t0 + r) * a.n_kv_heads + h) * D * ESZ + 16 * c;
      *reinterpret_cast<uint4*>(static_cast<char*>(a.v_out) + o) = x;
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
  const size_t shm = (size_t)kTok * (a.head_dim * format_bytes(fmt) + 16);
  if (fmt == PKV_FMT_F32) return launch1(gather_kernel<4>, grid, dim3(64), shm, l, a);
  if (fmt == PKV_FMT_BF16) return launch1(gather_kernel<2>, grid, dim3(64), shm, l, a);
  return launch1(gather_kernel<1>, grid, dim3(64), shm, l, a);
}

}  // namespace pkv
