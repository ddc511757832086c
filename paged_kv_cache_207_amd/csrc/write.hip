// Page write: scatter new K/V rows into their pages (bit copy for f32/bf16
// pages, per-(token, KV head) int8 quantization for int8 pages).
//
// Addressing (tiny-llm paged_kv.py, module docstring): row i of sequence b
// goes to position t = start_pos[b] + (i - cu_new[b]), page
// table[b][t / page_size], slot t % page_size; the chunked form of the same
// write is AstrAI inference/cache.py PagedCache.write.  Quantization: one
// scale per (token, KV head) row, the Int8PerTokenHead page format of
// libmir-metal src/engine/kv/paged/mod.rs, with scale = max|x| / 127 and
// codes rint(x / scale) clamped to +-127.
//
// One workgroup (one wave) handles 16 consecutive input rows of one KV head
// of one layer (grid z: several layers in one launch, each layer's rows
// following the previous layer's in k_in / v_in).
// The rows are staged in LDS as 32-bit words (bf16 bits widened to the
// float32 value's bits), then K is stored as slot rows of head_dim (16-byte
// vector stores) and V as the dim-major slab (for each dim, consecutive
// lanes store consecutive slots of a page).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRows = 16;

struct RowMeta {
  int64_t k_off;  // element offset of the row's K slot row, -1 = skip
  int64_t v_off;  // element offset of (dim 0, slot) in the V slab
  int64_t s_off;  // scale index (slab * page_size + slot)
};

template <int FMT, int IN_BF16>
__global__ __launch_bounds__(64) void write_kernel(WriteArgs a) {
  extern __shared__ uint32_t smem[];
  const int D = a.head_dim;
  const int ld = D + 1;  // padded row pitch in words
  uint32_t* sk = smem;
  uint32_t* sv = smem + kRows * ld;
  __shared__ RowMeta meta[kRows];
  __shared__ float sscale[2][kRows];

  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kRows;
  const int64_t layer_page0 = a.layer_page0 + (int64_t)blockIdx.z * a.n_pages;
  const int64_t in_row0 = (int64_t)blockIdx.z * a.total_new;  // this layer's rows in k_in/v_in

  // ---- row metadata: sequence, position, page, slot ----
  if (lane < kRows) {
    RowMeta m{-1, 0, 0};
    const int r = row0 + lane;
    int b = -1, t = -1;
    if (a.decode_lens && r < a.total_new) {
      // decode step: row r is sequence r's newest token (none if its length is 0)
      b = r;
      t = a.decode_lens[b] - 1;
      if (t < 0) b = -1;
    } else if (r < a.total_new) {
      // largest b with cu_new[b] <= r, kept inside [0, batch-1]
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a.cu_new[mid] <= r) lo = mid; else hi = mid - 1;
      }
      b = lo;
      t = a.start_pos[b] + (r - a.cu_new[b]);
    }
    if (b >= 0) {
      const int j = t >= 0 ? t / a.page_size : -1;
      if (t < 0 || j >= a.table_stride) {
        report(a.status, PKV_DEV_WRITE_TABLE);
      } else {
        const int page = a.table[(int64_t)b * a.table_stride + j];
        if (page < 0 || page >= a.n_pages) {
          report(a.status, PKV_DEV_WRITE_PAGE);
        } else {
          const int slot = t - j * a.page_size;
          const int64_t slab = (layer_page0 + page) * a.n_kv_heads + h;
          m.k_off = (slab * a.page_size + slot) * D;
          m.v_off = slab * a.page_size * D + slot;
          m.s_off = slab * a.page_size + slot;
        }
      }
    }
    meta[lane] = m;
  }

  // ---- stage the 16 rows of K and V (this head) in LDS as 32-bit words ----
  {
    constexpr int EPV = IN_BF16 ? 8 : 4;  // elements per 16-byte vector
    const int vpr = D / EPV;
    for (int vi = lane; vi < kRows * vpr; vi += 64) {
      const int rr = vi / vpr, d0 = (vi - rr * vpr) * EPV;
      const int r = row0 + rr;
      uint4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (r < a.total_new) {
        const int64_t e = ((in_row0 + r) * a.n_kv_heads + h) * D + d0;
        const int esz = IN_BF16 ? 2 : 4;
        kx = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_in) + e * esz);
        vx = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_in) + e * esz);
      }
      uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w}, vw[4] = {vx.x, vx.y, vx.z, vx.w};
      uint32_t* dk = sk + rr * ld + d0;
      uint32_t* dv = sv + rr * ld + d0;
      if (IN_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dk[2 * i] = kw[i] << 16;
          dk[2 * i + 1] = kw[i] & 0xffff0000u;
          dv[2 * i] = vw[i] << 16;
          dv[2 * i + 1] = vw[i] & 0xffff0000u;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dk[i] = kw[i];
          dv[i] = vw[i];
        }
      }
    }
  }
  __syncthreads();

  if (FMT != PKV_FMT_INT8) {
    // ---- native: bit copy ----
    constexpr int OESZ = FMT == PKV_FMT_F32 ? 4 : 2;
    constexpr int OEPV = 16 / OESZ;
    const int vpr = D / OEPV;
    for (int vi = lane; vi < kRows * vpr; vi += 64) {
      const int rr = vi / vpr, d0 = (vi - rr * vpr) * OEPV;
      const RowMeta m = meta[rr];
      if (m.k_off < 0) continue;
      const uint32_t* src = sk + rr * ld + d0;
      uint4 o;
      if (OESZ == 2) {
        o.x = (src[0] >> 16) | (src[1] & 0xffff0000u);
        o.y = (src[2] >> 16) | (src[3] & 0xffff0000u);
        o.z = (src[4] >> 16) | (src[5] & 0xffff0000u);
        o.w = (src[6] >> 16) | (src[7] & 0xffff0000u);
      } else {
        o = {src[0], src[1], src[2], src[3]};
      }
      *reinterpret_cast<uint4*>(static_cast<char*>(a.k_pages) + (m.k_off + d0) * OESZ) = o;
    }
    const int rr = lane & (kRows - 1);
    const RowMeta m = meta[rr];
    if (m.k_off >= 0) {
      for (int d = lane >> 4; d < D; d += 4) {
        const uint32_t w = sv[rr * ld + d];
        const int64_t e = m.v_off + (int64_t)d * a.page_size;
        if (OESZ == 2)
          static_cast<uint16_t*>(a.v_pages)[e] = (uint16_t)(w >> 16);
        else
          static_cast<uint32_t*>(a.v_pages)[e] = w;
      }
    }
  } else {
    // ---- int8: per (row, head) scale, then codes ----
    {
      const int rr = lane >> 2, part = lane & 3;
      float mk = 0.f, mv = 0.f;
      for (int d = part; d < D; d += 4) {
        mk = fmaxf(mk, fabsf(__uint_as_float(sk[rr * ld + d])));
        mv = fmaxf(mv, fabsf(__uint_as_float(sv[rr * ld + d])));
      }
      mk = fmaxf(mk, __shfl_xor(mk, 1, 64));
      mk = fmaxf(mk, __shfl_xor(mk, 2, 64));
      mv = fmaxf(mv, __shfl_xor(mv, 1, 64));
      mv = fmaxf(mv, __shfl_xor(mv, 2, 64));
      const float s_k = __fdiv_rn(mk, 127.0f);
      const float s_v = __fdiv_rn(mv, 127.0f);
      if (part == 0) {
        sscale[0][rr] = s_k;
        sscale[1][rr] = s_v;
        const RowMeta m = meta[rr];
        if (m.k_off >= 0) {
          a.k_scales[m.s_off] = s_k;
          a.v_scales[m.s_off] = s_v;
        }
      }
    }
    __syncthreads();
    auto code = [](float x, float s) -> uint32_t {
      if (s == 0.f) return 0u;
      float c = rintf(__fdiv_rn(x, s));
      c = fminf(fmaxf(c, -127.f), 127.f);
      return (uint32_t)(int32_t)c & 0xffu;
    };
    // K: slot rows of head_dim int8 codes, 4 codes per 32-bit store
    const int wpr = D / 4;
    for (int wi = lane; wi < kRows * wpr; wi += 64) {
      const int rr = wi / wpr, d0 = (wi - rr * wpr) * 4;
      const RowMeta m = meta[rr];
      if (m.k_off < 0) continue;
      const float s = sscale[0][rr];
      const uint32_t* src = sk + rr * ld + d0;
      uint32_t w = code(__uint_as_float(src[0]), s) | (code(__uint_as_float(src[1]), s) << 8) |
                   (code(__uint_as_float(src[2]), s) << 16) |
                   (code(__uint_as_float(src[3]), s) << 24);
      *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(a.k_pages) + m.k_off + d0) = w;
    }
    // V: dim-major slab, one code byte per (dim, slot)
    const int rr = lane & (kRows - 1);
    const RowMeta m = meta[rr];
    if (m.k_off >= 0) {
      const float s = sscale[1][rr];
      for (int d = lane >> 4; d < D; d += 4) {
        const int64_t e = m.v_off + (int64_t)d * a.page_size;
        static_cast<uint8_t*>(a.v_pages)[e] = (uint8_t)code(__uint_as_float(sv[rr * ld + d]), s);
      }
    }
  }
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, int fmt, int in_dtype, const Launch& l) {
  if (a.total_new <= 0) return hipSuccess;
  dim3 grid((a.total_new + kRows - 1) / kRows, a.n_kv_heads, a.n_layers_w);
  const size_t shm = 2 * kRows * (a.head_dim + 1) * sizeof(uint32_t);
  const bool bf = in_dtype == PKV_DT_BF16;
  if (fmt == PKV_FMT_F32)
    return launch1(write_kernel<PKV_FMT_F32, 0>, grid, dim3(64), shm, l, a);
  else if (fmt == PKV_FMT_BF16)
    return launch1(write_kernel<PKV_FMT_BF16, 1>, grid, dim3(64), shm, l, a);
  else if (bf)
    return launch1(write_kernel<PKV_FMT_INT8, 1>, grid, dim3(64), shm, l, a);
  else
    return launch1(write_kernel<PKV_FMT_INT8, 0>, grid, dim3(64), shm, l, a);
}

}  // namespace pkv
