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
// One workgroup (one wave) handles a window of 16 slots of one KV head of one
// layer (grid z: several layers in one launch, each layer's rows following
// the previous layer's in k_in / v_in).  A prefill write's windows are
// aligned to the sequence's positions: window w of sequence b covers
// positions 16 * (floor(start_pos[b] / 16) + w) .. +15, so with page sizes
// that are multiples of 16 a window is 16 consecutive slots of one page, and
// only the first and last window of a sequence are partly filled.  Sequence
// b's windows are grid blocks floor(cu_new[b] / 16) + 2b onwards (that range
// holds at least floor(n / 16) + 2 >= ceil((start % 16 + n) / 16) windows for
// n rows), so a block finds its sequence by one binary search over cu_new.
// A decode write (one row per sequence) takes 16 sequences per window.
//
// Every input load is issued first, into registers, so the rows are in
// flight while the slot metadata (table entry) is worked out.  K goes out of
// registers as slot rows of head_dim (a bit copy, or int8 codes); V is
// transposed through LDS into the dim-major slab, each dim's run of 8 (bf16,
// int8) or 4 (f32) consecutive aligned slots of one page stored as one
// vector where the window's rows allow it.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRows = 16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RowMeta {
  int64_t k_off;  // element offset of the row's K slab, -1 = skip
  int slot;       // the row's slot in its page
  int64_t v_off;  // element offset of (dim 0, slot) in the V slab
  int64_t s_off;  // scale index (slab * page_size + slot)
};

// Whether window rows rr0 .. rr0+n-1 go to consecutive slots of one page,
// the first slot a multiple of n (so n slots of a V dim row are one aligned
// vector), with n dividing the page size.
__device__ __forceinline__ bool group_is_run(const RowMeta* meta, int rr0, int n, int bs) {
  if (bs % n != 0) return false;
  const RowMeta m0 = meta[rr0];
  if (m0.k_off < 0 || (m0.s_off % bs) % n != 0) return false;
  for (int i = 1; i < n; ++i)
    if (meta[rr0 + i].k_off < 0 || meta[rr0 + i].v_off != m0.v_off + i) return false;
  return true;
}

// Where the row of sequence b at position t goes, or k_off = -1 when the
// position has no page (reported in the status word).
__device__ __forceinline__ RowMeta slot_meta(const WriteArgs& a, int b, int t, int h,
                                             int64_t layer_page0) {
  RowMeta m{-1, 0, 0, 0};
  const int j = t >= 0 ? t / a.page_size : -1;
  if (t < 0 || j >= a.table_stride) {
    report(a.status, PKV_DEV_WRITE_TABLE);
    return m;
  }
  const int page = a.table[(int64_t)b * a.table_stride + j];
  if (page < 0 || page >= a.n_pages) {
    report(a.status, PKV_DEV_WRITE_PAGE);
    return m;
  }
  const int slot = t - j * a.page_size;
  const int64_t slab = (layer_page0 + page) * a.n_kv_heads + h;
  m.k_off = slab * a.page_size * a.head_dim;
  m.slot = slot;
  m.v_off = slab * a.page_size * a.head_dim + slot;
  m.s_off = slab * a.page_size + slot;
  return m;
}

// int8 codes of one row: code = clamp(rint(x / s), -127, 127), the quotient
// one IEEE float32 division rounded to nearest even, 0 when s = 0.
__device__ __forceinline__ uint32_t int8_code_exact(float x, float s) {
  if (s == 0.f) return 0u;
  const float c = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.f), 127.f);
  return (uint32_t)(int32_t)c & 0xffu;
}

// Element e of a 16-byte input vector as a float (bf16 or f32 rows).
template <int IN_BF16>
__device__ __forceinline__ float elem(const u32x4& x, int e) {
  const uint32_t w = x[IN_BF16 ? e >> 1 : e];
  if (IN_BF16) return __uint_as_float(e & 1 ? w & 0xffff0000u : w << 16);
  return __uint_as_float(w);
}

// Codes of the EPV elements of one 16-byte input vector, packed 4 to a word
// (element e in byte e % 4 of word e / 4).  Fast form: |x / s| <= 127.00002
// for s = fl(max|x| / 127), and x * r with r = rcp(s) (within 1 ulp) lies
// within 2.3e-5 of x / s, which is within 3.9e-6 of its float32 rounding; so
// unless x * r is within 2^-14 (6.1e-5) of a half-integer it rounds to the
// same integer as the correctly rounded quotient, and needs no clamp.  An
// element near a tie or with a non-finite product, and every element when
// s = 0 or s < 2^-100 (where rcp may overflow), takes the correctly rounded
// division instead.
template <int IN_BF16>
__device__ __forceinline__ void vector_codes(const u32x4& x, float s, uint32_t* out) {
  constexpr int EPV = IN_BF16 ? 8 : 4;
  const float r = __builtin_amdgcn_rcpf(s);
  const bool all_exact = !(s >= 0x1p-100f);
  uint32_t redo = 0;  // bit e: element e needs the correctly rounded division
#pragma unroll
  for (int w = 0; w < EPV / 4; ++w) {
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // q + 1.5 * 2^23 rounds q to an integer (nearest even) held in the
      // low mantissa bits, so its low byte is the two's-complement code
      const float q = elem<IN_BF16>(x, 4 * w + e) * r;
      const float m = q + 0x1.8p23f;
      if (all_exact || !(fabsf(q - (m - 0x1.8p23f)) < 0.5f - 0x1p-14f)) redo |= 1u << (4 * w + e);
      packed |= (__float_as_uint(m) & 0xffu) << (8 * e);
    }
    out[w] = packed;
  }
  if (redo) {
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      if (redo & (1u << e)) {
        const uint32_t sh = 8 * (e & 3);
        out[e >> 2] = (out[e >> 2] & ~(0xffu << sh)) | (int8_code_exact(elem<IN_BF16>(x, e), s) << sh);
      }
  }
}

// NIT: 16-byte input vectors per lane per tensor (16 rows x head_dim / 64
// lanes, rounded up to a power of two).
template <int FMT, int IN_BF16, int NIT>
__global__ __launch_bounds__(64) void write_kernel(WriteArgs a) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ RowMeta meta[kRows];
  __shared__ uint32_t rmax[2][kRows];
  constexpr int EPV = IN_BF16 ? 8 : 4;  // input elements per 16-byte vector
  const int D = a.head_dim;
  const int vpr = D / EPV;
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t layer_page0 = a.layer_page0 + (int64_t)blockIdx.z * a.n_pages;
  const int64_t in_row0 = (int64_t)blockIdx.z * a.total_new;  // this layer's rows in k_in/v_in

  // ---- the window: sequence, position and input row of slot 0, used slots ----
  int b = 0, t0 = 0, i0, lo = 0, hi = kRows;
  if (a.decode_lens) {
    i0 = blockIdx.x * kRows;  // slot rr is sequence i0 + rr's newest row
    hi = min(kRows, a.total_new - i0);
  } else {
    const int x = blockIdx.x;
    int l = 0, u = a.batch - 1;  // largest b with floor(cu_new[b] / 16) + 2b <= x
    while (l < u) {
      const int mid = (l + u + 1) >> 1;
      if ((a.cu_new[mid] >> 4) + 2 * mid <= x) l = mid; else u = mid - 1;
    }
    b = l;
    const int c0 = a.cu_new[b], c1 = a.cu_new[b + 1], s = a.start_pos[b];
    if (c0 < 0 || c1 < c0 || c1 > a.total_new) {
      if (lane == 0) report(a.status, PKV_DEV_WRITE_ROWS);
      return;
    }
    t0 = (s & ~(kRows - 1)) + kRows * (x - ((c0 >> 4) + 2 * b));
    lo = max(s - t0, 0);
    hi = min(s + (c1 - c0) - t0, kRows);
    i0 = c0 + (t0 - s);
  }
  if (lo >= hi) return;  // an unused window (uniform over the block)

  // ---- vector it of a lane is vector lane + 64 it of the window: row rr_[it],
  // elements d0_[it] .. +EPV-1 (one division, then carries) ----
  int rr_[NIT], d0_[NIT];
  {
    int rr = lane / vpr, dd = lane - rr * vpr;
    const int q64 = 64 / vpr, r64 = 64 - q64 * vpr;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      rr_[it] = rr;
      d0_[it] = dd * EPV;
      dd += r64;
      rr += q64;
      if (dd >= vpr) {
        dd -= vpr;
        ++rr;
      }
    }
  }
  // ---- every input load first (indexes clamped in bounds; extras unused) ----
  // (byte offsets from the window's slot-0 row, which may lie before the
  // rows: only clamped rows are read)
  u32x4 kx[NIT], vx[NIT];
  {
    constexpr int esz = IN_BF16 ? 2 : 4;
    const int row_bytes = a.n_kv_heads * D * esz;
    const int64_t base = (((in_row0 + i0) * a.n_kv_heads + h) * D) * esz;
    const char* kb = static_cast<const char*>(a.k_in) + base;
    const char* vb = static_cast<const char*>(a.v_in) + base;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = min(rr_[it], kRows - 1), d0 = rr_[it] < kRows ? d0_[it] : 0;
      const int r = min(max(i0 + rr, 0), a.total_new - 1);
      const int off = (r - i0) * row_bytes + d0 * esz;
      kx[it] = *reinterpret_cast<const u32x4*>(kb + off);
      vx[it] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  }
  if (lane < kRows) {
    RowMeta m{-1, 0, 0};
    if (lane >= lo && lane < hi) {
      if (a.decode_lens) {
        const int bb = i0 + lane;
        const int t = a.decode_lens[bb] - 1;  // none if the length is 0
        if (t >= 0) m = slot_meta(a, bb, t, h, layer_page0);
      } else {
        m = slot_meta(a, b, t0 + lane, h, layer_page0);
      }
    }
    meta[lane] = m;
  }
  if (FMT == PKV_FMT_INT8 && lane < 2 * kRows) rmax[lane / kRows][lane % kRows] = 0u;

  if constexpr (FMT != PKV_FMT_INT8) {
    // ---- native: bit copy ----
    constexpr int OESZ = FMT == PKV_FMT_F32 ? 4 : 2;
    // V rows staged row-major as raw bits, pitch pw words (16-byte aligned)
    const int pw = D * OESZ / 4 + 4;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = rr_[it], d0 = d0_[it];
      if (rr < kRows) {
        *reinterpret_cast<u32x4*>(smem + rr * pw + d0 * OESZ / 4) = vx[it];
      }
    }
    __syncthreads();
    // K: slot rows straight from registers
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = rr_[it], d0 = d0_[it];
      if (rr < kRows) {
        const int64_t k_off = meta[rr].k_off;
        if (k_off >= 0)  // 16 bytes: inside one 64-byte piece where K rows are pieced
          *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_pages) + k_off * OESZ +
                                    k_byte(meta[rr].slot, d0 * OESZ, a.page_size, D * OESZ)) =
              kx[it];
      }
    }
    // V: groups of GV rows.  A group whose rows are consecutive slots of one
    // page from an aligned slot stores each dim as one 16-byte vector;
    // otherwise each row's element goes out on its own.
    constexpr int GV = 16 / OESZ;
    constexpr int NG = kRows / GV;
    const int gi = lane % NG, rr0 = gi * GV;
    const bool packed = group_is_run(meta, rr0, GV, a.page_size);
    const int64_t bs = a.page_size;
    if constexpr (OESZ == 2) {
      // word column c holds dims 2c (low half) and 2c+1 (high half)
      for (int c = lane / NG; c < D / 2; c += 64 / NG) {
        uint32_t w[GV];
#pragma unroll
        for (int i = 0; i < GV; ++i) w[i] = smem[(rr0 + i) * pw + c];
        if (packed) {
          uint4 lo4, hi4;
          lo4.x = (w[0] & 0xffffu) | (w[1] << 16);
          lo4.y = (w[2] & 0xffffu) | (w[3] << 16);
          lo4.z = (w[4] & 0xffffu) | (w[5] << 16);
          lo4.w = (w[6] & 0xffffu) | (w[7] << 16);
          hi4.x = (w[0] >> 16) | (w[1] & 0xffff0000u);
          hi4.y = (w[2] >> 16) | (w[3] & 0xffff0000u);
          hi4.z = (w[4] >> 16) | (w[5] & 0xffff0000u);
          hi4.w = (w[6] >> 16) | (w[7] & 0xffff0000u);
          uint16_t* dst = static_cast<uint16_t*>(a.v_pages) + meta[rr0].v_off + 2 * c * bs;
          *reinterpret_cast<uint4*>(dst) = lo4;
          *reinterpret_cast<uint4*>(dst + bs) = hi4;
        } else {
#pragma unroll
          for (int i = 0; i < GV; ++i) {
            const RowMeta m = meta[rr0 + i];
            if (m.k_off < 0) continue;
            uint16_t* dst = static_cast<uint16_t*>(a.v_pages) + m.v_off + 2 * c * bs;
            dst[0] = (uint16_t)(w[i] & 0xffffu);
            dst[bs] = (uint16_t)(w[i] >> 16);
          }
        }
      }
    } else {
      for (int d = lane / NG; d < D; d += 64 / NG) {
        uint32_t w[GV];
#pragma unroll
        for (int i = 0; i < GV; ++i) w[i] = smem[(rr0 + i) * pw + d];
        if (packed) {
          *reinterpret_cast<uint4*>(static_cast<uint32_t*>(a.v_pages) + meta[rr0].v_off + d * bs) =
              uint4{w[0], w[1], w[2], w[3]};
        } else {
#pragma unroll
          for (int i = 0; i < GV; ++i) {
            const RowMeta m = meta[rr0 + i];
            if (m.k_off >= 0) static_cast<uint32_t*>(a.v_pages)[m.v_off + d * bs] = w[i];
          }
        }
      }
    }
  } else {
    // ---- int8: per (row, head) scale = max|x| / 127, then codes ----
    // Row maxima through LDS atomics on the float bits (non-negative floats
    // order like their bit patterns); fmaxf drops NaN inputs from the max.
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = rr_[it];
      if (rr < kRows) {
        float mk = 0.f, mv = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          mk = fmaxf(mk, fabsf(elem<IN_BF16>(kx[it], e)));
          mv = fmaxf(mv, fabsf(elem<IN_BF16>(vx[it], e)));
        }
        atomicMax(&rmax[0][rr], __float_as_uint(mk));
        atomicMax(&rmax[1][rr], __float_as_uint(mv));
      }
    }
    __syncthreads();
    // scales once per row, kept in LDS (rmax's words) for the codes
    if (lane < 2 * kRows) {
      const int rr = lane % kRows, kv = lane / kRows;
      const float sc = __fdiv_rn(__uint_as_float(rmax[kv][rr]), 127.0f);
      const RowMeta m = meta[rr];
      if (m.k_off >= 0) (kv ? a.v_scales : a.k_scales)[m.s_off] = sc;
      rmax[kv][rr] = __float_as_uint(sc);
    }
    __syncthreads();
    // K codes straight to the slot rows; V codes row-major into LDS (pitch
    // D + 8 bytes) for the transpose
    const int pb = D + 8;
    uint8_t* cv = reinterpret_cast<uint8_t*>(smem);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = rr_[it], d0 = d0_[it];
      if (rr < kRows) {
        uint32_t kc[EPV / 4], vc[EPV / 4];
        vector_codes<IN_BF16>(kx[it], __uint_as_float(rmax[0][rr]), kc);
        vector_codes<IN_BF16>(vx[it], __uint_as_float(rmax[1][rr]), vc);
        const int64_t k_off = meta[rr].k_off;
        int8_t* dst = static_cast<int8_t*>(a.k_pages) + k_off +
                      k_byte(meta[rr].slot, d0, a.page_size, D);
        if constexpr (EPV == 8) {
          if (k_off >= 0) *reinterpret_cast<uint2*>(dst) = uint2{kc[0], kc[EPV / 4 - 1]};
          *reinterpret_cast<uint2*>(cv + rr * pb + d0) = uint2{vc[0], vc[EPV / 4 - 1]};
        } else {
          if (k_off >= 0) *reinterpret_cast<uint32_t*>(dst) = kc[0];
          *reinterpret_cast<uint32_t*>(cv + rr * pb + d0) = vc[0];
        }
      }
    }
    __syncthreads();
    // V: a lane takes 4 dims of a group of 8 rows: 8 words (4 codes of one
    // row each) byte-transposed into 4 dims x 8 rows.  A group in consecutive
    // aligned slots of one page stores each dim's 8 codes as one 8-byte
    // vector, otherwise one code byte per (dim, slot).
    const int g = lane & 1, rr0 = 8 * g;
    const bool packed = group_is_run(meta, rr0, 8, a.page_size);
    const int64_t bs = a.page_size;
    for (int dq = lane >> 1; dq < D / 4; dq += 32) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = *reinterpret_cast<const uint32_t*>(cv + (rr0 + i) * pb + 4 * dq);
      // per half (rows 0-3, 4-7): t0 = bytes 0,1 of rows (0,1) interleaved,
      // t1 = bytes 2,3 of rows (0,1), t2/t3 the same for rows (2,3); then dim
      // j's word gathers byte j of the four rows
      uint32_t dimw[2][4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t* a4 = w + 4 * hf;
        const uint32_t t0 = __builtin_amdgcn_perm(a4[1], a4[0], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(a4[1], a4[0], 0x07030602u);
        const uint32_t t2 = __builtin_amdgcn_perm(a4[3], a4[2], 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(a4[3], a4[2], 0x07030602u);
        dimw[hf][0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
        dimw[hf][1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
        dimw[hf][2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
        dimw[hf][3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
      }
      if (packed) {
        uint8_t* dst = static_cast<uint8_t*>(a.v_pages) + meta[rr0].v_off + 4 * dq * bs;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(dst + j * bs) = uint2{dimw[0][j], dimw[1][j]};
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const RowMeta m = meta[rr0 + i];
          if (m.k_off < 0) continue;
          uint8_t* dst = static_cast<uint8_t*>(a.v_pages) + m.v_off + 4 * dq * bs;
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[j * bs] = (uint8_t)(w[i] >> (8 * j));
        }
      }
    }
  }
}

template <int FMT, int IN_BF16>
hipError_t launch_fmt(const WriteArgs& a, dim3 grid, const Launch& l) {
  constexpr int EPV = IN_BF16 ? 8 : 4;
  const int per_lane = (kRows * (a.head_dim / EPV) + 63) / 64;
  const int shm_native = kRows * (a.head_dim * (FMT == PKV_FMT_F32 ? 4 : 2) / 4 + 4) * 4;
  const size_t shm = FMT == PKV_FMT_INT8 ? (size_t)kRows * (a.head_dim + 8) : (size_t)shm_native;
  if (per_lane <= 1) return launch1(write_kernel<FMT, IN_BF16, 1>, grid, dim3(64), shm, l, a);
  if (per_lane <= 2) return launch1(write_kernel<FMT, IN_BF16, 2>, grid, dim3(64), shm, l, a);
  if (per_lane <= 4) return launch1(write_kernel<FMT, IN_BF16, 4>, grid, dim3(64), shm, l, a);
  if (per_lane <= 8) return launch1(write_kernel<FMT, IN_BF16, 8>, grid, dim3(64), shm, l, a);
  if (!IN_BF16 && per_lane <= 16)
    return launch1(write_kernel<FMT, IN_BF16, IN_BF16 ? 8 : 16>, grid, dim3(64), shm, l, a);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, int fmt, int in_dtype, const Launch& l) {
  if (a.total_new <= 0) return hipSuccess;
  // prefill: floor(total_new / 16) + 2 * batch position-aligned windows;
  // decode: one window per 16 sequences
  const int64_t windows = a.decode_lens ? (a.total_new + kRows - 1) / kRows
                                        : (int64_t)a.total_new / kRows + 2 * (int64_t)a.batch;
  if (windows > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)windows, a.n_kv_heads, a.n_layers_w);
  if (fmt == PKV_FMT_F32) return launch_fmt<PKV_FMT_F32, 0>(a, grid, l);
  if (fmt == PKV_FMT_BF16) return launch_fmt<PKV_FMT_BF16, 1>(a, grid, l);
  if (in_dtype == PKV_DT_BF16) return launch_fmt<PKV_FMT_INT8, 1>(a, grid, l);
  return launch_fmt<PKV_FMT_INT8, 0>(a, grid, l);
}

}  // namespace pkv
