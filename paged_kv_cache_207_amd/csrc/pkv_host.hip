// Host side of the C ABI: argument validation, the split-K planner, kernel
// launches, the refcounted page pool and the host block tables.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int check_layout(const pkv_layout* l) {
  if (!l) return fail(PKV_EINVAL, "layout is null");
  if (l->n_layers < 1 || l->n_pages < 1 || l->page_size < 1 || l->n_kv_heads < 1)
    return fail(PKV_EINVAL, "layout sizes must be positive");
  if (l->head_dim < 16 || l->head_dim > 256 || l->head_dim % 16)
    return fail(PKV_EINVAL, "head_dim must be a multiple of 16 in [16, 256], got %d", l->head_dim);
  if (l->format < PKV_FMT_F32 || l->format > PKV_FMT_INT8)
    return fail(PKV_EINVAL, "unknown page format %d", l->format);
  return PKV_OK;
}

int64_t gcd64(int64_t a, int64_t b) { return b ? gcd64(b, a % b) : a; }

// Split granularity: a multiple of 64 (the vector kernel's token tile) and of
// the page size (so a split never starts inside a page).
int64_t split_unit(int page_size) { return 64 / gcd64(64, page_size) * page_size; }

int plan_split(const pkv_cache* c, int batch, int n_q_heads, int max_len) {
  // Measured on the matrix-core path (persistent grid, work list): long
  // splits are best, 1024 tokens up to 16k-token bounds; beyond, 4096 for
  // bf16 pages (8 x 32k tokens: step 169.4-169.8 us against 170.9-172.7 with
  // 2048 and 198-200 with 8192, alternating runs on one MI355X) and 2048 for
  // the others, whose shorter steps need more waves streaming.  Halve while
  // the batch would give fewer than 512 (split, KV head) items, so a small
  // batch still spreads over the compute units.
  const int64_t unit = split_unit(c->L.page_size);
  int64_t split = max_len <= 16384 ? 1024 : c->L.format == PKV_FMT_BF16 ? 4096 : 2048;
  const int64_t heads = (int64_t)std::max(batch, 1) * c->L.n_kv_heads;
  while (split > 256 && heads * ((std::max(max_len, 1) + split - 1) / split) < 512) split /= 2;
  split = (split + unit - 1) / unit * unit;
  (void)n_q_heads;
  return (int)split;
}

// splits per sequence; the combine kernel keeps one weight per split in LDS
constexpr int kMaxSplits = 16384;

int check_split(const pkv_cache* c, int32_t split) {
  if (split < 0) return fail(PKV_EINVAL, "split_tokens must be >= 0");
  if (split > 0 && split % split_unit(c->L.page_size))
    return fail(PKV_EINVAL, "split_tokens %d must be a multiple of %lld", split,
                (long long)split_unit(c->L.page_size));
  return PKV_OK;
}

// Workspace: first a fixed region of split counters (one u32 per (sequence,
// KV head) for up to kMaxMfmaBatch sequences x kMaxMfmaKvHeads heads), then
// the partials o and (m, l) in f32, then the balanced schedule's record of
// the schedule it took (one i32, in its own 256 bytes) and its unit records
// (two i32 per (sequence, KV head)).  The partials region holds
// either schedule's rows: [B][Hq][S] for fixed splits, [B Hkv + waves][G]
// for the balanced one.  The counters must be zero before the first call
// and every call leaves them zero; their region does not move with the
// call's shape, so one zeroed workspace serves calls of any batch, length
// bound or split size.
constexpr uint64_t kCounterBytes = (uint64_t)pkv::kMaxMfmaBatch * pkv::kMaxMfmaKvHeads * 4;

// Compute units of the current device (256 when it cannot be asked).
int device_cus() {
  static thread_local int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
  }
  return cus;
}

// Balanced schedule: its wave bound per compute unit (0 = fixed splits) and
// the set-up cost of a (sequence, KV head) unit, in 32-token steps.
// Measured on one MI355X (split pass, µs, fixed splits -> balanced):
// bf16 pages with uneven lengths (32 sequences of 512-4096 tokens)
// 59.3 -> 54.7 at 4 waves per CU and a cost of 3 (1-8 and 3-5 waves per CU
// within 2 µs of it, 8 waves per CU no gain); 8 x 32k tokens 165.3 -> 165.6
// (the same partition as 2048-token splits).  int8 pages were never faster
// balanced (94.3 fixed, 96.3 at best, and up to 150 with cheap set-ups):
// their steps are short, and every extra cold start costs more than the
// balance gains.
constexpr int kMaxBalWavesPerCu = 4;
int bal_waves_per_cu(int fmt) { return fmt == PKV_FMT_BF16 ? kMaxBalWavesPerCu : 0; }
constexpr int kUnitCost = 3;

// Shared-prefix chunks: the target length, and the most one wave's page-id
// vector covers.
constexpr int kPrefixChunkTarget = 512;
constexpr int kPrefixChunkMax = 1024;

// Query heads per matrix-core group: G itself up to 16; above, the largest
// divisor of G that is at most 16 (each KV head then stands as G / that
// many groups), or 0 when that divisor is below 8 (the vector path takes
// the call).
int mfma_group(int G) {
  if (G <= 16) return G;
  for (int d = 16; d >= 8; --d)
    if (G % d == 0) return d;
  return 0;
}

struct WsLayout {
  uint64_t o_off, ml_off, sched_off, desc_off, total;
  uint64_t pre_o_off = 0, pre_ml_off = 0;  // shared-prefix partials (after the rest)
};

WsLayout ws_layout(const pkv_cache* c, int batch, int n_q_heads, int n_split) {
  WsLayout w;
  const int n_kv_heads = c->L.n_kv_heads, head_dim = c->L.head_dim;
  const uint64_t rows_split = (uint64_t)batch * n_q_heads * n_split;
  const uint64_t rows_bal =
      bal_waves_per_cu(c->L.format) > 0
          ? ((uint64_t)batch * n_kv_heads + (uint64_t)kMaxBalWavesPerCu * device_cus()) *
                (n_q_heads / std::max(n_kv_heads, 1))
          : 0;
  const uint64_t rows = std::max(rows_split, rows_bal);
  w.o_off = kCounterBytes;
  w.ml_off = (w.o_off + rows * head_dim * sizeof(float) + 255) / 256 * 256;
  w.sched_off = (w.ml_off + rows * 2 * sizeof(float) + 255) / 256 * 256;
  w.desc_off = w.sched_off + 256;
  // one record per (sequence, group of query heads): more groups than KV
  // heads when a KV head stands as several
  const int G = n_q_heads / std::max(n_kv_heads, 1), gv = mfma_group(G);
  const uint64_t groups = (uint64_t)n_kv_heads * (gv > 0 ? G / gv : 1);
  w.total = w.desc_off + (uint64_t)batch * groups * 2 * sizeof(int32_t);
  return w;
}

// Tokens per prefix-pass partial: the prefix waves take one chunk each.
// Longer chunks mean fewer partials for the combine but longer prefix waves,
// which must finish beside the split pass's.  Measured on the 256-sequence,
// 1024-token-prefix workload (one MI355X, split launch + combine per step):
// 256 tokens 75.8-76.6 us, 512 74.8-74.9, 1024 75.3.  A chunk spans at most
// 64 pages (one page id per lane) and is a multiple of 32 tokens.
int prefix_chunk_tokens(int page_size) {
  const int cap = std::min(kPrefixChunkMax, 64 * page_size / 32 * 32);
  return std::max(32, std::min(cap, kPrefixChunkTarget));
}
int prefix_chunks(int prefix_len, int page_size) {
  const int c = prefix_chunk_tokens(page_size);
  return (prefix_len + c - 1) / c;
}

// ws_layout plus the shared-prefix partials: [batch][n_q_heads][chunks] rows.
WsLayout ws_layout_prefix(const pkv_cache* c, int batch, int n_q_heads, int n_split,
                          int prefix_len) {
  WsLayout w = ws_layout(c, batch, n_q_heads, n_split);
  const uint64_t rows =
      (uint64_t)batch * n_q_heads * prefix_chunks(prefix_len, c->L.page_size);
  w.pre_o_off = (w.total + 255) / 256 * 256;
  w.pre_ml_off = (w.pre_o_off + rows * c->L.head_dim * sizeof(float) + 255) / 256 * 256;
  w.total = w.pre_ml_off + rows * 2 * sizeof(float);
  return w;
}

// A shared prefix: the first `len` tokens of every sequence sit in `pages`;
// with `next_upd`, the launch also writes the next step's table updates.
struct Prefix {
  const int32_t* pages;
  int32_t len;
  const int32_t* next_upd = nullptr;
  int32_t n_next_upd = 0;
  int32_t* table = nullptr;
};

// The kernels read an update list in place: device memory or pinned host
// memory (a pageable host list would fault the device).
bool readable_in_place(const void* p) {
  hipPointerAttribute_t at;
  const hipError_t pe = hipPointerGetAttributes(&at, p);
  if (pe != hipSuccess || at.type == hipMemoryTypeUnregistered || !at.devicePointer) {
    (void)hipGetLastError();  // leave no sticky error for later launches
    return false;
  }
  return true;
}

// Timing: while enabled, each kernel pass is launched with an event pair
// that its dispatch stamps with the kernel's start and end; the pairs are
// kept for pkv_timing_read.
struct Timer {
  pkv_cache* c;
  int kind;
  pkv::Launch l;
  Timer(pkv_cache* c_, int kind_, hipStream_t s, bool allowed = true) : c(c_), kind(kind_) {
    l.s = s;
    if (!c->timing || !allowed) return;
    if (hipEventCreate(&l.e0) != hipSuccess) {
      l.e0 = nullptr;
    } else if (hipEventCreate(&l.e1) != hipSuccess) {
      (void)hipEventDestroy(l.e0);
      l.e0 = l.e1 = nullptr;
    }
  }
  // after the launch: keep the pair if a kernel was launched with it
  void stop(hipError_t e) {
    if (!l.e0) return;
    if (e == hipSuccess && l.used) {
      c->events[kind].emplace_back(l.e0, l.e1);
    } else {
      (void)hipEventDestroy(l.e0);
      (void)hipEventDestroy(l.e1);
    }
    l.e0 = l.e1 = nullptr;
  }
};

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err; }

int pkv_timing_enable(pkv_cache* c, int32_t on) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  c->timing = on != 0;
  return PKV_OK;
}

int pkv_timing_read(pkv_cache* c, double* ms, int32_t* counts) {
  if (!c || !ms || !counts) return fail(PKV_EINVAL, "null argument");
  int rc = PKV_OK;
  for (int k = 0; k < PKV_T_COUNT; ++k) {
    double sum = 0.0;
    for (auto& e : c->events[k]) {
      float t = 0.f;
      if (hipEventSynchronize(e.second) != hipSuccess ||
          hipEventElapsedTime(&t, e.first, e.second) != hipSuccess)
        rc = fail(PKV_EHIP, "event query failed");
      sum += t;
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
    ms[k] = sum;
    counts[k] = (int32_t)c->events[k].size();
    c->events[k].clear();
  }
  return rc;
}

int32_t pkv_probe_blocks(uint64_t bytes) { return pkv::probe_blocks(bytes); }

int pkv_probe_stream(const void* src, void* dst, float* sink, uint64_t bytes, int32_t mode,
                     void* stream) {
  if (mode < 0 || mode > 2) return fail(PKV_EINVAL, "mode must be 0, 1 or 2");
  if (bytes == 0) return PKV_OK;
  if (bytes % 16) return fail(PKV_EINVAL, "bytes must be a multiple of 16");
  if (mode == 2) {
    const uint64_t n_blk = bytes / 4096;
    if (bytes % 4096 || (n_blk & (n_blk - 1)) || n_blk > (1ull << 31))
      return fail(PKV_EINVAL, "a scrambled read needs 4 KiB times a power of two bytes");
  }
  if (bytes / 4096 > 0xffffffffull) return fail(PKV_EINVAL, "buffer too large for the probe");
  if (!src || (mode == 1 && !dst) || (mode != 1 && !sink))
    return fail(PKV_EINVAL, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return fail(PKV_EINVAL, "pointers must be 16-byte aligned");
  hipError_t e = pkv::launch_probe(src, dst, sink, bytes, mode, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "probe launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_layout_bytes(const pkv_layout* l, uint64_t* kv_bytes, uint64_t* scale_bytes) {
  if (int e = check_layout(l)) return e;
  const uint64_t slots = (uint64_t)l->n_layers * l->n_pages * l->n_kv_heads * l->page_size;
  if (kv_bytes) *kv_bytes = slots * l->head_dim * pkv::format_bytes(l->format);
  if (scale_bytes) *scale_bytes = l->format == PKV_FMT_INT8 ? slots * sizeof(float) : 0;
  return PKV_OK;
}

int pkv_cache_create(const pkv_layout* l, void* k_pages, void* v_pages, float* k_scales,
                     float* v_scales, int32_t* dev_status, pkv_cache** out) {
  if (int e = check_layout(l)) return e;
  if (!out) return fail(PKV_EINVAL, "out is null");
  if (!k_pages || !v_pages) return fail(PKV_EINVAL, "page arrays are null");
  if (l->format == PKV_FMT_INT8 && (!k_scales || !v_scales))
    return fail(PKV_EINVAL, "int8 pages need scale arrays");
  if ((reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages)) & 15)
    return fail(PKV_EINVAL, "page arrays must be 16-byte aligned");
  pkv_cache* c = new (std::nothrow) pkv_cache;
  if (!c) return fail(PKV_ENOMEM, "out of host memory");
  c->L = *l;
  c->k_pages = k_pages;
  c->v_pages = v_pages;
  c->k_scales = l->format == PKV_FMT_INT8 ? k_scales : nullptr;
  c->v_scales = l->format == PKV_FMT_INT8 ? v_scales : nullptr;
  c->status = dev_status;
  *out = c;
  return PKV_OK;
}

void pkv_cache_destroy(pkv_cache* c) {
  if (!c) return;
  for (auto& v : c->events)
    for (auto& e : v) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
  delete c;
}

int pkv_paged_write(pkv_cache* c, int32_t layer, const int32_t* table, int32_t table_stride,
                    int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                    int32_t total_new, const void* k, const void* v, int32_t in_dtype,
                    int32_t format, void* stream) {
  return pkv_paged_write_layers(c, layer, 1, table, table_stride, batch, start_pos, cu_new,
                                total_new, k, v, in_dtype, format, stream);
}

int pkv_paged_write_layers(pkv_cache* c, int32_t layer0, int32_t n_layers,
                           const int32_t* table, int32_t table_stride, int32_t batch,
                           const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                           const void* k, const void* v, int32_t in_dtype, int32_t format,
                           void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (n_layers < 1 || layer0 < 0 || (int64_t)layer0 + n_layers > c->L.n_layers)
    return fail(PKV_ERANGE, "layers [%d, %d) outside [0, %d)", layer0, layer0 + n_layers,
                c->L.n_layers);
  if (format != c->L.format)
    return fail(PKV_EFORMAT, "write format %d differs from the store's %d", format, c->L.format);
  if (in_dtype != PKV_DT_F32 && in_dtype != PKV_DT_BF16)
    return fail(PKV_EINVAL, "unknown input dtype %d", in_dtype);
  if ((c->L.format == PKV_FMT_F32 && in_dtype != PKV_DT_F32) ||
      (c->L.format == PKV_FMT_BF16 && in_dtype != PKV_DT_BF16))
    return fail(PKV_EFORMAT, "native pages take rows of their own dtype");
  if (batch < 0 || total_new < 0 || table_stride < 1)
    return fail(PKV_EINVAL, "negative batch/total_new or table_stride < 1");
  if (total_new == 0) return PKV_OK;
  if (batch == 0) return fail(PKV_EINVAL, "rows given for an empty batch");
  if (!table || !start_pos || !cu_new || !k || !v) return fail(PKV_EINVAL, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(PKV_EINVAL, "k and v must be 16-byte aligned");
  pkv::WriteArgs a;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.status = c->status;
  a.table = table;
  a.start_pos = start_pos;
  a.cu_new = cu_new;
  a.k_in = k;
  a.v_in = v;
  a.layer_page0 = (int64_t)layer0 * c->L.n_pages;
  a.n_pages = c->L.n_pages;
  a.page_size = c->L.page_size;
  a.n_kv_heads = c->L.n_kv_heads;
  a.head_dim = c->L.head_dim;
  a.table_stride = table_stride;
  a.batch = batch;
  a.total_new = total_new;
  a.n_layers_w = n_layers;
  a.decode_lens = nullptr;
  Timer tm(c, PKV_T_WRITE, static_cast<hipStream_t>(stream));
  hipError_t e = pkv::launch_write(a, c->L.format, in_dtype, tm.l);
  tm.stop(e);
  if (e != hipSuccess) return fail(PKV_EHIP, "write launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_attend_split(const pkv_cache* c, int32_t batch, int32_t n_q_heads, int32_t max_len,
                     int32_t* split_tokens) {
  if (!c || !split_tokens) return fail(PKV_EINVAL, "null argument");
  *split_tokens = plan_split(c, batch, n_q_heads, max_len);
  return PKV_OK;
}

int pkv_attend_workspace_size(const pkv_cache* c, int32_t batch, int32_t n_q_heads,
                              int32_t max_len, int32_t split_tokens, uint64_t* bytes) {
  if (!c || !bytes) return fail(PKV_EINVAL, "null argument");
  if (batch < 0 || n_q_heads < 1 || max_len < 0) return fail(PKV_EINVAL, "bad sizes");
  if (int e = check_split(c, split_tokens)) return e;
  const int split = split_tokens ? split_tokens : plan_split(c, batch, n_q_heads, max_len);
  const int n_split = std::max(1, (max_len + split - 1) / split);
  if (n_split > kMaxSplits)
    return fail(PKV_EINVAL, "%d splits of %d tokens exceed %d per sequence", n_split, split,
                kMaxSplits);
  *bytes = ws_layout(c, batch, n_q_heads, n_split).total;
  return PKV_OK;
}

}  // extern "C"

namespace {

// Shared body of pkv_paged_attend and pkv_decode_step (k_new/v_new non-null:
// the decode step's new rows, written at position lens[b] - 1 first).
int attend_impl(pkv_cache* c, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q_heads,
                const int32_t* table, int32_t table_stride, const int32_t* lens, int32_t batch,
                int32_t max_len, float scale, void* out, void* workspace,
                uint64_t workspace_bytes, int32_t split_tokens, uint32_t flags, void* stream,
                const void* k_new, const void* v_new, int32_t in_dtype, bool timed = true,
                const Prefix* pre = nullptr) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (layer < 0 || layer >= c->L.n_layers)
    return fail(PKV_ERANGE, "layer %d outside [0, %d)", layer, c->L.n_layers);
  if (q_dtype != PKV_DT_F32 && q_dtype != PKV_DT_BF16)
    return fail(PKV_EINVAL, "unknown q dtype %d", q_dtype);
  if (n_q_heads < 1 || n_q_heads % c->L.n_kv_heads)
    return fail(PKV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d",
                n_q_heads, c->L.n_kv_heads);
  if (batch < 0 || max_len < 0 || table_stride < 1)
    return fail(PKV_EINVAL, "negative batch/max_len or table_stride < 1");
  if ((int64_t)max_len > (int64_t)table_stride * c->L.page_size)
    return fail(PKV_ERANGE, "max_len %d exceeds the table row (%d pages of %d)", max_len,
                table_stride, c->L.page_size);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  if (flags & ~(PKV_ATTEND_VALU | PKV_ATTEND_COMBINE_KERNEL | PKV_ATTEND_COMBINE_FUSED))
    return fail(PKV_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & PKV_ATTEND_COMBINE_KERNEL) && (flags & PKV_ATTEND_COMBINE_FUSED))
    return fail(PKV_EINVAL, "conflicting combine flags");
  if (int e = check_split(c, split_tokens)) return e;
  const int P0 = pre ? pre->len : 0;
  if (pre) {
    if (P0 < 1 || P0 % c->L.page_size || (int64_t)P0 > (int64_t)table_stride * c->L.page_size)
      return fail(PKV_EINVAL, "prefix_len %d must be a positive multiple of page_size %d within "
                  "the table row", P0, c->L.page_size);
    if (flags & (PKV_ATTEND_VALU | PKV_ATTEND_COMBINE_FUSED))
      return fail(PKV_EINVAL, "the shared-prefix attend takes neither PKV_ATTEND_VALU nor "
                  "PKV_ATTEND_COMBINE_FUSED");
    if (!pkv::mfma_supported(c->L.format, q_dtype == PKV_DT_BF16, c->L.head_dim,
                             c->L.page_size, n_q_heads / c->L.n_kv_heads, std::max(batch, 1),
                             c->L.n_kv_heads))
      return fail(PKV_EFORMAT, "no shared-prefix kernel for this cache (needs bf16/int8 pages, "
                  "a bf16 query, head_dim 64 or 128, page_size 16 or a multiple of 32, at most "
                  "16 query heads per KV head)");
    if (k_new && in_dtype != PKV_DT_BF16)
      return fail(PKV_EFORMAT, "the shared-prefix decode step takes bf16 rows");
  }
  if (batch == 0) return PKV_OK;
  if (!q || !out || !table || !lens || !workspace) return fail(PKV_EINVAL, "null device pointer");
  if (pre && !pre->pages) return fail(PKV_EINVAL, "null prefix page list");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  // the split pass covers the tokens past the shared prefix
  const int sfx_max = std::max(max_len - P0, 0);
  const int split = split_tokens ? split_tokens : plan_split(c, batch, n_q_heads, sfx_max);
  const int n_split = std::max(1, (sfx_max + split - 1) / split);
  if (n_split > kMaxSplits)
    return fail(PKV_EINVAL, "%d splits of %d tokens exceed %d per sequence", n_split, split,
                kMaxSplits);
  const WsLayout w = pre ? ws_layout_prefix(c, batch, n_q_heads, n_split, P0)
                         : ws_layout(c, batch, n_q_heads, n_split);
  if (workspace_bytes < w.total)
    return fail(PKV_ENOMEM, "workspace holds %llu bytes, %llu needed",
                (unsigned long long)workspace_bytes, (unsigned long long)w.total);

  pkv::AttendArgs a;
  a.q = q;
  a.out = out;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.status = c->status;
  a.table = table;
  a.lens = lens;
  a.counters = static_cast<uint32_t*>(workspace);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.o_off);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.ml_off);
  a.ws_desc = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.desc_off);
  a.ws_sched = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.sched_off);
  a.bal_waves = 0;
  a.unit_cost = kUnitCost;
  a.layer_page0 = (int64_t)layer * c->L.n_pages;
  a.qk_scale_log2 = scale * pkv::kLog2eHost;
  a.n_pages = c->L.n_pages;
  a.page_size = c->L.page_size;
  a.n_kv_heads = c->L.n_kv_heads;
  a.head_dim = c->L.head_dim;
  a.n_q_heads = n_q_heads;
  a.group = n_q_heads / c->L.n_kv_heads;
  a.table_stride = table_stride;
  a.batch = batch;
  a.max_len = max_len;
  a.split_tokens = split;
  a.n_split = n_split;
  a.q_bf16 = q_dtype == PKV_DT_BF16;
  if (pre) {
    a.table = table + P0 / c->L.page_size;  // the split pass sees the private suffixes
    a.table_full = table;
    a.prefix_pages = pre->pages;
    a.prefix_len = P0;
    a.pchunk = prefix_chunk_tokens(c->L.page_size);
    a.n_pchunks = prefix_chunks(P0, c->L.page_size);
    a.ws_pre_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.pre_o_off);
    a.ws_pre_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.pre_ml_off);
    a.next_upd = pre->next_upd;
    a.n_next_upd = pre->n_next_upd;
    a.upd_table = pre->table;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // More than 16 query heads per KV head: the matrix-core kernel takes each
  // KV head as kv_rep groups of gv query heads (its n_kv_heads and group
  // count those groups; the pages keep the KV heads).
  const int gv = mfma_group(a.group), rep = gv > 0 ? a.group / gv : 1;
  const bool mfma = !(flags & PKV_ATTEND_VALU) && gv > 0 &&
                    pkv::mfma_supported(c->L.format, a.q_bf16, a.head_dim, a.page_size, gv,
                                        batch, c->L.n_kv_heads * rep);
  if (mfma && rep > 1) {
    a.group = gv;
    a.n_kv_heads = c->L.n_kv_heads * rep;
    a.kv_rep = rep;
  }
  a.k_new = a.v_new = nullptr;
  if (k_new) {
    if (mfma && (sfx_max > 0 || pre) && in_dtype == PKV_DT_BF16) {
      a.k_new = k_new;  // the split pass writes and uses the new rows
      a.v_new = v_new;
    } else {
      // write the new rows first (row b at position lens[b] - 1), then attend
      pkv::WriteArgs w;
      w.k_pages = c->k_pages;
      w.v_pages = c->v_pages;
      w.k_scales = c->k_scales;
      w.v_scales = c->v_scales;
      w.status = c->status;
      w.table = table;
      w.start_pos = nullptr;
      w.cu_new = nullptr;
      w.k_in = k_new;
      w.v_in = v_new;
      w.layer_page0 = (int64_t)layer * c->L.n_pages;
      w.n_pages = c->L.n_pages;
      w.page_size = c->L.page_size;
      w.n_kv_heads = c->L.n_kv_heads;
      w.head_dim = c->L.head_dim;
      w.table_stride = table_stride;
      w.batch = batch;
      w.total_new = batch;
      w.decode_lens = lens;
      Timer tw(c, PKV_T_WRITE, s, timed);
      e = pkv::launch_write(w, c->L.format, in_dtype, tw.l);
      tw.stop(e);
      if (e != hipSuccess) return fail(PKV_EHIP, "write launch failed: %s", hipGetErrorString(e));
    }
  }
  // The combine kernel by default: measured against the in-kernel combine
  // it is faster on every workload here (the in-kernel merge is done by one
  // wave per (sequence, KV head) and lengthens the tail).  Flags can force
  // either.
  a.fuse_combine = mfma && (flags & PKV_ATTEND_COMBINE_FUSED) != 0;
  a.single_done = mfma && max_len > 0 && !pre;
  // The vector path with every sequence in one split writes the outputs
  // itself (the row-tiled kernel): no combine launch.
  a.direct_out = !mfma && !pre && max_len > 0 && n_split == 1 &&
                 pkv::valu_rows_supported(a.page_size, a.head_dim);
  // The balanced schedule where the library plans the work (split_tokens 0)
  // on the matrix-core path for the page formats it pays off on, unless the
  // in-kernel combine is asked for (it counts fixed splits); its flat slot
  // count must fit 31 bits.  Not for max_len 0: no split pass runs then to
  // record its choice, and the combine writes the zero outputs itself.
  const int wpc = bal_waves_per_cu(c->L.format);
  if (mfma && wpc > 0 && sfx_max > 0 && !a.fuse_combine && split_tokens == 0 &&
      (int64_t)batch * a.n_kv_heads * ((sfx_max + 31) / 32 + kUnitCost) < (int64_t)INT32_MAX) {
    a.bal_waves = wpc * device_cus();
  }
  // With a shared prefix the split pass's launch also runs the prefix pass
  // (its extra workgroups); a decode step runs the split work even without
  // suffix tokens, which reports rows that would land inside the prefix.
  a.split_wanted = sfx_max > 0 || a.k_new ? 1 : 0;
  if (sfx_max > 0 || (pre && (a.k_new || max_len > 0 || a.n_next_upd > 0))) {
    Timer tm(c, PKV_T_ATTEND_SPLIT, s, timed);
    e = mfma ? pkv::launch_attend_mfma(a, c->L.format, tm.l)
             : pkv::launch_attend_valu(a, c->L.format, tm.l);
    tm.stop(e);
    if (e != hipSuccess) return fail(PKV_EHIP, "attend launch failed: %s", hipGetErrorString(e));
    if (a.fuse_combine || a.direct_out) return PKV_OK;  // the split pass wrote the outputs
    // fixed splits on the matrix cores with every sequence in one split: the
    // split pass wrote each output directly (zeros for an empty sequence)
    if (mfma && a.bal_waves == 0 && n_split == 1 && a.single_done) return PKV_OK;
  }
  Timer tm(c, PKV_T_ATTEND_COMBINE, s, timed);
  e = pkv::launch_reduce(a, tm.l);
  tm.stop(e);
  if (e != hipSuccess) return fail(PKV_EHIP, "reduce launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attend(pkv_cache* c, int32_t layer, const void* q, int32_t q_dtype,
                     int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                     const int32_t* lens, int32_t batch, int32_t max_len, float scale, void* out,
                     void* workspace, uint64_t workspace_bytes, int32_t split_tokens,
                     uint32_t flags, void* stream) {
  return attend_impl(c, layer, q, q_dtype, n_q_heads, table, table_stride, lens, batch, max_len,
                     scale, out, workspace, workspace_bytes, split_tokens, flags, stream, nullptr,
                     nullptr, 0);
}

}  // extern "C"

// The allocation-free attend's workspace: one static array per device, held
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name stands for a host-side shadow, not device
// memory): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
static constexpr uint64_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (null and a message on failure).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    fail(PKV_EHIP, "no usable current device for the static scratch");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      fail(PKV_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int pkv_paged_attend_noalloc(pkv_cache* c, int32_t layer, const void* q, int32_t q_dtype,
                             int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                             const int32_t* lens, int32_t batch, int32_t max_len, float scale,
                             void* out, int32_t split_tokens, uint32_t flags, void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (flags & PKV_ATTEND_COMBINE_FUSED)
    return fail(PKV_EINVAL, "the static-scratch attend has no in-kernel combine");
  if (n_q_heads < 1 || batch < 0 || max_len < 0) return fail(PKV_EINVAL, "bad sizes");
  if (int e = check_split(c, split_tokens)) return e;
  const int split = split_tokens ? split_tokens : plan_split(c, batch, n_q_heads, max_len);
  const int n_split = std::max(1, (max_len + split - 1) / split);
  if (n_split > kMaxSplits)
    return fail(PKV_EINVAL, "%d splits of %d tokens exceed %d per sequence", n_split, split,
                kMaxSplits);
  const uint64_t need = ws_layout(c, batch, n_q_heads, n_split).total;
  if (need > kScratchBytes)
    return fail(PKV_ENOMEM, "these sizes need %llu bytes of workspace, the static scratch holds %llu",
                (unsigned long long)need, (unsigned long long)kScratchBytes);
  if (batch == 0) return PKV_OK;
  void* ws = device_scratch();
  if (!ws) return PKV_EHIP;
  return attend_impl(c, layer, q, q_dtype, n_q_heads, table, table_stride, lens, batch, max_len,
                     scale, out, ws, kScratchBytes, split_tokens, flags, stream, nullptr, nullptr,
                     0, /*timed=*/false);  // kernel timing would create events
}

int pkv_paged_attend_multi(pkv_cache* c, int32_t layer, const void* q, int32_t q_dtype,
                           int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                           const int32_t* lens, const int32_t* cu_q, int32_t batch,
                           int32_t total_q, int32_t max_q, int32_t max_len, float scale,
                           void* out, void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (layer < 0 || layer >= c->L.n_layers)
    return fail(PKV_ERANGE, "layer %d outside [0, %d)", layer, c->L.n_layers);
  if (q_dtype != PKV_DT_BF16) return fail(PKV_EINVAL, "queries must be bf16 (dtype %d)", q_dtype);
  if (n_q_heads < 1 || n_q_heads % c->L.n_kv_heads)
    return fail(PKV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d",
                n_q_heads, c->L.n_kv_heads);
  if (batch < 0 || total_q < 0 || max_q < 0 || max_len < 0 || table_stride < 1)
    return fail(PKV_EINVAL, "negative sizes or table_stride < 1");
  if ((int64_t)max_len > (int64_t)table_stride * c->L.page_size)
    return fail(PKV_ERANGE, "max_len %d exceeds the table row (%d pages of %d)", max_len,
                table_stride, c->L.page_size);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  const int group = n_q_heads / c->L.n_kv_heads;
  if (!pkv::mfma_supported(c->L.format, 1, c->L.head_dim, c->L.page_size, group, 1,
                           c->L.n_kv_heads))
    return fail(PKV_EFORMAT,
                "no multi-query kernel for this cache (needs bf16/int8 pages, head_dim 64 or "
                "128, page_size 16 or a multiple of 32, at most 16 query heads per KV head)");
  if (batch == 0 || total_q == 0 || max_q == 0) return PKV_OK;
  if (!q || !out || !table || !lens || !cu_q) return fail(PKV_EINVAL, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  pkv::MultiArgs a;
  a.q = q;
  a.out = out;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.status = c->status;
  a.table = table;
  a.lens = lens;
  a.cu_q = cu_q;
  a.layer_page0 = (int64_t)layer * c->L.n_pages;
  a.qk_scale_log2 = scale * pkv::kLog2eHost;
  a.n_pages = c->L.n_pages;
  a.page_size = c->L.page_size;
  a.n_kv_heads = c->L.n_kv_heads;
  a.head_dim = c->L.head_dim;
  a.n_q_heads = n_q_heads;
  a.group = group;
  a.table_stride = table_stride;
  a.batch = batch;
  a.max_len = max_len;
  a.total_q = total_q;
  a.max_q = max_q;
  a.n_pos = 16 / group;
  const int per_block = pkv::multi_positions_per_block(group);
  a.n_qgroups = (max_q + per_block - 1) / per_block;
  if (pkv::multi_grid(batch, c->L.n_kv_heads, a.n_qgroups) > INT32_MAX)
    return fail(PKV_EINVAL, "too many work items (batch %d, max_q %d)", batch, max_q);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Timer tm(c, PKV_T_ATTEND_MULTI, s);
  const hipError_t e = pkv::launch_attend_multi(a, c->L.format, tm.l);
  tm.stop(e);
  if (e != hipSuccess) return fail(PKV_EHIP, "multi-query launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_decode_step(pkv_cache* c, int32_t layer, const int32_t* table, int32_t table_stride,
                    const int32_t* lens, int32_t batch, int32_t max_len, const void* k_new,
                    const void* v_new, int32_t in_dtype, const void* q, int32_t q_dtype,
                    int32_t n_q_heads, float scale, void* out, void* workspace,
                    uint64_t workspace_bytes, int32_t split_tokens, uint32_t flags,
                    void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (in_dtype != PKV_DT_F32 && in_dtype != PKV_DT_BF16)
    return fail(PKV_EINVAL, "unknown input dtype %d", in_dtype);
  if ((c->L.format == PKV_FMT_F32 && in_dtype != PKV_DT_F32) ||
      (c->L.format == PKV_FMT_BF16 && in_dtype != PKV_DT_BF16))
    return fail(PKV_EFORMAT, "native pages take rows of their own dtype");
  if (batch > 0 && (!k_new || !v_new)) return fail(PKV_EINVAL, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  return attend_impl(c, layer, q, q_dtype, n_q_heads, table, table_stride, lens, batch, max_len,
                     scale, out, workspace, workspace_bytes, split_tokens, flags, stream, k_new,
                     v_new, in_dtype);
}

int pkv_prefix_workspace_size(const pkv_cache* c, int32_t batch, int32_t n_q_heads,
                              int32_t max_len, int32_t prefix_len, int32_t split_tokens,
                              uint64_t* bytes) {
  if (!c || !bytes) return fail(PKV_EINVAL, "null argument");
  if (batch < 0 || n_q_heads < 1 || max_len < 0 || prefix_len < 1)
    return fail(PKV_EINVAL, "bad sizes");
  if (int e = check_split(c, split_tokens)) return e;
  const int sfx_max = std::max(max_len - prefix_len, 0);
  const int split = split_tokens ? split_tokens : plan_split(c, batch, n_q_heads, sfx_max);
  const int n_split = std::max(1, (sfx_max + split - 1) / split);
  if (n_split > kMaxSplits)
    return fail(PKV_EINVAL, "%d splits of %d tokens exceed %d per sequence", n_split, split,
                kMaxSplits);
  *bytes = ws_layout_prefix(c, batch, n_q_heads, n_split, prefix_len).total;
  return PKV_OK;
}

int pkv_decode_step_prefix(pkv_cache* c, int32_t layer, int32_t* table,
                           int32_t table_stride, const int32_t* lens, int32_t batch,
                           int32_t max_len, const int32_t* prefix_pages, int32_t prefix_len,
                           const void* k_new, const void* v_new, int32_t in_dtype, const void* q,
                           int32_t q_dtype, int32_t n_q_heads, float scale, void* out,
                           void* workspace, uint64_t workspace_bytes, const int32_t* next_upd,
                           int32_t n_next_upd, int32_t split_tokens, uint32_t flags,
                           void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (!k_new != !v_new) return fail(PKV_EINVAL, "k_new and v_new must both be given or both null");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (n_next_upd < 0) return fail(PKV_EINVAL, "negative update count");
  if (n_next_upd > 0 && !next_upd) return fail(PKV_EINVAL, "null update list");
  if (n_next_upd > 0 && !readable_in_place(next_upd))
    return fail(PKV_EINVAL, "next_upd is neither device memory nor pinned host memory");
  Prefix pre{prefix_pages, prefix_len};
  if (batch > 0 && n_next_upd > 0) {
    pre.next_upd = next_upd;
    pre.n_next_upd = n_next_upd;
    pre.table = table;
  }
  return attend_impl(c, layer, q, q_dtype, n_q_heads, table, table_stride, lens, batch, max_len,
                     scale, out, workspace, workspace_bytes, split_tokens, flags, stream, k_new,
                     v_new, in_dtype, true, &pre);
}

int pkv_gather(pkv_cache* c, int32_t layer, const int32_t* table_row, int32_t len, void* k_out,
               void* v_out, float* k_scale_out, float* v_scale_out, void* stream) {
  if (!c) return fail(PKV_EINVAL, "cache is null");
  if (layer < 0 || layer >= c->L.n_layers)
    return fail(PKV_ERANGE, "layer %d outside [0, %d)", layer, c->L.n_layers);
  if (len < 0) return fail(PKV_EINVAL, "negative len");
  if (len == 0) return PKV_OK;
  if (!table_row || !k_out || !v_out) return fail(PKV_EINVAL, "null device pointer");
  if (c->L.format == PKV_FMT_INT8 && (!k_scale_out || !v_scale_out))
    return fail(PKV_EINVAL, "int8 gather needs scale outputs");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(PKV_EINVAL, "outputs must be 16-byte aligned");
  pkv::GatherArgs a;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.status = c->status;
  a.table_row = table_row;
  a.k_out = k_out;
  a.v_out = v_out;
  a.ks_out = k_scale_out;
  a.vs_out = v_scale_out;
  a.layer_page0 = (int64_t)layer * c->L.n_pages;
  a.n_pages = c->L.n_pages;
  a.page_size = c->L.page_size;
  a.n_kv_heads = c->L.n_kv_heads;
  a.head_dim = c->L.head_dim;
  a.len = len;
  Timer tm(c, PKV_T_GATHER, static_cast<hipStream_t>(stream));
  hipError_t e = pkv::launch_gather(a, c->L.format, tm.l);
  tm.stop(e);
  if (e != hipSuccess) return fail(PKV_EHIP, "gather launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_table_apply(int32_t* table, int32_t table_stride, int32_t batch, const int32_t* upd,
                    int32_t n, void* stream) {
  if (n < 0 || table_stride < 1 || batch < 0) return fail(PKV_EINVAL, "bad sizes");
  if (n == 0) return PKV_OK;
  if (!table || !upd) return fail(PKV_EINVAL, "null device pointer");
  if (!readable_in_place(upd))
    return fail(PKV_EINVAL, "upd is neither device memory nor pinned host memory");
  hipError_t e = pkv::launch_table_apply(table, table_stride, batch, upd, n,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "table update launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_read_device_status(pkv_cache* c, void* stream, int32_t* out) {
  if (!c || !out) return fail(PKV_EINVAL, "null argument");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out, c->status, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_EHIP, "status read failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_copy_pages(pkv_cache* c, const int32_t* pairs, int32_t n, void* stream) {
  if (!c || n < 0) return fail(PKV_EINVAL, "bad arguments");
  if (n == 0) return PKV_OK;
  if (!pairs) return fail(PKV_EINVAL, "null device pointer");
  pkv::CopyArgs a;
  a.k_pages = c->k_pages;
  a.v_pages = c->v_pages;
  a.k_scales = c->k_scales;
  a.v_scales = c->v_scales;
  a.status = c->status;
  a.pairs = pairs;
  a.page_bytes = (int64_t)c->L.n_kv_heads * c->L.page_size * c->L.head_dim *
                 pkv::format_bytes(c->L.format);
  a.scale_bytes = (int64_t)c->L.n_kv_heads * c->L.page_size * (int64_t)sizeof(float);
  a.n_pairs = n;
  a.n_layers = c->L.n_layers;
  a.n_pages = c->L.n_pages;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Timer tm(c, PKV_T_COPY_PAGES, s);
  const hipError_t e = pkv::launch_copy_pages(a, tm.l);
  tm.stop(e);
  if (e != hipSuccess) return fail(PKV_EHIP, "page copy launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- pool ----

struct pkv_pool {
  std::vector<int32_t> refs;
  // Hand-out order: page order[k] is the k-th choice.  Lowest-first is the
  // identity; a shuffled pool sorts the pages by a SplitMix64 draw per page.
  std::vector<int32_t> order, rank_of;  // rank_of[order[k]] = k
  std::set<int32_t> free_ranks;         // ordered: begin() is the next page handed out
  int32_t take() {
    const int32_t k = *free_ranks.begin();
    free_ranks.erase(free_ranks.begin());
    const int32_t i = order[k];
    refs[i] = 1;
    return i;
  }
};

namespace {

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014; the reference splitmix64.c of Vigna): output n
// (n = 0, 1, ...) of the generator seeded with `seed` is the mix of
// seed + (n + 1) * 0x9e3779b97f4a7c15.
uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

int pkv_pool_create(int32_t n_pages, uint64_t shuffle_seed, pkv_pool** out) {
  if (!out || n_pages < 1) return fail(PKV_EINVAL, "bad pool size or null out");
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return fail(PKV_ENOMEM, "out of host memory");
  p->refs.assign(n_pages, 0);
  p->order.resize(n_pages);
  for (int32_t i = 0; i < n_pages; ++i) p->order[i] = i;
  if (shuffle_seed != 0) {
    std::vector<uint64_t> key(n_pages);
    for (int32_t i = 0; i < n_pages; ++i) key[i] = splitmix64_at(shuffle_seed, (uint64_t)i);
    std::stable_sort(p->order.begin(), p->order.end(),
                     [&](int32_t x, int32_t y) { return key[x] < key[y]; });
  }
  p->rank_of.resize(n_pages);
  for (int32_t k = 0; k < n_pages; ++k) p->rank_of[p->order[k]] = k;
  for (int32_t k = 0; k < n_pages; ++k) p->free_ranks.insert(p->free_ranks.end(), k);
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* p) { delete p; }

int pkv_pool_alloc(pkv_pool* p, int32_t* id) {
  if (!p || !id) return fail(PKV_EINVAL, "null argument");
  if (p->free_ranks.empty()) return fail(PKV_ENOMEM, "all %zu pages in use", p->refs.size());
  *id = p->take();
  return PKV_OK;
}

int pkv_pool_alloc_n(pkv_pool* p, int32_t n, int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return fail(PKV_EINVAL, "bad arguments");
  if ((size_t)n > p->free_ranks.size())
    return fail(PKV_ENOMEM, "%d pages asked, %zu free", n, p->free_ranks.size());
  for (int32_t k = 0; k < n; ++k) ids[k] = p->take();
  return PKV_OK;
}

int pkv_pool_retain(pkv_pool* p, int32_t id) {
  if (!p || id < 0 || (size_t)id >= p->refs.size()) return fail(PKV_EINVAL, "page id out of range");
  if (p->refs[id] == 0) return fail(PKV_EINVAL, "page %d is not in use", id);
  ++p->refs[id];
  return PKV_OK;
}

int pkv_pool_release(pkv_pool* p, int32_t id) {
  if (!p || id < 0 || (size_t)id >= p->refs.size()) return fail(PKV_EINVAL, "page id out of range");
  if (p->refs[id] == 0) return fail(PKV_EDOUBLEFREE, "page %d released twice or never allocated", id);
  if (--p->refs[id] == 0) p->free_ranks.insert(p->rank_of[id]);
  return PKV_OK;
}

int32_t pkv_pool_refcount(const pkv_pool* p, int32_t id) {
  if (!p || id < 0 || (size_t)id >= p->refs.size()) return -1;
  return p->refs[id];
}

int32_t pkv_pool_num_free(const pkv_pool* p) { return p ? (int32_t)p->free_ranks.size() : -1; }

}  // extern "C"

// ------------------------------------------------------------ block tables --

struct pkv_seqs {
  pkv_pool* pool;
  int32_t batch, stride, page_size;
  std::vector<int32_t> table, lens, npages;
  std::vector<int64_t> admit_no;  // admission order of each sequence (0 = empty)
  int64_t admits = 0;
  std::vector<int32_t> updates;  // queued (b, j, page) triples, oldest first
  size_t upd_head = 0;
  std::vector<int32_t> copies;  // queued (src, dst) page copies, oldest first
  size_t copy_head = 0;
  void set(int32_t b, int32_t j, int32_t page) {
    table[(size_t)b * stride + j] = page;
    updates.push_back(b);
    updates.push_back(j);
    updates.push_back(page);
  }
  int32_t last_page(int32_t b) const { return table[(size_t)b * stride + npages[b] - 1]; }
  // Whether growing b by n tokens writes into its last page while another
  // sequence still holds it (copy-on-write), given that page's reference count.
  bool needs_copy(int32_t b, int32_t n, int32_t refs) const {
    return n > 0 && lens[b] % page_size != 0 && refs > 1;
  }
  int32_t new_pages(int32_t b, int32_t n) const {
    const int64_t need = ((int64_t)lens[b] + n + page_size - 1) / page_size;
    return (int32_t)std::max<int64_t>(need - npages[b], 0);
  }
  // Grow b by n tokens from ids (copy first if `copy`): the shared last page
  // is replaced by a fresh one whose contents the device copies over.
  void grow(int32_t b, int32_t n, bool copy, const int32_t* ids) {
    size_t k = 0;
    if (copy) {
      const int32_t old = last_page(b), fresh = ids[k++];
      copies.push_back(old);
      copies.push_back(fresh);
      set(b, npages[b] - 1, fresh);
      pkv_pool_release(pool, old);  // still held by the sharers
    }
    const int32_t extra = new_pages(b, n);
    for (int32_t e = 0; e < extra; ++e) set(b, npages[b] + e, ids[k++]);
    npages[b] += extra;
    lens[b] += n;
    if (lens[b] > 0 && admit_no[b] == 0) admit_no[b] = ++admits;
  }
};

namespace {

// Pages the appends n[b] need, in sequence order, with the copy-on-write
// decisions they imply (a copy lowers the shared page's count for the
// sequences after it).  ERANGE if a row would overflow.
int plan_growth(const pkv_seqs* s, const int32_t* n, std::vector<char>& copy, int64_t& total) {
  std::map<int32_t, int32_t> refs;  // simulated counts of shared last pages
  copy.assign(s->batch, 0);
  total = 0;
  for (int32_t b = 0; b < s->batch; ++b) {
    if (n[b] < 0) return fail(PKV_EINVAL, "n[%d] = %d is negative", b, n[b]);
    const int64_t need = ((int64_t)s->lens[b] + n[b] + s->page_size - 1) / s->page_size;
    if (need > s->stride)
      return fail(PKV_ERANGE, "sequence %d would need %lld pages, the row holds %d", b,
                  (long long)need, s->stride);
    if (s->npages[b] > 0 && n[b] > 0 && s->lens[b] % s->page_size) {
      const int32_t last = s->last_page(b);
      // a page held once never needs a copy (simulated counts only fall),
      // so only shared pages go through the map
      const int32_t held = pkv_pool_refcount(s->pool, last);
      if (held <= 1) {
        total += s->new_pages(b, n[b]);
        continue;
      }
      auto it = refs.find(last);
      if (it == refs.end()) it = refs.emplace(last, held).first;
      if (s->needs_copy(b, n[b], it->second)) {
        copy[b] = 1;
        --it->second;
        ++total;
      }
    }
    total += s->new_pages(b, n[b]);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_seqs_create(pkv_pool* pool, int32_t batch, int32_t table_stride, int32_t page_size,
                    pkv_seqs** out) {
  if (!pool || !out || batch < 1 || table_stride < 1 || page_size < 1)
    return fail(PKV_EINVAL, "bad arguments");
  pkv_seqs* s = new (std::nothrow) pkv_seqs;
  if (!s) return fail(PKV_ENOMEM, "out of host memory");
  s->pool = pool;
  s->batch = batch;
  s->stride = table_stride;
  s->page_size = page_size;
  s->table.assign((size_t)batch * table_stride, -1);
  s->lens.assign(batch, 0);
  s->npages.assign(batch, 0);
  s->admit_no.assign(batch, 0);
  *out = s;
  return PKV_OK;
}

int pkv_seqs_release(pkv_seqs* s, int32_t b) {
  if (!s || b < 0 || b >= s->batch) return fail(PKV_EINVAL, "bad sequence");
  for (int32_t j = 0; j < s->npages[b]; ++j) {
    int e = pkv_pool_release(s->pool, s->table[(size_t)b * s->stride + j]);
    if (e) return e;
    s->set(b, j, -1);
  }
  s->npages[b] = 0;
  s->lens[b] = 0;
  s->admit_no[b] = 0;
  return PKV_OK;
}

void pkv_seqs_destroy(pkv_seqs* s) {
  if (!s) return;
  for (int32_t b = 0; b < s->batch; ++b) pkv_seqs_release(s, b);
  delete s;
}

int pkv_seqs_append(pkv_seqs* s, int32_t b, int32_t n) {
  if (!s || b < 0 || b >= s->batch || n < 0) return fail(PKV_EINVAL, "bad arguments");
  std::vector<int32_t> one(s->batch, 0);
  one[b] = n;
  return pkv_seqs_append_all(s, one.data());
}

int pkv_seqs_append_all(pkv_seqs* s, const int32_t* n) {
  if (!s || !n) return fail(PKV_EINVAL, "null argument");
  std::vector<char> copy;
  int64_t total = 0;
  if (int e = plan_growth(s, n, copy, total)) return e;
  if (total > INT32_MAX) return fail(PKV_ENOMEM, "too many pages asked for");
  std::vector<int32_t> ids((size_t)total);
  if (total > 0)
    if (int e = pkv_pool_alloc_n(s->pool, (int32_t)total, ids.data())) return e;
  size_t next = 0;  // sequence by sequence, lowest pages first: as appends in sequence order
  for (int32_t b = 0; b < s->batch; ++b) {
    const size_t used = (size_t)copy[b] + (size_t)s->new_pages(b, n[b]);
    s->grow(b, n[b], copy[b] != 0, ids.data() + next);
    next += used;
  }
  return PKV_OK;
}

int pkv_seqs_fork(pkv_seqs* s, int32_t dst, int32_t src) {
  if (!s || dst < 0 || dst >= s->batch || src < 0 || src >= s->batch || dst == src)
    return fail(PKV_EINVAL, "bad arguments");
  if (s->npages[dst] != 0 || s->lens[dst] != 0)
    return fail(PKV_EINVAL, "sequence %d is not empty", dst);
  for (int32_t j = 0; j < s->npages[src]; ++j) {
    const int32_t page = s->table[(size_t)src * s->stride + j];
    if (int e = pkv_pool_retain(s->pool, page)) return e;
    s->set(dst, j, page);
  }
  s->npages[dst] = s->npages[src];
  s->lens[dst] = s->lens[src];
  if (s->lens[dst] > 0) s->admit_no[dst] = ++s->admits;
  return PKV_OK;
}

int32_t pkv_seqs_reserve(pkv_seqs* s, const int32_t* n, int32_t* victims, int32_t cap) {
  if (!s || !n || !victims || cap < s->batch) return fail(PKV_EINVAL, "bad arguments");
  int32_t count = 0;
  std::vector<int32_t> m(n, n + s->batch);
  for (;;) {
    std::vector<char> copy;
    int64_t total = 0;
    if (int e = plan_growth(s, m.data(), copy, total)) return e;
    if (total <= pkv_pool_num_free(s->pool)) return count;
    int32_t v = -1;
    for (int32_t b = 0; b < s->batch; ++b)
      if (s->lens[b] > 0 && (v < 0 || s->admit_no[b] > s->admit_no[v])) v = b;
    if (v < 0) return count;  // nothing left to preempt
    if (int e = pkv_seqs_release(s, v)) return e;
    m[v] = 0;  // requeued by the caller
    victims[count++] = v;
  }
}

int32_t pkv_seqs_take_copies(pkv_seqs* s, int32_t* pairs, int32_t cap) {
  if (!s || cap < 0 || (cap > 0 && !pairs)) return fail(PKV_EINVAL, "bad arguments");
  const size_t avail = (s->copies.size() - s->copy_head) / 2;
  const size_t n = std::min<size_t>(avail, (size_t)cap);
  std::copy(s->copies.begin() + s->copy_head, s->copies.begin() + s->copy_head + 2 * n, pairs);
  s->copy_head += 2 * n;
  if (s->copy_head == s->copies.size()) {
    s->copies.clear();
    s->copy_head = 0;
  }
  return (int32_t)n;
}

int pkv_seqs_share(pkv_seqs* s, int32_t dst, int32_t src, int32_t n_pages) {
  if (!s || dst < 0 || dst >= s->batch || src < 0 || src >= s->batch || dst == src || n_pages < 0)
    return fail(PKV_EINVAL, "bad arguments");
  if (s->npages[dst] != 0) return fail(PKV_EINVAL, "sequence %d is not empty", dst);
  if ((int64_t)n_pages * s->page_size > s->lens[src])
    return fail(PKV_EINVAL, "only full pages of sequence %d can be shared", src);
  for (int32_t j = 0; j < n_pages; ++j) {
    const int32_t page = s->table[(size_t)src * s->stride + j];
    if (int e = pkv_pool_retain(s->pool, page)) return e;
    s->set(dst, j, page);
  }
  s->npages[dst] = n_pages;
  s->lens[dst] = n_pages * s->page_size;
  if (s->lens[dst] > 0) s->admit_no[dst] = ++s->admits;
  return PKV_OK;
}

const int32_t* pkv_seqs_table(const pkv_seqs* s) { return s ? s->table.data() : nullptr; }
const int32_t* pkv_seqs_lens(const pkv_seqs* s) { return s ? s->lens.data() : nullptr; }

int32_t pkv_seqs_take_updates(pkv_seqs* s, int32_t* upd, int32_t cap) {
  if (!s || cap < 0 || (cap > 0 && !upd)) return fail(PKV_EINVAL, "bad arguments");
  const size_t avail = (s->updates.size() - s->upd_head) / 3;
  const size_t n = std::min<size_t>(avail, (size_t)cap);
  std::copy(s->updates.begin() + s->upd_head, s->updates.begin() + s->upd_head + 3 * n, upd);
  s->upd_head += 3 * n;
  if (s->upd_head == s->updates.size()) {
    s->updates.clear();
    s->upd_head = 0;
  }
  return (int32_t)n;
}

}  // extern "C"
