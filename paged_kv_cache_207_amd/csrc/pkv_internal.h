// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>
#include <vector>

#include "../../include/pkv.h"

struct pkv_cache {
  pkv_layout L;
  void* k_pages;
  void* v_pages;
  float* k_scales;
  float* v_scales;
  int32_t* status;
  bool timing = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events[PKV_T_COUNT];  // (start, end) per pass
};

namespace pkv {

constexpr float kLog2eHost = 1.4426950408889634f;

// Arguments of the page-write kernel (one launch = one paged_write call).
struct WriteArgs {
  void* k_pages;
  void* v_pages;
  float* k_scales;
  float* v_scales;
  int32_t* status;
  const int32_t* table;
  const int32_t* start_pos;
  const int32_t* cu_new;
  const void* k_in;
  const void* v_in;
  int64_t layer_page0;  // first layer * n_pages
  int32_t n_pages, page_size, n_kv_heads, head_dim;
  int32_t table_stride, batch, total_new;
  int32_t n_layers_w = 1;  // layers written (k_in/v_in: [n_layers_w][total_new][Hkv][D])
  const int32_t* decode_lens;  // non-null: row b goes to position decode_lens[b] - 1 of sequence b
};

// Arguments shared by the split-K attention kernels and the reduce kernel.
struct AttendArgs {
  const void* q;
  void* out;
  const void* k_pages;
  const void* v_pages;
  const float* k_scales;
  const float* v_scales;
  int32_t* status;
  const int32_t* table;
  const int32_t* lens;
  float* ws_o;   // [batch][n_q_heads][n_split][head_dim] unnormalised partial outputs
  float* ws_ml;  // [batch][n_q_heads][n_split][2] running max (log2 units) and sum
  // Balanced schedule (bal_waves > 0): partials are indexed by slot * group
  // + head-in-group instead, where a piece's slot is (b * n_kv_heads + g) +
  // its wave; ws_desc[2 u] and [2 u + 1] give unit u's first slot and its
  // number of pieces (written by the split pass for units of 2+ pieces).
  int32_t* ws_desc;
  int32_t* ws_sched;  // balanced schedule requested: 1 if the split pass used it, 0 if it
                      // took fixed splits (every non-empty length equal)
  int32_t bal_waves;  // 0: fixed splits; else the balanced schedule's wave bound
  int32_t unit_cost;  // balanced schedule: set-up cost of a unit, in steps
  uint32_t* counters;  // [batch][n_kv_heads] splits finished (zero between calls)
  const void* k_new;   // decode step: [batch][n_kv_heads][head_dim] bf16 rows at len - 1,
  const void* v_new;   // written and attended by the matrix-core kernel (null: none)
  int64_t layer_page0;
  float qk_scale_log2;  // softmax scale * log2(e)
  int32_t n_pages, page_size, n_kv_heads, head_dim, n_q_heads, group;
  int32_t table_stride, batch, max_len, split_tokens, n_split;
  int32_t q_bf16;  // 1: q and out are bf16, 0: float32
  int32_t fuse_combine;  // matrix-core path: 1 = combine in the split pass, 0 = combine kernel
  int32_t single_done;   // combine kernel: single-split sequences are already written
  // matrix-core path: n_kv_heads / kv_rep KV heads hold the pages, each seen
  // as kv_rep groups of `group` query heads (more than 16 query heads per KV
  // head); n_kv_heads and group count those groups
  int32_t kv_rep = 1;
  int32_t direct_out = 0;  // vector path, one split: the split pass writes every output
                           // (zeros for an empty sequence) and no combine runs
  // Shared-prefix mode (prefix_len > 0): the first prefix_len tokens of every
  // sequence sit in the pages prefix_pages lists (the same physical pages in
  // every table row).  The prefix pass attends over them for all sequences at
  // once and leaves n_pchunks partials per (sequence, query head) in
  // ws_pre_o / ws_pre_ml ([batch][n_q_heads][n_pchunks] rows); the split
  // pass then sees table + prefix_len / page_size and lengths lens -
  // prefix_len (the private suffixes) and leaves partials for every piece;
  // the combine merges both.
  const int32_t* prefix_pages = nullptr;
  const int32_t* table_full = nullptr;  // the unshifted table (the prefix pass checks its rows)
  float* ws_pre_o = nullptr;
  float* ws_pre_ml = nullptr;
  int32_t prefix_len = 0;
  int32_t pchunk = 0;  // tokens per prefix chunk (a multiple of 32, at most 64 pages)
  int32_t n_pchunks = 0;
  // shared-prefix mode: the split pass's launch holds split_blocks workgroups
  // of split work (none when split_wanted is 0: no suffix tokens, no new
  // rows), then the prefix pass's waves
  int32_t split_blocks = 0;
  int32_t split_wanted = 1;
  // waves of the split pass (each takes its own items; a launch's workgroups
  // hold several, set by the launcher)
  int32_t split_waves = 0;
  // shared-prefix mode: the waves of a prefix workgroup that take work (the
  // rest exit at once), so that the prefix workgroups spread over every
  // compute unit
  int32_t pre_group_waves = 1;
  // shared-prefix mode: table updates for the next step (upd_table[b *
  // table_stride + block] = page for each (b, block, page) row), each for an
  // entry this launch does not read
  const int32_t* next_upd = nullptr;
  int32_t n_next_upd = 0;
  int32_t* upd_table = nullptr;
};

// Arguments of the several-queries-per-sequence kernel (one launch = one
// pkv_paged_attend_multi call).
struct MultiArgs {
  const void* q;  // [total_q][n_q_heads][head_dim] bf16
  void* out;      // same shape, bf16
  const void* k_pages;
  const void* v_pages;
  const float* k_scales;
  const float* v_scales;
  int32_t* status;
  const int32_t* table;
  const int32_t* lens;
  const int32_t* cu_q;  // [batch + 1] query rows of each sequence
  int64_t layer_page0;
  float qk_scale_log2;  // softmax scale * log2(e)
  int32_t n_pages, page_size, n_kv_heads, head_dim, n_q_heads, group;
  int32_t table_stride, batch, max_len, total_q, max_q;
  int32_t n_pos;      // query positions per wave (16 / group)
  int32_t n_qgroups;  // workgroups per (sequence, KV head): ceil(max_q / positions per block)
};

// Arguments of the page-copy kernel (copy-on-write).
struct CopyArgs {
  void* k_pages;
  void* v_pages;
  float* k_scales;  // null unless int8
  float* v_scales;
  int32_t* status;
  const int32_t* pairs;  // [n_pairs][2] (src, dst) page ids
  int64_t page_bytes;    // one layer's page of K (or V): n_kv_heads * page_size * head_dim * elem
  int64_t scale_bytes;   // one layer's page of scales: n_kv_heads * page_size * 4
  int32_t n_pairs, n_layers, n_pages;
};

struct GatherArgs {
  const void* k_pages;
  const void* v_pages;
  const float* k_scales;
  const float* v_scales;
  int32_t* status;
  const int32_t* table_row;
  void* k_out;
  void* v_out;
  float* ks_out;
  float* vs_out;
  int64_t layer_page0;
  int32_t n_pages, page_size, n_kv_heads, head_dim, len;
};

// Element size of a page format in bytes.
inline int format_bytes(int fmt) { return fmt == PKV_FMT_F32 ? 4 : fmt == PKV_FMT_BF16 ? 2 : 1; }

// Where a kernel goes: the stream and, while timing is on, two events that
// the dispatch itself stamps with the kernel's start and end (no marker
// packets between kernels, so timing does not lengthen a step).  `used` is
// set once a kernel has been launched with them.
struct Launch {
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  mutable bool used = false;
};

// Launch a kernel whose only parameter is an argument struct.
template <typename K, typename A>
inline hipError_t launch1(K kernel, dim3 grid, dim3 block, size_t shm, const Launch& l, A arg) {
  void* args[] = {&arg};
  l.used = true;
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, shm, l.s,
                            l.e0, l.e1, 0);
}

// Launchers (return the hipError_t of the launch).
hipError_t launch_write(const WriteArgs& a, int fmt, int in_dtype, const Launch& l);
hipError_t launch_gather(const GatherArgs& a, int fmt, const Launch& l);
hipError_t launch_attend_valu(const AttendArgs& a, int fmt, const Launch& l);
// Whether the vector path takes the row-tiled kernel for this page size and
// head dim (the one that can write outputs directly).
bool valu_rows_supported(int page_size, int head_dim);
// Returns hipErrorNotSupported when the shape has no matrix-core variant.  In
// shared-prefix mode (prefix_len > 0) the launch also runs the prefix pass.
hipError_t launch_attend_mfma(const AttendArgs& a, int fmt, const Launch& l);
constexpr int kMaxMfmaBatch = 4096;   // the work list lives in LDS: 12 bytes per sequence
constexpr int kMaxMfmaKvHeads = 64;  // split counters: a fixed region of the workspace
bool mfma_supported(int fmt, int q_bf16, int head_dim, int page_size, int group, int batch,
                    int n_kv_heads);
hipError_t launch_reduce(const AttendArgs& a, const Launch& l);
// Returns hipErrorNotSupported when the shape has no matrix-core variant.
hipError_t launch_attend_multi(const MultiArgs& a, int fmt, const Launch& l);
int64_t multi_grid(int batch, int n_kv_heads, int n_qgroups);
int multi_positions_per_block(int group);
hipError_t launch_copy_pages(const CopyArgs& a, const Launch& l);
hipError_t launch_probe(const void* src, void* dst, float* sink, uint64_t bytes, int mode,
                        hipStream_t s);
int probe_blocks(uint64_t bytes);
hipError_t launch_table_apply(int32_t* table, int32_t stride, int32_t batch, const int32_t* upd,
                              int32_t n, hipStream_t s);

}  // namespace pkv
