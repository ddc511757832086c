/*
 * pkv.h - paged KV cache for MI355X (gfx950): page write, in-place paged
 * decode attention, gather, and the host page pool / block-table plumbing.
 *
 * The method.  A sequence's K/V rows live in fixed-size pages of a shared
 * pool; a per-sequence block table maps logical block j to a physical page,
 * so token t of the sequence lives at (table[t / page_size], t % page_size)
 * (tiny-llm paged_kv.py, module docstring).  Pages may sit anywhere in the
 * pool, several tables may name the same page (libmir-metal
 * src/engine/kv/paged/mod.rs, PagedStore::snapshot), and only real tokens are
 * stored.  Decode attention reads the pages in place through the table
 * instead of gathering them into a contiguous copy first (tiny-llm
 * paged_kv.py docstring: the gather is the toy's extra copy).
 *
 * Conventions for every call:
 *   - "device" pointers are device addresses (hipMalloc memory or the data
 *     pointer of a torch GPU tensor); "host" pointers are ordinary memory.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory and never synchronises a stream.  Kernels are enqueued
 *     on `stream` (a hipStream_t; NULL = the default stream) and read their
 *     inputs when they run, so buffers must stay alive until the stream has
 *     passed them.
 *   - Calls return PKV_OK or a negative PKV_E* status; pkv_last_error()
 *     returns a message for the calling thread's last failure.  Arguments
 *     are validated on the host before anything is enqueued: a failing call
 *     enqueues nothing.
 *   - Device-side checks never fault: a table entry outside [0, n_pages), a
 *     write position past the table row or a length past the bound makes the
 *     kernel skip that row/page (or clamp the length) and OR a PKV_DEV_* bit
 *     into the cache's device status word.
 *
 * Page layout in HBM (chosen for gfx950, see the pool layout note below):
 *   K pages  [n_layers][n_pages][n_kv_heads][slab], one slab of page_size rows
 *            of head_dim per page and KV head.  With row bytes R = head_dim *
 *            element size: rows of 64 or 128 bytes are stored in 64-byte
 *            pieces, piece-major (byte b of slot t's row at
 *            ((b / 64) * page_size + m(t)) * 64 + b % 64, with m(t) =
 *            ((t >> 2) & 1) * page_size / 2 + (t >> 3) * 4 + (t & 3) when
 *            page_size is a multiple of 8, else m(t) = t: the rows one score
 *            tile of a 32-token step reads lie together); other rows are
 *            whole, in slot order (byte b of slot t at t * R + b)
 *   V pages  [n_layers][n_pages][n_kv_heads][head_dim][page_size]
 *            (per page and KV head one dim-major slab: for each dim, the
 *             page_size slots are contiguous)
 *   element  float32 (PKV_FMT_F32), bfloat16 (PKV_FMT_BF16) or an int8 code
 *            (PKV_FMT_INT8)
 *   int8 scales, K and V each: float32 [n_layers][n_pages][n_kv_heads][page_size]
 *            (a separate array per K and V as in libmir-metal's Arena
 *             key_scales / value_scales, indexed by the same physical page)
 * Row buffers crossing the ABI (write input, gather output) are token-major
 * [n_rows][n_kv_heads][head_dim], like AstrAI inference/cache.py's
 * PagedCache.write input.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK 0
#define PKV_EINVAL (-1)      /* null pointer, bad shape, bad enum, G does not divide */
#define PKV_ERANGE (-2)      /* layer out of range, length bound past the table */
#define PKV_EFORMAT (-3)     /* write format differs from the store, dtype not accepted */
#define PKV_ENOMEM (-4)      /* pool exhausted, workspace too small */
#define PKV_EHIP (-5)        /* a HIP launch failed */
#define PKV_EDOUBLEFREE (-6) /* release of a page that is not in use */

/* ---- device status bits (OR-ed into the cache's status word) ------------ */
#define PKV_DEV_WRITE_PAGE 1u   /* a written row's table entry is outside [0, n_pages) */
#define PKV_DEV_WRITE_TABLE 2u  /* a written row's position is negative or past the table row */
#define PKV_DEV_READ_PAGE 4u    /* attend/gather met a table entry outside [0, n_pages) */
#define PKV_DEV_LEN 8u          /* attend met lens[b] < 0 or > max_len (clamped) */
#define PKV_DEV_QROWS 16u       /* multi-query attend met cu_q outside [0, total_q] or
                                   decreasing (that sequence skipped), a chunk longer than
                                   its sequence (rows before position 0 give zeros) or
                                   longer than max_q (rows past max_q may be left
                                   unwritten) */
#define PKV_DEV_WRITE_ROWS 32u  /* paged_write met a sequence whose rows cu_new[b] ..
                                   cu_new[b+1] are decreasing or outside [0, total_new]
                                   (that sequence skipped) */
#define PKV_DEV_PREFIX 64u      /* shared-prefix attend met a table row whose first pages
                                   differ from the shared list (its result is wrong), or a
                                   decode-step row that would land inside the shared prefix
                                   (not written) */
#define PKV_DEV_TABLE_NEXT 128u /* a next-step table update (pkv_decode_step_prefix) named an
                                   entry the step itself reads (that update skipped) */

typedef enum { PKV_FMT_F32 = 0, PKV_FMT_BF16 = 1, PKV_FMT_INT8 = 2 } pkv_format;
typedef enum { PKV_DT_F32 = 0, PKV_DT_BF16 = 1 } pkv_dtype;

/* pkv_paged_attend flags */
#define PKV_ATTEND_VALU 1u /* force the vector-ALU kernel even where the matrix-core one applies */
#define PKV_ATTEND_COMBINE_KERNEL 2u /* matrix-core path: combine splits in a second kernel */
#define PKV_ATTEND_COMBINE_FUSED 4u  /* matrix-core path: combine splits in the split pass */

typedef struct pkv_layout {
  int32_t n_layers;
  int32_t n_pages;
  int32_t page_size;  /* tokens per page, >= 1 */
  int32_t n_kv_heads;
  int32_t head_dim;   /* multiple of 16, at most 256 */
  int32_t format;     /* pkv_format */
} pkv_layout;

typedef struct pkv_cache pkv_cache;

/* Bytes of one K (or V) page array and of one K (or V) scale array for this
 * layout (scale bytes are 0 unless the format is int8).  EINVAL on a bad
 * layout. */
int pkv_layout_bytes(const pkv_layout* layout, uint64_t* kv_bytes, uint64_t* scale_bytes);

/* Bind caller-owned device page arrays to a cache handle (the PagedStore /
 * Arena pair of libmir-metal paged/mod.rs).  k_pages/v_pages: device, the
 * layout above.  k_scales/v_scales: device float32, required for int8 and
 * ignored otherwise.  dev_status: device int32 status word (the caller
 * zeroes it; kernels only OR bits into it).  The handle keeps the pointers
 * until pkv_cache_destroy. */
int pkv_cache_create(const pkv_layout* layout, void* k_pages, void* v_pages, float* k_scales,
                     float* v_scales, int32_t* dev_status, pkv_cache** out);
void pkv_cache_destroy(pkv_cache* cache);

/* paged_write(layer, table, start_pos, k, v, format).
 * Row i of sequence b (rows cu_new[b] .. cu_new[b+1]-1 of k and v) is stored
 * at position t = start_pos[b] + (i - cu_new[b]), i.e. in page
 * table[b * table_stride + t / page_size], slot t % page_size (AstrAI
 * cache.py PagedCache.write, with one start position per sequence as in
 * tiny-llm paged_kv.py's per-slot lengths).  No other slot is touched.
 *   table      device int32 [batch][table_stride]; entries past the rows a
 *              write reaches are never read.
 *   start_pos  device int32 [batch]; cu_new device int32 [batch + 1],
 *              non-decreasing, cu_new[0] = 0, cu_new[batch] = total_new.
 *              Device-side, a sequence whose row range is decreasing or
 *              outside [0, total_new] is skipped and sets PKV_DEV_WRITE_ROWS;
 *              positions without a page set PKV_DEV_WRITE_TABLE/_PAGE.
 *   k, v       device [total_new][n_kv_heads][head_dim] of in_dtype.
 *   format     must equal the store's format (EFORMAT otherwise).
 * F32 pages take f32 rows and BF16 pages bf16 rows, copied bit for bit.
 * INT8 pages take bf16 or f32 rows and quantize each (token, KV head) row of
 * K and of V on its own: scale = max|x| / 127 (one IEEE float32 division),
 * code = clamp(rint(x / scale), -127, 127) with ties to even; an all-zero row
 * stores scale 0 and codes 0 (the KvPageFormat::Int8PerTokenHead of
 * libmir-metal paged/mod.rs; the rule itself is not printed there). */
int pkv_paged_write(pkv_cache* cache, int32_t layer, const int32_t* table, int32_t table_stride,
                    int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                    int32_t total_new, const void* k, const void* v, int32_t in_dtype,
                    int32_t format, void* stream);

/* pkv_paged_write for layers layer0 .. layer0 + n_layers - 1 in one launch,
 * through the one block table all layers share (tiny-llm paged_kv.py: a
 * block holds the same token positions in every layer's pool).  k and v are
 * device [n_layers][total_new][n_kv_heads][head_dim]: layer l's rows follow
 * layer l-1's, and every layer's rows go to the same positions.  ERANGE if
 * the layers leave the store. */
int pkv_paged_write_layers(pkv_cache* cache, int32_t layer0, int32_t n_layers,
                           const int32_t* table, int32_t table_stride, int32_t batch,
                           const int32_t* start_pos, const int32_t* cu_new, int32_t total_new,
                           const void* k, const void* v, int32_t in_dtype, int32_t format,
                           void* stream);

/* The planned split size (tokens per split-K partition): 1024 tokens (when
 * max_len > 16384: 4096 for bf16 pages, 2048 for the others), halved down to
 * 256 while batch * n_kv_heads * splits < 512; rounded up to a multiple of 64
 * and of page_size.
 * pkv_paged_attend called with split_tokens = 0 uses it, except where it
 * balances the work instead (see there). */
int pkv_attend_split(const pkv_cache* cache, int32_t batch, int32_t n_q_heads, int32_t max_len,
                     int32_t* split_tokens);

/* Workspace bytes pkv_paged_attend needs for these sizes (split_tokens 0 =
 * the library's plan, either schedule). */
int pkv_attend_workspace_size(const pkv_cache* cache, int32_t batch, int32_t n_q_heads,
                              int32_t max_len, int32_t split_tokens, uint64_t* bytes);

/* paged_attend(q, table, lens, scale): one decode query per sequence.
 * For sequence b and query head h (KV head g = h / (n_q_heads / n_kv_heads)):
 *   out[b][h] = sum_{t < lens[b]} softmax_t(scale * <q[b][h], k_t>) v_t
 * with k_t, v_t read in place from the pages of table row b (int8: code times
 * its per-token scale).  lens[b] counts every stored token, including one
 * written in the same step, and no other mask applies (tiny-llm paged_kv.py
 * begin_step masks positions <= the pre-step length).  lens[b] = 0 gives
 * zeros.  Work is split over tokens and the partial results (running max,
 * sum and weighted V) are combined by a second kernel or, on the matrix-core
 * path with PKV_ATTEND_COMBINE_FUSED, by the workgroup that finishes a
 * sequence's last split (through counters in the workspace).
 *   split_tokens > 0: fixed partitions of that many tokens (a multiple of 64
 *   and of page_size).  A sequence's result depends only on its own tokens,
 *   the split size and the combine choice.
 *   split_tokens = 0: the library's plan.  For bf16 pages on the
 *   matrix-core path (without PKV_ATTEND_COMBINE_FUSED) this is the
 *   balanced schedule: every (sequence, KV head) is a run of 32-token steps
 *   plus a fixed set-up cost, and each wave of the persistent grid takes an
 *   equal share of that flat space, so batches of uneven lengths keep every
 *   wave busy to the end.  Pieces then start wherever the shares fall, so a
 *   result depends (in its last bits) on every length of the batch; with the
 *   same lengths it is reproducible bit for bit (page permutation and prefix
 *   sharing included).  Elsewhere the planned split size of
 *   pkv_attend_split.
 *   q          device [batch][n_q_heads][head_dim] of q_dtype; out has the
 *              same shape and dtype (bf16 rounded to nearest even).
 *   table      device int32 [batch][table_stride].
 *   lens       device int32 [batch]; max_len is a host upper bound on them,
 *              at most table_stride * page_size (ERANGE otherwise).
 *   scale      softmax scale (float32).
 *   workspace  device scratch of at least pkv_attend_workspace_size bytes
 *              (ENOMEM otherwise), 256-byte aligned.  Its first 1 MiB holds
 *              split counters that must be zero before the first call: zero
 *              the buffer once.  Every completed call leaves them zero, so
 *              one workspace (large enough for the biggest call) serves
 *              calls of any shape on one stream; calls that may overlap need
 *              separate workspaces.
 *   flags      0, or PKV_ATTEND_VALU, and/or one of PKV_ATTEND_COMBINE_KERNEL
 *              / PKV_ATTEND_COMBINE_FUSED.
 * The matrix-core kernel serves bf16/int8 pages with a bf16 query, head_dim
 * 64 or 128, page_size 16 or a multiple of 32, batch <= 4096, and G =
 * n_q_heads / n_kv_heads query heads per KV head either up to 16 or with a
 * divisor g in [8, 16] (the largest is taken: each KV head then counts as
 * G / g groups of g heads), with at most 64 such groups; every other shape
 * runs on the vector-ALU kernels.
 * A split size gives at most 16384 splits per sequence (EINVAL otherwise). */
int pkv_paged_attend(pkv_cache* cache, int32_t layer, const void* q, int32_t q_dtype,
                     int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                     const int32_t* lens, int32_t batch, int32_t max_len, float scale, void* out,
                     void* workspace, uint64_t workspace_bytes, int32_t split_tokens,
                     uint32_t flags, void* stream);

/* pkv_paged_attend without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the split partials go to a static
 * device array of the library, 64 MiB per device, which each device the
 * library runs on holds until the process ends.  The call allocates
 * nothing itself (no hipMalloc, hipFree, events or library allocations; the
 * caller still passes q, out, table and lens) and enqueues exactly what
 * pkv_paged_attend with the same arguments enqueues, so its outputs are
 * identical.  Every call on a device shares that device's array and leaves
 * in it the last call's partials: calls that may overlap on one device
 * (other streams, other threads) race and must not be issued.  Nothing in
 * the array has to start at zero.
 *   Errors as pkv_paged_attend, plus ENOMEM when the sizes need more than
 *   the 64 MiB (pkv_attend_workspace_size gives the need) and EINVAL for
 *   PKV_ATTEND_COMBINE_FUSED, whose counters this variant does not keep. */
int pkv_paged_attend_noalloc(pkv_cache* cache, int32_t layer, const void* q, int32_t q_dtype,
                             int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                             const int32_t* lens, int32_t batch, int32_t max_len, float scale,
                             void* out, int32_t split_tokens, uint32_t flags, void* stream);

/* One decode step: paged_write of one new row per sequence, then
 * paged_attend, as a single call.  Row b of k_new / v_new (device
 * [batch][n_kv_heads][head_dim] of in_dtype) is stored at position
 * lens[b] - 1 of sequence b (lens counts the new token; a sequence with
 * lens[b] = 0 gets no row and a zero output), then every sequence attends
 * over its lens[b] tokens exactly as pkv_paged_attend does.  Pages and
 * outputs equal those of pkv_paged_write (start_pos = lens - 1, one row per
 * sequence) followed by pkv_paged_attend.  On the matrix-core path with bf16
 * rows, the workgroup that owns a sequence's last split writes the row and
 * uses it directly (one launch, no write kernel); otherwise the write kernel
 * runs first.  The new token's page must not be shared with another
 * sequence.  Other arguments and errors as pkv_paged_write and
 * pkv_paged_attend (this tiny-llm paged_kv.py begin_step + update pair
 * writes each slot's token, then attends). */
int pkv_decode_step(pkv_cache* cache, int32_t layer, const int32_t* table, int32_t table_stride,
                    const int32_t* lens, int32_t batch, int32_t max_len, const void* k_new,
                    const void* v_new, int32_t in_dtype, const void* q, int32_t q_dtype,
                    int32_t n_q_heads, float scale, void* out, void* workspace,
                    uint64_t workspace_bytes, int32_t split_tokens, uint32_t flags,
                    void* stream);

/* Decode attention (and, with k_new, the decode step's row write) for a
 * batch whose sequences share their first prefix_len tokens: the pages that
 * hold them are listed once, in prefix_pages, and every table row lists the
 * same pages first (the refcounted sharing of libmir-metal
 * PagedStore::snapshot; tiny-llm paged_kv.py: one block serves every reader).
 * The results are those of pkv_decode_step / pkv_paged_attend over the same
 * tables, computed so that the shared pages are read once for all sequences:
 * a prefix pass attends over them with (sequence, query head) pairs as the
 * columns of its matrix-core tiles, the split pass covers only each
 * sequence's tokens past prefix_len (both in one launch, the prefix waves
 * beside the split pass's), and the combine merges them.
 *   prefix_pages  device int32 [prefix_len / page_size]; prefix_len a
 *                 positive multiple of page_size within the table row.
 *                 Sequence b sees t < min(lens[b], prefix_len) of the shared
 *                 tokens; its table row must list prefix_pages for those
 *                 tokens (a row that does not is reported as PKV_DEV_PREFIX
 *                 and its result is wrong).
 *   k_new, v_new  null (attend only) or device bf16 [batch][n_kv_heads]
 *                 [head_dim]: row b is written at position lens[b] - 1 and
 *                 attended, as in pkv_decode_step; a position inside the
 *                 shared prefix is not written and sets PKV_DEV_PREFIX.
 *   workspace     at least pkv_prefix_workspace_size bytes, 256-byte aligned,
 *                 zeroed once (as for pkv_paged_attend).
 *   next_upd      null, or n_next_upd block-table updates for the next step,
 *                 in pkv_table_apply's form (int32 [n][3]: sequence, logical
 *                 block, page; device memory or pinned host memory, read in
 *                 place): the step's launch writes them into the table, so a
 *                 decode loop needs no table-update launch of its own (the
 *                 host grows its tables one step ahead: tiny-llm paged_kv.py
 *                 begin_step, applied with the previous step).  Each must name
 *                 an entry this step does not read, block * page_size >=
 *                 lens[b]; one that does is skipped and sets
 *                 PKV_DEV_TABLE_NEXT.  Rows outside the table are skipped, as
 *                 by pkv_table_apply.  The host must neither change nor free
 *                 the list until the stream has run the step.  The table is
 *                 written only through these updates.
 *   flags         0 or PKV_ATTEND_COMBINE_KERNEL (EINVAL otherwise).
 * Matrix-core shapes only (bf16/int8 pages, bf16 q, head_dim 64/128, page
 * size 16 or a multiple of 32, groups of at most 16): EFORMAT otherwise.
 * Other arguments and errors as pkv_decode_step. */
int pkv_prefix_workspace_size(const pkv_cache* cache, int32_t batch, int32_t n_q_heads,
                              int32_t max_len, int32_t prefix_len, int32_t split_tokens,
                              uint64_t* bytes);
int pkv_decode_step_prefix(pkv_cache* cache, int32_t layer, int32_t* table,
                           int32_t table_stride, const int32_t* lens, int32_t batch,
                           int32_t max_len, const int32_t* prefix_pages, int32_t prefix_len,
                           const void* k_new, const void* v_new, int32_t in_dtype, const void* q,
                           int32_t q_dtype, int32_t n_q_heads, float scale, void* out,
                           void* workspace, uint64_t workspace_bytes, const int32_t* next_upd,
                           int32_t n_next_upd, int32_t split_tokens, uint32_t flags,
                           void* stream);

/* Several queries per sequence (a chunk of new tokens, as in chunked
 * prefill).  Sequence b's T_b = cu_q[b+1] - cu_q[b] query rows stand for its
 * last T_b tokens, which a page write has already stored (AstrAI cache.py
 * PagedCache.write with seq_len > 1): row cu_q[b] + i sits at position
 * lens[b] - T_b + i and attends to the tokens t <= that position (the
 * valid-slot rule of metrale_storage high_speed_swap/impl_more.rs: a query
 * at q_pos sees the first q_pos % page_size + 1 slots of its own block; with
 * T_b = 1 this is pkv_paged_attend).  Query head h uses KV head
 * h / (n_q_heads / n_kv_heads).  A row whose position is below 0 gives zeros.
 *   q          device [total_q][n_q_heads][head_dim] bf16 (q_dtype must be
 *              PKV_DT_BF16); out the same shape, bf16 rounded to nearest even.
 *   table      device int32 [batch][table_stride].
 *   lens       device int32 [batch], stored tokens (chunk included); max_len a
 *              host upper bound on them, at most table_stride * page_size.
 *   cu_q       device int32 [batch + 1], non-decreasing, cu_q[0] = 0,
 *              cu_q[batch] = total_q; max_q a host upper bound on T_b.
 * Matrix-core kernel only: BF16 or INT8 pages, head_dim 64 or 128, page_size
 * 16 or a multiple of 32, n_q_heads / n_kv_heads at most 16; other shapes
 * return EFORMAT.  No workspace: every row is computed whole by one wave.
 * Device-side, malformed cu_q / chunk lengths set PKV_DEV_QROWS (see there);
 * lens are clamped as in pkv_paged_attend.  Nothing is synchronised. */
int pkv_paged_attend_multi(pkv_cache* cache, int32_t layer, const void* q, int32_t q_dtype,
                           int32_t n_q_heads, const int32_t* table, int32_t table_stride,
                           const int32_t* lens, const int32_t* cu_q, int32_t batch,
                           int32_t total_q, int32_t max_q, int32_t max_len, float scale,
                           void* out, void* stream);

/* gather(table, len): rows 0 .. len-1 of one sequence copied out in token
 * order (AstrAI cache.py PagedCache.gather truncated by CacheView;
 * libmir-metal PagedStore::context).  k_out, v_out: device
 * [len][n_kv_heads][head_dim] in the page element type (int8 pages give raw
 * codes); k_scale_out, v_scale_out: device float32 [len][n_kv_heads], int8
 * only (ignored otherwise).  Only table_row[0 .. ceil(len/page_size)-1] is
 * read.  Kept to compare the in-place read against a gather-first one. */
int pkv_gather(pkv_cache* cache, int32_t layer, const int32_t* table_row, int32_t len,
               void* k_out, void* v_out, float* k_scale_out, float* v_scale_out, void* stream);

/* Copy n pages: for every (src, dst) pair of the device int32 [n][2] list
 * and every layer, page src's K and V (all KV heads) and, for int8 pages,
 * its scales are copied to page dst.  This is the device half of
 * copy-on-write (pkv_seqs_take_copies hands out the pairs); run it before any
 * write into the dst pages.  The copies of one call run concurrently: no dst
 * may also be a src of the same call.  Pairs with an id outside the pool are
 * skipped and set PKV_DEV_WRITE_PAGE. */
int pkv_copy_pages(pkv_cache* cache, const int32_t* pairs, int32_t n, void* stream);

/* Apply n block-table updates: table[upd[3i] * table_stride + upd[3i+1]] =
 * upd[3i+2], with upd an int32 [n][3] list (sequence, logical block,
 * physical page), as tiny-llm paged_kv.py's begin_step mirrors newly
 * allocated blocks into its device table.  upd is device memory or pinned
 * host memory (hipHostMalloc), which the kernel reads in place, so a host
 * list needs no copy launch; the host must neither change nor free it until
 * the stream has run the update.  EINVAL if upd is neither device memory nor
 * pinned host memory.  Entries outside the table are skipped. */
int pkv_table_apply(int32_t* table, int32_t table_stride, int32_t batch, const int32_t* upd,
                    int32_t n, void* stream);

/* Copy the cache's device status word (the PKV_DEV_* bits the kernels have
 * OR-ed in) to host *out, after everything already enqueued on `stream`:
 * this call synchronises the stream, so it is meant for tests and checks,
 * not for a decode loop.  EHIP if the copy or the wait fails. */
int pkv_read_device_status(pkv_cache* cache, void* stream, int32_t* out);

const char* pkv_last_error(void);

/* ---- measurement -----------------------------------------------------------
 * Kernel timing: while enabled on a cache, pkv_paged_write, pkv_paged_attend,
 * pkv_decode_step and pkv_gather launch each kernel pass with a pair of HIP
 * events (created by the library) that the kernel's own dispatch stamps
 * with its start and end, so no marker packet is added between kernels;
 * nothing else changes.
 * pkv_timing_read waits for the recorded events, returns the summed
 * milliseconds and the number of passes timed per kind (PKV_T_*), then
 * forgets them.  ms[] and counts[] are host arrays of PKV_T_COUNT entries. */
#define PKV_T_WRITE 0
#define PKV_T_ATTEND_SPLIT 1  /* the split-K partial pass */
#define PKV_T_ATTEND_COMBINE 2
#define PKV_T_GATHER 3
#define PKV_T_ATTEND_MULTI 4
#define PKV_T_COPY_PAGES 5
#define PKV_T_COUNT 6
int pkv_timing_enable(pkv_cache* cache, int32_t on);
int pkv_timing_read(pkv_cache* cache, double* ms, int32_t* counts);

/* Streaming probes, the denominators of a bandwidth figure: mode 0 reads
 * `bytes` from src in order (16-byte loads, every byte once, 4 KiB blocks per
 * wave; one float per workgroup goes to sink); mode 2 reads the same 4 KiB
 * blocks in a scrambled order, as the pages of a fragmented pool are read
 * (bytes must then be 4 KiB times a power of two, EINVAL otherwise); mode 1
 * copies src to dst.  bytes must be a multiple of 16 and both pointers
 * 16-byte aligned.  pkv_probe_blocks gives the sink length modes 0 and 2
 * need. */
int32_t pkv_probe_blocks(uint64_t bytes);
int pkv_probe_stream(const void* src, void* dst, float* sink, uint64_t bytes, int32_t mode,
                     void* stream);

/* ---- host page pool (refcounted) ---------------------------------------
 * AstrAI cache.py PagedCache.alloc / alloc_n / free: the lowest free page is
 * handed out with count 1; alloc_n is all-or-nothing; release drops one
 * reference and the page is free again at zero.  retain adds one (the
 * sharing of libmir-metal PagedStore::snapshot).  Releasing or retaining a
 * page that is not in use is EDOUBLEFREE / EINVAL (tiny-llm BlockAllocator).
 * One pool is used from one thread at a time.
 *   shuffle_seed  0: lowest free page first (AstrAI's rule).  Otherwise the
 *                 pages are ranked by one SplitMix64 draw each (page i gets
 *                 output i of the generator seeded with shuffle_seed, ties by
 *                 page id) and the free page of lowest rank is handed out
 *                 first, so a fresh pool hands out a seeded permutation of
 *                 its pages, the shuffled page ids of a fragmented cache. */
typedef struct pkv_pool pkv_pool;
int pkv_pool_create(int32_t n_pages, uint64_t shuffle_seed, pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);
int pkv_pool_alloc(pkv_pool* pool, int32_t* id);                /* ENOMEM when full */
int pkv_pool_alloc_n(pkv_pool* pool, int32_t n, int32_t* ids); /* host ids[n]; ENOMEM, nothing granted */
int pkv_pool_retain(pkv_pool* pool, int32_t id);
int pkv_pool_release(pkv_pool* pool, int32_t id);
int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t id);    /* -1 for an id outside the pool */
int32_t pkv_pool_num_free(const pkv_pool* pool);

/* ---- host block tables over a pool --------------------------------------
 * batch sequences, each with a host table row of table_stride entries (-1
 * past its pages) and a length.  Growth allocates pages from the pool as a
 * sequence's length crosses a page boundary (tiny-llm begin_step;
 * libmir-metal allocation::ensure), sharing retains another sequence's
 * pages, release returns them.  Every change to a table entry is also queued
 * as an update triple for pkv_table_apply, so the device copy of the table
 * follows without re-sending the whole table. */
typedef struct pkv_seqs pkv_seqs;
int pkv_seqs_create(pkv_pool* pool, int32_t batch, int32_t table_stride, int32_t page_size,
                    pkv_seqs** out);
void pkv_seqs_destroy(pkv_seqs* seqs); /* releases every page still held */
/* Grow sequence b by n tokens (allocating pages as needed, all or nothing):
 * ENOMEM leaves the sequence unchanged, ERANGE if the row would overflow. */
int pkv_seqs_append(pkv_seqs* seqs, int32_t b, int32_t n);
/* Grow every sequence b by n[b] tokens (host int32 [batch], each >= 0) in
 * one call, all or nothing over the batch: pages go out as if
 * pkv_seqs_append(b, n[b]) ran for b = 0, 1, ... in order; ENOMEM or ERANGE
 * (checked for every sequence first) leave every sequence unchanged. */
int pkv_seqs_append_all(pkv_seqs* seqs, const int32_t* n);
/* Sequence dst (which must be empty) shares the first n_pages pages of src:
 * each gets one more reference.  Its length becomes n_pages * page_size. */
int pkv_seqs_share(pkv_seqs* seqs, int32_t dst, int32_t src, int32_t n_pages);
/* Sequence dst (which must be empty) becomes a copy of src that shares all
 * of its pages, a partly filled last page included, with one more reference
 * each, and takes its length (libmir-metal PagedStore::snapshot).
 * Copy-on-write: whenever an append (pkv_seqs_append, pkv_seqs_append_all)
 * would write into a sequence's last page while that page is partly filled
 * and held by another sequence as well, the sequence gets a fresh page in its
 * place, drops its reference to the shared one and queues a (shared, fresh)
 * page copy for pkv_copy_pages. */
int pkv_seqs_fork(pkv_seqs* seqs, int32_t dst, int32_t src);
/* Make room for appending n[b] tokens to every sequence (host int32
 * [batch]): while the pages those appends need (copies included) exceed the
 * free pages, the sequence admitted last (by its first append, share or fork)
 * among those holding tokens is preempted: its pages are released and its
 * length becomes 0, for the caller to requeue (tiny-llm paged_kv.py
 * reserve_step, which frees the newest sequences first).  Writes the
 * preempted sequences, newest first, to host victims[cap] (cap >= batch) and
 * returns their number, or a negative status (ERANGE if an append would
 * overflow its row). */
int32_t pkv_seqs_reserve(pkv_seqs* seqs, const int32_t* n, int32_t* victims, int32_t cap);
/* Move up to cap queued (src, dst) page copies into host pairs[cap][2];
 * returns the number moved (the rest stay queued), or a negative status. */
int32_t pkv_seqs_take_copies(pkv_seqs* seqs, int32_t* pairs, int32_t cap);
int pkv_seqs_release(pkv_seqs* seqs, int32_t b);
const int32_t* pkv_seqs_table(const pkv_seqs* seqs); /* host [batch][table_stride] */
const int32_t* pkv_seqs_lens(const pkv_seqs* seqs);  /* host [batch] */
/* Move up to cap queued update triples into host upd[cap][3]; returns the
 * number moved (the rest stay queued), or a negative status. */
int32_t pkv_seqs_take_updates(pkv_seqs* seqs, int32_t* upd, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
