/*
 * rpa.h -- C ABI of the MI355X (gfx950) ragged paged attention library.
 *
 * Two operations, mirroring the ragged-paged-attention v3 interface (ejkernel
 * docs, "ragged_page_attention_v3" signature and parameter list):
 *
 *   rpa_update_kv_cache  writes each step's new K/V tokens into their pages
 *                        (tpu-inference v3 kernel diff, "_update_kv_cache").
 *   rpa_forward          optionally performs that update, then attention of
 *                        the concatenated ragged queries over the paged cache
 *                        (same diff, "flash_attention_step1_qk_softmax" and
 *                        "flash_attention_step2_pv"; the v3 call returns the
 *                        output and the updated cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *   never allocates, frees or copies caller memory, and never synchronises
 *   the stream.  All work is enqueued on `stream` (a hipStream_t, NULL = the
 *   default stream).
 * - All shape checks happen on the host before anything is enqueued: a call
 *   that returns an error has no side effect.
 * - Layouts (row-major, contiguous):
 *     queries            [total_tokens, num_q_heads, head_dim]      in q_dtype
 *     out                [total_tokens, num_q_heads, head_dim]      in q_dtype, or BF16
 *                        when q_dtype is FP8_E4M3
 *     keys, values       [total_tokens, num_kv_heads, head_dim]     in kv_in_dtype
 *     kv_cache           [num_pages, page_size, 2*num_kv_heads, head_dim_padded]
 *                        in cache_dtype.  This is the same memory as the v3
 *                        shape [num_pages, page_size, 2*num_kv_heads/kv_packing,
 *                        kv_packing, head_dim_padded]: combined head 2h holds
 *                        K of kv head h and 2h+1 holds its V (the v3 kernel
 *                        diff keeps a head's K and V in one packed row).  Lanes
 *                        [head_dim, head_dim_padded) are zero-filled on update.
 *     kv_lens            int32[max_num_seqs]   kv length INCLUDING the new tokens
 *     block_tables       int32[max_num_seqs * pages_per_seq]  page ids per sequence
 *     query_start_loc    int32[max_num_seqs + 1]  cumulative query lengths
 *     distribution       int32[3] = (decode, prefill, mixed) sequence counts;
 *                        num_seqs = their sum.  Entries of the metadata past
 *                        num_seqs are never read.
 *     attention_sink     float32[num_q_heads] or NULL
 * - Sequence s owns query rows [qsl[s], qsl[s+1]); its queries are the LAST
 *   q_len = qsl[s+1]-qsl[s] positions of a kv_len-token sequence (vLLM
 *   differential_flash_attn.py, context_len/query_len/seq_len diagram), so
 *   query t sits at position kv_len - q_len + t and sees keys j <= that
 *   position (and, with a window W > 0, the W most recent of them).
 * - Device-side preconditions (not checked by the update or the attention
 *   calls; rpa_validate_metadata checks them on the device):
 *   0 <= q_len <= kv_len <= pages_per_seq*page_size; qsl non-decreasing from
 *   0 with qsl[num_seqs] <= total_tokens; block-table entries that cover
 *   [0, kv_len) are < num_pages; the slots written by one update are
 *   distinct, and none of them holds a context key (a position below
 *   kv_len - q_len) of any sequence of the call: rpa_forward writes the new
 *   tokens of prefill sequences while it attends.  Block-table entries past
 *   ceil(kv_len/page_size) are not read.
 */
#ifndef RPA_H_
#define RPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  The pages raise NotImplementedError / ValueError / assert
 * for unsupported features, bad head sizes and shape mismatches (tpu-inference
 * layers/vllm/attention.py and vLLM differential_flash_attn.py); the C ABI
 * returns codes instead. */
enum {
  RPA_OK = 0,
  RPA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
  RPA_ERR_INVALID_SHAPE = 2,  /* non-positive or inconsistent sizes */
  RPA_ERR_UNSUPPORTED = 3,    /* head_dim / page_size / dtype combination not built */
  RPA_ERR_INVALID_OPTION = 4, /* negative window or cap, non-finite scale */
  RPA_ERR_WORKSPACE = 5,      /* workspace missing or smaller than rpa_workspace_bytes */
  RPA_ERR_HIP = 6             /* a HIP launch failed (see rpa_error_string) */
};

typedef enum {
  RPA_F32 = 0,
  RPA_BF16 = 1,
  RPA_FP8_E4M3 = 2 /* OCP e4m3fn: bias 7, max 448, no infinity, NaN = 0x7F/0xFF */
} rpa_dtype;

/* Static sizes of a call.  Passed by pointer, read on the host only. */
typedef struct rpa_desc {
  int32_t total_tokens;     /* rows of queries / keys / values / out */
  int32_t max_num_seqs;     /* length of kv_lens (query_start_loc has +1) */
  int32_t pages_per_seq;    /* row length of block_tables */
  int32_t num_pages;        /* pages in kv_cache */
  int32_t page_size;        /* tokens per page: 16, 32, 64 or 128 */
  int32_t num_q_heads;      /* multiple of num_kv_heads (GQA) */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t head_dim_padded;  /* >= head_dim; head_dim_padded*elem_size % 16 == 0 */
  int32_t q_dtype;          /* rpa_dtype of queries and out */
  int32_t kv_in_dtype;      /* rpa_dtype of keys / values */
  int32_t cache_dtype;      /* rpa_dtype of kv_cache */
} rpa_desc;
/* Supported (q, kv_in, cache) dtype triples: (F32, F32, F32),
 * (BF16, BF16, BF16), (BF16, BF16, FP8_E4M3), (BF16, FP8_E4M3, FP8_E4M3), and
 * with 8-bit queries ("w8a8", tpu-inference layers/vllm/attention.py,
 * quantisation block; the q_scale argument of the ejkernel interface):
 * (FP8_E4M3, BF16, FP8_E4M3), (FP8_E4M3, FP8_E4M3, FP8_E4M3).  E4M3 queries
 * are codes whose values are code * q_scale; their output is BF16. */

/* Scalar options of rpa_forward (the v3 keyword arguments). */
typedef struct rpa_options {
  float softmax_scale;      /* multiplies q.k (v3 default 1.0; pass it explicitly).  Any
                               finite value: 0 gives every visible key equal weight, a
                               negative scale favours the least similar keys */
  int32_t sliding_window;   /* 0 = off; W > 0: key j visible iff pos - j < W */
  float logits_soft_cap;    /* 0 = off; c > 0: s -> c * tanh(s / c), after all scales */
  float q_scale;            /* 0 = none (1.0); multiplies the logits (for e4m3 queries:
                               Q as read = stored code * q_scale) */
  float k_scale;            /* 0 = none (1.0); K as read = stored element * k_scale */
  float v_scale;            /* 0 = none (1.0); V as read = stored element * v_scale */
  int32_t chunk_prefill_size;      /* tuning hints; 0 = automatic; results do */
  int32_t num_kv_pages_per_block;  /* not depend on them */
  int32_t num_queries_per_block;
  int64_t lds_limit_bytes;         /* the v3 vmem_limit_bytes; 0 = automatic */
} rpa_options;

/* Paged KV-cache update (the scatter).
 *
 * For every valid sequence s and every t < q_len: with pos = kv_len - q_len + t,
 * page = block_tables[s*pages_per_seq + pos/page_size], off = pos % page_size,
 * and for every kv head h:
 *   kv_cache[page][off][2h  ][0:head_dim] = encode(keys  [qsl[s]+t][h][:], k_scale)
 *   kv_cache[page][off][2h+1][0:head_dim] = encode(values[qsl[s]+t][h][:], v_scale)
 *   lanes [head_dim, head_dim_padded) of both rows = 0.
 * No other byte of kv_cache changes.  encode() is a bit copy when
 * kv_in_dtype == cache_dtype; for an FP8_E4M3 cache fed with BF16 keys it is
 * the quantisation step applied before the v3 kernel ("quantize_kv" in
 * tpu-inference layers/vllm/attention.py): y = x / scale in float32 (IEEE
 * round-to-nearest-even), clamped to [-448, 448], rounded to the nearest
 * e4m3fn code with ties to even (NaN -> 0x7F with its sign).  A scale of 0
 * means 1.0.  The result is bit-exact and independent of launch geometry.
 * `distribution` supplies num_seqs.  Returns RPA_OK or an error code.
 */
int rpa_update_kv_cache(const rpa_desc* desc, const void* keys, const void* values,
                        void* kv_cache, const int32_t* kv_lens, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* distribution,
                        float k_scale, float v_scale, void* stream);

/* Flat cache slot of every new token row: the slot mapping of the update's
 * split-cache form (vLLM differential_flash_attn.py, the metadata builder's
 * "Compute slot mapping" step and its PAD_SLOT_ID padding).  For every valid
 * sequence s and t < q_len, with pos = kv_len - q_len + t:
 *   slot_mapping[qsl[s] + t] = block_tables[s*pages_per_seq + pos/page_size] * page_size
 *                              + pos % page_size,
 * the same (page, offset) rpa_update_kv_cache writes.  Rows qsl[num_seqs] ..
 * total_tokens-1 get -1 (padding).  slot_mapping is int64[total_tokens] in
 * device memory.  Uses total_tokens, max_num_seqs, pages_per_seq and
 * page_size of desc; the other fields are checked as for the other calls.
 * Returns RPA_OK or an error code. */
int rpa_slot_mapping(const rpa_desc* desc, const int32_t* kv_lens, const int32_t* block_tables,
                     const int32_t* query_start_loc, const int32_t* distribution,
                     int64_t* slot_mapping, void* stream);

/* The update in its slot-mapping form, into split K and V caches (vLLM
 * differential_flash_attn.py, populate_kv_cache: reshape_and_cache_flash on
 * kv_cache[0] and kv_cache[1] with the flattened slot mapping, the cache dtype
 * and the k/v scales).
 *   key_cache, value_cache  [num_pages, page_size, num_kv_heads, head_dim_padded]
 *                           in cache_dtype (num_pages = blocks, page_size = block size)
 *   keys, values            [total_tokens, num_kv_heads, head_dim] in kv_in_dtype
 *   slot_mapping            int64[total_tokens]
 * For every row i with 0 <= slot = slot_mapping[i] < num_pages*page_size and
 * every kv head h:
 *   key_cache  [slot/page_size][slot%page_size][h][0:head_dim] = encode(keys  [i][h][:], k_scale)
 *   value_cache[slot/page_size][slot%page_size][h][0:head_dim] = encode(values[i][h][:], v_scale)
 *   lanes [head_dim, head_dim_padded) of both rows = 0.
 * Rows with any other slot (-1 padding, or past the pool) are skipped, and no
 * other byte changes.  encode() is the one of rpa_update_kv_cache.  Slots of
 * one call must be distinct.  Returns RPA_OK or an error code. */
int rpa_reshape_and_cache(const rpa_desc* desc, const void* keys, const void* values,
                          void* key_cache, void* value_cache, const int64_t* slot_mapping,
                          float k_scale, float v_scale, void* stream);

/* Block copies within split caches, for every layer (vLLM
 * differential_flash_attn.py, copy_blocks: ops.copy_blocks on the K plane
 * kv_cache[0] and the V plane kv_cache[1] of every layer's cache with one
 * pair table).  For every layer l < num_layers and pair i < num_pairs with
 * (s, d) = (src_to_dst[2i], src_to_dst[2i+1]):
 *   key_caches[l] block d   = key_caches[l] block s
 *   value_caches[l] block d = value_caches[l] block s
 * A block is block_bytes bytes; a cache holds num_blocks of them.
 *   key_caches, value_caches  HOST arrays of num_layers DEVICE pointers
 *                             (16-byte aligned; num_layers <= 64)
 *   src_to_dst                DEVICE int64[2 * num_pairs]
 * Destinations must be distinct and none may also be a source (copies run
 * in parallel).  Pairs with an index outside [0, num_blocks) are skipped.
 * block_bytes must be a positive multiple of 16.  Returns RPA_OK or an
 * error code. */
int rpa_copy_blocks(void* const* key_caches, void* const* value_caches, int32_t num_layers,
                    int64_t num_blocks, int64_t block_bytes, const int64_t* src_to_dst,
                    int32_t num_pairs, void* stream);

/* Block moves between two caches, e.g. device and pinned host memory for
 * swapping (vLLM differential_flash_attn.py, swap_blocks: ops.swap_blocks on
 * the K plane and the V plane with one src_to_dst table; call once per
 * plane).  For every pair i: dst block src_to_dst[2i+1] = src block
 * src_to_dst[2i], block_bytes bytes each, one async copy per pair on
 * `stream`.  src_to_dst is a HOST int64[2 * num_pairs] (it drives the copies
 * from the host).  Host memory must be pinned (hipHostMalloc) for the copies
 * to be asynchronous.  Pairs outside [0, src_blocks) x [0, dst_blocks) are
 * rejected with RPA_ERR_INVALID_SHAPE before any copy is enqueued.  Returns
 * RPA_OK or an error code. */
int rpa_swap_blocks(const void* src_cache, void* dst_cache, int64_t src_blocks,
                    int64_t dst_blocks, int64_t block_bytes, const int64_t* src_to_dst,
                    int32_t num_pairs, void* stream);

/* Bytes of device workspace rpa_forward needs for these sizes and options
 * (plan, work lists and split-KV partial results).  Writes *bytes; returns a
 * status code (the same host checks rpa_forward makes). */
int rpa_workspace_bytes(const rpa_desc* desc, const rpa_options* opts, size_t* bytes);

/* Ragged paged attention (v3 semantics), optionally preceded by the update.
 *
 * If keys and values are both non-NULL, first performs exactly
 * rpa_update_kv_cache(desc, keys, values, kv_cache, ..., opts->k_scale,
 * opts->v_scale, stream); if both are NULL the cache is used as it is.
 * Then for every valid sequence s, query row r = qsl[s] + t (t < q_len) and
 * q head h (kv head g = h / (num_q_heads/num_kv_heads)):
 *   s_j  = softmax_scale * q_scale * k_scale * (q[r][h] . Kstored[s][j][g])
 *   s_j  = cap * tanh(s_j / cap)                       if cap > 0
 *   out[r][h] = sum_{j visible} e^{s_j} v_scale*Vstored[s][j][g]
 *               / (sum_{j visible} e^{s_j} + e^{sink[h]} if a sink is given)
 * computed with an online softmax in float32 and rounded (nearest even) to
 * q_dtype (BF16 for e4m3 queries).  Rows >= qsl[num_seqs] of `out` are not
 * written.  The result does
 * not depend on `distribution` beyond num_seqs, nor on the tuning hints.
 * `workspace` must hold rpa_workspace_bytes() bytes (device memory, caller
 * owned, contents need not be initialised; it is overwritten).
 * Concurrent calls must use distinct workspaces.
 * When the batch has more tokens than max_num_seqs (so some sequence has
 * prefill rows), the prefill kernel runs on a side stream of the library's:
 * one per (device, caller stream), created with two events on the first such
 * call from that stream and kept until the process ends.  It is forked off
 * `stream` after the planner and joined back before the call returns, so all
 * of the call's work is still ordered on `stream`, including under HIP graph
 * capture; calls from different streams never share a side stream, so a
 * capture on one stream does not reach calls made from another.
 */
int rpa_forward(const rpa_desc* desc, const rpa_options* opts, const void* queries,
                const void* keys, const void* values, void* kv_cache, const int32_t* kv_lens,
                const int32_t* block_tables, const int32_t* query_start_loc,
                const int32_t* distribution, const float* attention_sink, void* out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Tracing.  With the environment variable RPA_TRACE set (to anything but
 * "0"), every rpa_forward call writes its trace to stderr: one "[rpa] forward"
 * line with the sizes and options, one "[rpa] workspace" line with the byte
 * offset of every workspace section and the bounds they are sized for, one
 * "[rpa] streams" line, one "[rpa] launch" line per kernel (name, grid,
 * block, LDS bytes, stream), and a last "[rpa] plan" line with the plan
 * header the device wrote (its counts of rows, items, chunks, merges and
 * prefill tiles, and the side-by-side flag).  Reading the plan back
 * synchronises the stream, so it is skipped while the stream is being
 * captured into a graph.  The tpu-inference v3 kernel diff has the same kind
 * of switchable debug printing ("[RPA debug]" lines).
 *
 * rpa_trace_format writes into buf the trace an rpa_forward with these sizes
 * and options (with or without the update) would print before its plan line,
 * without touching any device memory or launching anything: the same checks,
 * workspace layout and launch sequence, run dry.  The text is NUL-terminated
 * and cut to buf_bytes - 1 characters; *text_bytes (if non-NULL) receives its
 * full length.  Returns the status rpa_forward would return from its host
 * checks. */
int rpa_trace_format(const rpa_desc* desc, const rpa_options* opts, int with_update, char* buf,
                     size_t buf_bytes, size_t* text_bytes);

/* Bytes of the library's own device scratch that rpa_forward_noalloc uses in
 * place of a workspace (one copy per GPU, held until the process ends). */
#define RPA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* rpa_forward without a workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc.  Same arguments and
 * results as rpa_forward minus the workspace: the plan, work lists and split
 * partials go to a device array of the library's, RPA_NOALLOC_SCRATCH_BYTES
 * per GPU.  Calls whose rpa_workspace_bytes() exceeds that return
 * RPA_ERR_WORKSPACE before touching the device.  The call allocates nothing
 * and creates nothing: every kernel runs on `stream` (no side stream for
 * prefill tiles, so mixed batches run their kernels one after another), no
 * profile events are recorded, and RPA_TRACE prints no plan line.  All calls
 * on one GPU share its scratch array, which keeps the last call's contents
 * (every call rewrites what it reads): calls that overlap on one GPU, from
 * different streams or threads, race and must be ordered by the caller. */
int rpa_forward_noalloc(const rpa_desc* desc, const rpa_options* opts, const void* queries,
                        const void* keys, const void* values, void* kv_cache,
                        const int32_t* kv_lens, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* distribution,
                        const float* attention_sink, void* out, void* stream);

/* Bits of the device status word written by rpa_validate_metadata. */
enum {
  RPA_META_QSL = 1,           /* qsl[0] != 0, qsl decreasing, or qsl[num_seqs] > total_tokens */
  RPA_META_LENS = 2,          /* kv_len < 0, q_len > kv_len, or kv_len > pages_per_seq*page_size */
  RPA_META_BLOCK_TABLE = 4,   /* an entry covering [0, kv_len) outside [0, num_pages) */
  RPA_META_SLOTS = 8,         /* two new tokens of the update map to one cache slot */
  RPA_META_DISTRIBUTION = 16, /* a negative count, or counts summing past max_num_seqs */
  RPA_META_WRITE_IN_CONTEXT = 32 /* a slot the update writes holds a context key of a sequence */
};

/* Device-side check of the metadata preconditions listed at the top of this
 * file, for the sizes in `desc` (total_tokens, max_num_seqs, pages_per_seq,
 * num_pages, page_size).  The pages state the cache-update rule (position
 * kv_len - q_len + t of a sequence goes to slot (block_tables page, offset))
 * but not what an inconsistent table does; the update and attention calls do
 * not check it on the device, so a caller can run this first.
 * Enqueues four small kernels on `stream` and returns without a host sync;
 * when they have run, *status (device int32) holds the OR of the RPA_META_*
 * bits of every violated precondition, 0 when all hold.  slot_bits is device
 * scratch of (num_pages * page_size + 31) / 32 uint32 words, caller owned,
 * contents need not be initialised (cleared by a fill kernel, so the call can
 * be captured in a HIP graph).  Every read stays inside the documented array
 * sizes whatever their contents.  Returns RPA_OK or a host-side error code
 * (NULL pointer, invalid shape, HIP launch failure).
 */
int rpa_validate_metadata(const rpa_desc* desc, const int32_t* kv_lens,
                          const int32_t* block_tables, const int32_t* query_start_loc,
                          const int32_t* distribution, uint32_t* slot_bits, int32_t* status,
                          void* stream);

/* Human-readable text of a status code (for RPA_ERR_HIP, includes the last
 * HIP error seen by the library). */
const char* rpa_error_string(int status);

/* Kernel timing for measurement.  While enabled, every kernel the library
 * launches is bracketed by a pair of hipEvents recorded on the launch stream.
 * rpa_profile_read() waits for the recorded events, writes up to `max`
 * per-kernel aggregates and clears the record; it returns the number of
 * kernels written, or a negative status.  Off by default. */
typedef struct rpa_kernel_stat {
  char name[32];      /* kernel name */
  int32_t launches;   /* number of launches recorded */
  double total_ms;    /* summed event-to-event duration */
} rpa_kernel_stat;

int rpa_profile_enable(int on);
int rpa_profile_read(rpa_kernel_stat* stats, int max);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H_ */
