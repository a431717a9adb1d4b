// Internal declarations shared by the host library and the HIP kernels:
// the plan the device-side planner writes into the caller's workspace, the
// kernel parameter blocks, and the launch entry points of each kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa.h"

namespace rpa {

// ---------------------------------------------------------------------------
// Tunables of the plan.
// ---------------------------------------------------------------------------
// Row-kernel work: the visible key ranges of the rows, in row order, form one
// stream cut into at most row_chunks_max(resident row-kernel waves, Hkv)
// chunks (one per resident wave and kv head, never more than kTargetItems)
// of at least kMinSplit keys; a chunk's pieces of rows are the items, so
// there are at most chunks + rows items, at most 2 * chunks split partials
// (the rows cut by a chunk boundary) and fewer than chunks split rows.
constexpr int kTargetItems = 2048;    // chunks at most
// Never cut a row's KV range finer than kMinSplit keys.  Finer pieces add
// partials to merge without speeding up the row kernel: a long row over few
// kv heads (one 200K-key row at Hkv 1) ran 80 us in all at 128 keys, 51 us at
// 256; at 512 the row kernel of small batches had too few waves.
constexpr int kMinSplit = 256;
// Chunks the planner may make for a row kernel with this many resident waves;
// the row kernel is launched with this many waves per kv head.
__host__ __device__ inline int row_chunks_max(int row_waves, int Hkv) {
  const int c = row_waves / (Hkv > 0 ? Hkv : 1);
  return c < 1 ? 1 : (c > kTargetItems ? kTargetItems : c);
}
// Side by side (co_run): the row kernel keeps kCoRowEighths / 8 of its
// resident waves and the prefill kernel takes the rest of each CU's slots.
// An even split gives every CU one workgroup of each; with 5/8 the rows'
// equal chunks ran unevenly (mixed bf16 batch: 0.490 against 0.461 ms).
constexpr int kCoRowEighths = 4;
constexpr int kPlanThreads = 1024;    // the planner is one workgroup
constexpr int kPlanCacheSeqs = 4000;  // planner keeps per-sequence data in LDS up to this (48 KB)
// dynamic LDS words of the planner for max_num_seqs sequences
inline int plan_lds_words(int max_num_seqs) {
  return (max_num_seqs + 1) * (max_num_seqs <= kPlanCacheSeqs ? 3 : 1);
}
constexpr int kWavesPerWG = 4;        // row kernel: one item per wave
constexpr int kPrefillBQ = 128;       // query tokens per prefill tile (4 waves x 32)

// ---------------------------------------------------------------------------
// Plan layout in the workspace (all offsets 256-byte aligned).
// ---------------------------------------------------------------------------
struct PlanHeader {
  int32_t num_seqs;      // min(sum(distribution), max_num_seqs)
  int32_t n_rows;        // query rows handled by the row kernel
  int32_t n_items;       // (row, split) items of the row kernel
  int32_t split;         // C, keys per chunk
  int32_t n_merge_rows;  // rows with more than one split
  int32_t n_pf_items;    // (sequence, query tile) items of the prefill kernel
  int32_t row_next;      // work counter of the row kernel (zeroed by the planner)
  int32_t pf_next;       // work counter of the prefill kernel (zeroed by the planner)
  int32_t n_chunks;      // chunks of the row kernel (chunk c = items [first[c], first[c+1]))
  int32_t co_run;        // 1: row and prefill kernels share the CUs (half the resident waves each)
  int32_t pad[6];
};

struct RowDesc {         // one query row of the row (decode) kernel
  int32_t token;         // row index into queries / out
  int32_t seq;
  int32_t lo, hi;        // visible key range [lo, hi) of this row
  int32_t n_split;
  int32_t part_base;     // first partial slot (n_split > 1), else -1
  int32_t pad[2];
};

struct ItemDesc {        // a split of one row: keys [lo, hi)
  int32_t token;         // row index into queries / out
  int32_t seq;
  int32_t lo, hi;
  int32_t part;          // partial slot, or -1 when the row has a single split
  int32_t row;
  int32_t pad[2];
};

struct MergeDesc {       // a row with more than one split, for the merge
  int32_t token;         // row index into queries / out
  int32_t part_base;     // its first partial slot
  int32_t n_split;       // its number of partials
  int32_t pad;
};

struct PrefillItem {     // a query tile of one prefill sequence
  int32_t seq;
  int32_t q_begin, q_end;  // query offsets within the sequence, [q_begin, q_end)
  int32_t pad;
};

constexpr int kZeroBytes = 1024;      // zero-filled source row for masked key loads

struct Workspace {       // byte offsets into the caller's workspace
  size_t header, zeros, rows, items, chunks, merge_rows, pf_items, part_ml, part_acc, total;
  int32_t max_rows, max_items, max_parts, max_pf_items, max_merge_rows;
  int32_t max_chunks;    // chunks of the row kernel at most (entries of the chunk table - 1)
};

Workspace workspace_layout(const rpa_desc& d, const rpa_options& o);

// Routing of sequences: rows of sequences with q_len >= prefill_min_q go to the
// MFMA prefill kernel (when the dtype has one), all others to the row kernel.
int prefill_min_q(const rpa_desc& d);

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value).
// ---------------------------------------------------------------------------
struct ScatterParams {
  const void* keys;
  const void* values;
  void* cache;
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* dist;
  int32_t T, max_num_seqs, pps, page_size, Hkv, D, Dpad;
  float inv_k_scale_src, inv_v_scale_src;  // the scales themselves (division done in-kernel)
  int32_t skip_min_q;    // tokens of sequences with q_len >= this are left to the prefill
                         // kernel (the fused update); INT_MAX: write every token
};

struct SlotMapParams {    // flat slot of each new token row
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* dist;
  int64_t* slots;
  int32_t T, max_num_seqs, pps, page_size;
};

struct ReshapeParams {    // new K / V rows into split caches by flat slot
  const void* keys;
  const void* values;
  void* key_cache;
  void* value_cache;
  const int64_t* slots;
  int64_t num_slots;      // num_blocks * block_size; slots outside [0, num_slots) are skipped
  int32_t T, Hkv, D, Dpad;
  float k_scale, v_scale;  // 1 when none
};

constexpr int kMaxCopyLayers = 64;

struct CopyBlocksParams {   // block copies within the split caches of every layer
  void* k[kMaxCopyLayers];
  void* v[kMaxCopyLayers];
  const int64_t* pairs;     // [num_pairs][2] = (source, destination)
  int64_t num_blocks, block_bytes;
  int32_t num_layers, num_pairs;
};

struct PlanParams {
  const int32_t* kv_lens;
  const int32_t* qsl;
  const int32_t* dist;
  char* ws;
  Workspace lay;
  int32_t max_num_seqs, T, window, prefill_min_q, Hkv;
  int32_t row_waves;     // resident waves of the row kernel (chunks = row_waves / Hkv)
  int32_t Hq, D, kv_elem;  // q heads, head_dim, bytes per cache element
  int32_t co_allowed;    // the prefill kernel runs on its own stream beside the row kernel
};

struct AttnParams {
  const void* q;
  const void* cache;
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const int32_t* qsl;
  const float* sink;
  void* out;
  char* ws;
  Workspace lay;
  int32_t Hq, Hkv, D, Dpad, page_size, pps, window;
  int32_t ps_shift;    // log2(page_size)
  float qk_scale;      // softmax_scale * q_scale * k_scale
  float v_scale;       // 1 when none
  float cap;           // 0 when none
  int32_t fuse_merge;  // prefill kernel: first merge the row kernel's split partials
  // Fused update (the prefill kernel's sequences): new tokens (positions
  // >= kv_len - q_len) are read from new_k / new_v, [T, Hkv, D] rows of
  // in_row_bytes, in the cache's own element type, and written into the
  // cache by the unit of the first q head of each kv head's group.
  int32_t fuse_update;
  uint32_t in_row_bytes;
  const void* new_k;
  const void* new_v;
  // Set by launch_prefill when the two-group prefill kernel is launched too:
  // it takes the batch unless the planner runs the prefill beside the rows
  // (co_run), and prefill_kernel takes it only then.
  int32_t pf_pair;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_scatter(const ScatterParams& p, rpa_dtype in_dt, rpa_dtype cache_dt,
                          hipStream_t s);
// planner, plus the cache update when sp is non-NULL (one launch)
hipError_t launch_prep(const PlanParams& pp, const ScatterParams* sp, rpa_dtype in_dt,
                       rpa_dtype cache_dt, hipStream_t s);
hipError_t launch_rows(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt, hipStream_t s);
// waves of the row kernel for these types and sizes that fit on the device at once
int row_waves(rpa_dtype q_dt, rpa_dtype cache_dt, int D, int Dpad, int Hkv, int G, bool cap);
// The MFMA row kernel's shared-load form: kv heads in groups of 4 whose rows
// carry no lane padding (a workgroup's 4 waves then read 4 heads' K and V as
// one contiguous run per token).
inline bool row_shared_loads(int Hkv, int Dpad, int D) { return Hkv % 4 == 0 && Dpad == D; }
hipError_t launch_merge(const AttnParams& p, rpa_dtype q_dt, hipStream_t s);
hipError_t launch_prefill(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt,
                          hipStream_t s);
bool prefill_supported(const rpa_desc& d);
hipError_t launch_slot_mapping(const SlotMapParams& p, hipStream_t s);

struct ValidateParams {   // rpa_validate_metadata
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* dist;
  uint32_t* slot_bits;    // one bit per cache slot (num_pages * page_size)
  int32_t* status;        // OR of RPA_META_* bits
  long long slot_words;
  int32_t max_num_seqs, T, pps, page_size, num_pages;
};
hipError_t launch_validate(const ValidateParams& p, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s);
hipError_t launch_reshape_and_cache(const ReshapeParams& p, rpa_dtype in_dt, rpa_dtype cache_dt,
                                    hipStream_t s);

// Profiling hooks used by the launchers' caller.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// Tracing hooks of the launchers (RPA_TRACE=1, and rpa_trace_format's dry
// run): trace_active() says whether this thread's call is traced;
// trace_launch() records a launch's kernel and geometry and returns true when
// the launch must be skipped (dry run).
bool trace_active();
bool trace_launch(const char* kernel, unsigned grid, unsigned block, size_t lds, hipStream_t s);
// element type names for traced kernel names (float, uint16_t = bf16, uint8_t = e4m3)
template <typename T>
constexpr const char* elem_name() {
  return sizeof(T) == 4 ? "f32" : sizeof(T) == 2 ? "bf16" : "fp8";
}

}  // namespace rpa
