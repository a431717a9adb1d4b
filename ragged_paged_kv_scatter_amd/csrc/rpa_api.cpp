// Host side of the C ABI: argument validation (all before any launch),
// workspace layout, kernel sequencing on the caller's stream, error strings
// and the optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "rpa.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

thread_local std::string g_last_hip_error;

int elem_size(int dt) { return dt == RPA_F32 ? 4 : dt == RPA_BF16 ? 2 : 1; }

bool valid_dtype(int dt) { return dt == RPA_F32 || dt == RPA_BF16 || dt == RPA_FP8_E4M3; }

bool supported_triple(int q, int in, int c) {
  return (q == RPA_F32 && in == RPA_F32 && c == RPA_F32) ||
         (q == RPA_BF16 && in == RPA_BF16 && c == RPA_BF16) ||
         (q == RPA_BF16 && in == RPA_BF16 && c == RPA_FP8_E4M3) ||
         (q == RPA_BF16 && in == RPA_FP8_E4M3 && c == RPA_FP8_E4M3) ||
         (q == RPA_FP8_E4M3 && in == RPA_BF16 && c == RPA_FP8_E4M3) ||
         (q == RPA_FP8_E4M3 && in == RPA_FP8_E4M3 && c == RPA_FP8_E4M3);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

constexpr int kMaxSeqs = 16000;  // planner keeps a per-sequence table in LDS

int check_desc(const rpa_desc* d) {
  if (!d) return RPA_ERR_NULL_POINTER;
  if (d->total_tokens < 0 || d->max_num_seqs < 0 || d->pages_per_seq <= 0 ||
      d->num_pages <= 0 || d->page_size <= 0 || d->num_q_heads <= 0 ||
      d->num_kv_heads <= 0 || d->head_dim <= 0 || d->head_dim_padded < d->head_dim)
    return RPA_ERR_INVALID_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return RPA_ERR_INVALID_SHAPE;
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_in_dtype) || !valid_dtype(d->cache_dtype))
    return RPA_ERR_UNSUPPORTED;
  if (!supported_triple(d->q_dtype, d->kv_in_dtype, d->cache_dtype)) return RPA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return RPA_ERR_UNSUPPORTED;
  const int ps = d->page_size;
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128) return RPA_ERR_UNSUPPORTED;
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return RPA_ERR_UNSUPPORTED;
  if (((long long)d->head_dim_padded * elem_size(d->cache_dtype)) % 16 != 0)
    return RPA_ERR_UNSUPPORTED;
  if (d->max_num_seqs > kMaxSeqs) return RPA_ERR_UNSUPPORTED;
  return RPA_OK;
}

int check_meta(const void* kv_lens, const void* bt, const void* qsl, const void* dist) {
  if (!kv_lens || !bt || !qsl || !dist) return RPA_ERR_NULL_POINTER;
  return RPA_OK;
}

int check_options(const rpa_options* o) {
  if (!o) return RPA_ERR_NULL_POINTER;
  if (!std::isfinite(o->softmax_scale)) return RPA_ERR_INVALID_OPTION;
  if (o->sliding_window < 0) return RPA_ERR_INVALID_OPTION;
  if (!finite_nonneg(o->logits_soft_cap)) return RPA_ERR_INVALID_OPTION;
  if (!finite_nonneg(o->q_scale) || !finite_nonneg(o->k_scale) || !finite_nonneg(o->v_scale))
    return RPA_ERR_INVALID_OPTION;
  if (o->chunk_prefill_size < 0 || o->num_kv_pages_per_block < 0 ||
      o->num_queries_per_block < 0 || o->lds_limit_bytes < 0)
    return RPA_ERR_INVALID_OPTION;
  return RPA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int hip_fail(hipError_t e) {
  g_last_hip_error = hipGetErrorString(e);
  return RPA_ERR_HIP;
}

// ---- profiling ------------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;
// A launch's begin and end are recorded by the thread that launches it, so
// the pending record is per thread: concurrent callers pair their own events.
thread_local ProfRec t_pending;
thread_local bool t_have_pending = false;
// Set during rpa_forward_noalloc: no profile events (creating one would
// allocate) and no plan read-back in the trace.
thread_local bool t_no_alloc = false;

// ---- tracing (RPA_TRACE=1, or rpa_trace_format's dry run) ------------------
// One call's trace: its sizes and options, the workspace layout, every launch
// with its geometry, and (RPA_TRACE only, outside graph capture) the plan
// header read back from the device.  In a dry run nothing is launched or
// recorded on a stream: the launchers report their geometry and return.
struct TraceState {
  bool on = false;
  bool dry = false;
  std::string* sink = nullptr;   // dry run: the text goes here, else to stderr
};
thread_local TraceState t_trace;

bool env_trace() {
  const char* v = std::getenv("RPA_TRACE");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

void trace_printf(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void trace_printf(const char* fmt, ...) {
  if (!t_trace.on) return;
  char buf[640];
  va_list ap;
  va_start(ap, fmt);
  const int n = std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (n <= 0) return;
  const size_t len = std::min((size_t)n, sizeof buf - 1);
  if (t_trace.sink) t_trace.sink->append(buf, len);
  else std::fwrite(buf, 1, len, stderr);
}

struct TraceScope {          // sets this thread's trace state for one call
  TraceState saved;
  TraceScope(bool on, bool dry, std::string* sink) : saved(t_trace) {
    t_trace.on = on;
    t_trace.dry = dry;
    t_trace.sink = sink;
  }
  ~TraceScope() {
    if (t_trace.on && !t_trace.sink) std::fflush(stderr);
    t_trace = saved;
  }
};

const char* dtype_name(int dt) {
  return dt == RPA_F32 ? "f32" : dt == RPA_BF16 ? "bf16" : dt == RPA_FP8_E4M3 ? "fp8_e4m3" : "?";
}

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---- side streams for the prefill kernel ----------------------------------
// rpa_forward forks the prefill kernel onto a side stream after the planner
// and joins it back before returning, so that prefill tiles can run beside
// the row kernel.  There is one side stream, with its fork / join events, per
// (device, caller stream): calls issued from different streams never share
// one, so a HIP graph capture on one stream cannot pull another stream's
// calls into it.  The record / wait pairs on one side stream are serialised
// by g_side_mu.  Side streams and their events live until the process ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::map<std::pair<int, hipStream_t>, SideStream> g_side;

// The side stream of `caller` (NULL: the current device's default stream),
// created on first use with the caller's device current; the caller holds
// g_side_mu.
hipError_t side_stream(hipStream_t caller, SideStream** out) {
  int dev = 0, cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (caller) {
    hipDevice_t d = 0;
    if ((e = hipStreamGetDevice(caller, &d)) != hipSuccess) return e;
    dev = d;
  }
  SideStream& ss = g_side[std::make_pair(dev, caller)];
  if (!ss.s) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e == hipSuccess && (e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) == hipSuccess)
      e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      if (f) (void)hipEventDestroy(f);
      if (st) (void)hipStreamDestroy(st);
      return e;
    }
    ss.s = st;
    ss.fork = f;
    ss.join = j;
  }
  *out = &ss;
  return hipSuccess;
}

}  // namespace

bool trace_active() { return t_trace.on; }

bool trace_launch(const char* kernel, unsigned grid, unsigned block, size_t lds, hipStream_t s) {
  trace_printf("[rpa] launch %s grid=%u block=%u lds=%zu stream=%p\n", kernel, grid, block, lds,
               (void*)s);
  return t_trace.dry;
}

void prof_begin(const char* name, hipStream_t s) {
  t_have_pending = false;
  if (t_trace.dry || t_no_alloc) return;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    t_pending.name = name;
    t_pending.start = take_event();
    t_pending.stop = take_event();
    if (!t_pending.start || !t_pending.stop) {
      if (t_pending.start) g_event_pool.push_back(t_pending.start);
      if (t_pending.stop) g_event_pool.push_back(t_pending.stop);
      return;
    }
  }
  t_have_pending = true;
  (void)hipEventRecord(t_pending.start, s);
}

void prof_end(hipStream_t s) {
  if (!t_have_pending) return;
  t_have_pending = false;
  (void)hipEventRecord(t_pending.stop, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_recs.push_back(t_pending);
}

bool prefill_supported(const rpa_desc& d);

int prefill_min_q(const rpa_desc& d) {
  return prefill_supported(d) ? 2 : INT_MAX;
}

// Resident waves of the row kernel for this call: the planner makes at most
// row_chunks_max(waves, Hkv) chunks, which bounds the work lists.
int row_waves_of(const rpa_desc& d, const rpa_options& o) {
  return row_waves((rpa_dtype)d.q_dtype, (rpa_dtype)d.cache_dtype, d.head_dim,
                   d.head_dim_padded, d.num_kv_heads, d.num_q_heads / d.num_kv_heads,
                   o.logits_soft_cap > 0.f);
}

Workspace workspace_layout(const rpa_desc& d, const rpa_options& o) {
  Workspace w = {};
  const long long T = d.total_tokens;
  const int pmq = prefill_min_q(d);
  long long max_rows = T;
  if (pmq != INT_MAX) max_rows = std::min<long long>(T, (long long)d.max_num_seqs * (pmq - 1));
  w.max_rows = (int32_t)std::max<long long>(max_rows, 1);
  // The rows' keys are cut into at most `chunks` chunks: every boundary
  // between two chunks adds one item and cuts at most one row, and a chunk
  // holds at most two pieces of rows it does not hold whole (its first and
  // its last), so there are at most 2 * chunks split partials and fewer than
  // `chunks` split rows.
  const int chunks = row_chunks_max(row_waves_of(d, o), d.num_kv_heads);
  w.max_chunks = chunks;
  w.max_items = chunks + w.max_rows;
  w.max_parts = std::min(2 * chunks, w.max_items);
  w.max_merge_rows = std::min(chunks, w.max_rows);
  w.max_pf_items = (pmq != INT_MAX)
                       ? (int32_t)((T + kPrefillBQ - 1) / kPrefillBQ + d.max_num_seqs + 1)
                       : 1;
  size_t off = 0;
  w.header = off;
  off = align256(off + sizeof(PlanHeader));
  w.zeros = off;
  off = align256(off + kZeroBytes);
  w.rows = off;
  off = align256(off + (size_t)w.max_rows * sizeof(RowDesc));
  w.items = off;
  off = align256(off + (size_t)w.max_items * sizeof(ItemDesc));
  w.chunks = off;
  off = align256(off + (size_t)(chunks + 1) * sizeof(int32_t));
  w.merge_rows = off;
  off = align256(off + (size_t)w.max_merge_rows * sizeof(MergeDesc));
  w.pf_items = off;
  off = align256(off + (size_t)w.max_pf_items * sizeof(PrefillItem));
  w.part_ml = off;
  off = align256(off + (size_t)w.max_parts * d.num_q_heads * 2 * sizeof(float));
  w.part_acc = off;
  off = align256(off + (size_t)w.max_parts * d.num_q_heads * d.head_dim * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace rpa

using namespace rpa;

extern "C" {

namespace {
ScatterParams scatter_params(const rpa_desc& d, const void* keys, const void* values,
                             void* kv_cache, const int32_t* kv_lens, const int32_t* block_tables,
                             const int32_t* qsl, const int32_t* dist, float k_scale,
                             float v_scale) {
  ScatterParams p = {};
  p.keys = keys;
  p.values = values;
  p.cache = kv_cache;
  p.kv_lens = kv_lens;
  p.block_tables = block_tables;
  p.qsl = qsl;
  p.dist = dist;
  p.T = d.total_tokens;
  p.max_num_seqs = d.max_num_seqs;
  p.pps = d.pages_per_seq;
  p.page_size = d.page_size;
  p.Hkv = d.num_kv_heads;
  p.D = d.head_dim;
  p.Dpad = d.head_dim_padded;
  p.inv_k_scale_src = k_scale > 0.f ? k_scale : 1.f;
  p.inv_v_scale_src = v_scale > 0.f ? v_scale : 1.f;
  p.skip_min_q = INT_MAX;
  return p;
}
}  // namespace

int rpa_update_kv_cache(const rpa_desc* desc, const void* keys, const void* values,
                        void* kv_cache, const int32_t* kv_lens, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* distribution,
                        float k_scale, float v_scale, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (!keys || !values || !kv_cache) return RPA_ERR_NULL_POINTER;
  if ((st = check_meta(kv_lens, block_tables, query_start_loc, distribution))) return st;
  if (!finite_nonneg(k_scale) || !finite_nonneg(v_scale)) return RPA_ERR_INVALID_OPTION;
  if (!aligned16(keys) || !aligned16(values) || !aligned16(kv_cache)) return RPA_ERR_INVALID_SHAPE;
  if (desc->total_tokens == 0 || desc->max_num_seqs == 0) return RPA_OK;
  const ScatterParams p = scatter_params(*desc, keys, values, kv_cache, kv_lens, block_tables,
                                         query_start_loc, distribution, k_scale, v_scale);
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_begin("scatter", s);
  hipError_t e = launch_scatter(p, (rpa_dtype)desc->kv_in_dtype, (rpa_dtype)desc->cache_dtype, s);
  prof_end(s);
  return e == hipSuccess ? RPA_OK : hip_fail(e);
}

int rpa_slot_mapping(const rpa_desc* desc, const int32_t* kv_lens, const int32_t* block_tables,
                     const int32_t* query_start_loc, const int32_t* distribution,
                     int64_t* slot_mapping, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (!slot_mapping) return RPA_ERR_NULL_POINTER;
  if ((st = check_meta(kv_lens, block_tables, query_start_loc, distribution))) return st;
  if (desc->total_tokens == 0) return RPA_OK;
  SlotMapParams p = {};
  p.kv_lens = kv_lens;
  p.block_tables = block_tables;
  p.qsl = query_start_loc;
  p.dist = distribution;
  p.slots = slot_mapping;
  p.T = desc->total_tokens;
  p.max_num_seqs = desc->max_num_seqs;
  p.pps = desc->pages_per_seq;
  p.page_size = desc->page_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_begin("slot_mapping", s);
  hipError_t e = launch_slot_mapping(p, s);
  prof_end(s);
  return e == hipSuccess ? RPA_OK : hip_fail(e);
}

int rpa_reshape_and_cache(const rpa_desc* desc, const void* keys, const void* values,
                          void* key_cache, void* value_cache, const int64_t* slot_mapping,
                          float k_scale, float v_scale, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (!keys || !values || !key_cache || !value_cache || !slot_mapping)
    return RPA_ERR_NULL_POINTER;
  if (!finite_nonneg(k_scale) || !finite_nonneg(v_scale)) return RPA_ERR_INVALID_OPTION;
  if (!aligned16(keys) || !aligned16(values) || !aligned16(key_cache) || !aligned16(value_cache))
    return RPA_ERR_INVALID_SHAPE;
  if (desc->total_tokens == 0) return RPA_OK;
  ReshapeParams p = {};
  p.keys = keys;
  p.values = values;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.slots = slot_mapping;
  p.num_slots = (int64_t)desc->num_pages * desc->page_size;
  p.T = desc->total_tokens;
  p.Hkv = desc->num_kv_heads;
  p.D = desc->head_dim;
  p.Dpad = desc->head_dim_padded;
  p.k_scale = k_scale > 0.f ? k_scale : 1.f;
  p.v_scale = v_scale > 0.f ? v_scale : 1.f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_begin("reshape_and_cache", s);
  hipError_t e = launch_reshape_and_cache(p, (rpa_dtype)desc->kv_in_dtype,
                                          (rpa_dtype)desc->cache_dtype, s);
  prof_end(s);
  return e == hipSuccess ? RPA_OK : hip_fail(e);
}

int rpa_copy_blocks(void* const* key_caches, void* const* value_caches, int32_t num_layers,
                    int64_t num_blocks, int64_t block_bytes, const int64_t* src_to_dst,
                    int32_t num_pairs, void* stream) {
  if (!key_caches || !value_caches || !src_to_dst) return RPA_ERR_NULL_POINTER;
  if (num_layers < 0 || num_layers > kMaxCopyLayers || num_pairs < 0 || num_blocks <= 0 ||
      block_bytes <= 0 || block_bytes % 16 != 0 || num_pairs > 65535)
    return RPA_ERR_INVALID_SHAPE;
  CopyBlocksParams p = {};
  for (int l = 0; l < num_layers; ++l) {
    if (!key_caches[l] || !value_caches[l]) return RPA_ERR_NULL_POINTER;
    if (!aligned16(key_caches[l]) || !aligned16(value_caches[l])) return RPA_ERR_INVALID_SHAPE;
    p.k[l] = key_caches[l];
    p.v[l] = value_caches[l];
  }
  if (num_layers == 0 || num_pairs == 0) return RPA_OK;
  p.pairs = src_to_dst;
  p.num_blocks = num_blocks;
  p.block_bytes = block_bytes;
  p.num_layers = num_layers;
  p.num_pairs = num_pairs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_begin("copy_blocks", s);
  hipError_t e = launch_copy_blocks(p, s);
  prof_end(s);
  return e == hipSuccess ? RPA_OK : hip_fail(e);
}

int rpa_swap_blocks(const void* src_cache, void* dst_cache, int64_t src_blocks,
                    int64_t dst_blocks, int64_t block_bytes, const int64_t* src_to_dst,
                    int32_t num_pairs, void* stream) {
  if (!src_cache || !dst_cache || (!src_to_dst && num_pairs > 0)) return RPA_ERR_NULL_POINTER;
  if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || block_bytes <= 0)
    return RPA_ERR_INVALID_SHAPE;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int64_t sb = src_to_dst[2 * i], db = src_to_dst[2 * i + 1];
    if (sb < 0 || sb >= src_blocks || db < 0 || db >= dst_blocks) return RPA_ERR_INVALID_SHAPE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* from = static_cast<const char*>(src_cache);
  char* to = static_cast<char*>(dst_cache);
  for (int32_t i = 0; i < num_pairs; ++i) {
    const hipError_t e = hipMemcpyAsync(to + src_to_dst[2 * i + 1] * block_bytes,
                                        from + src_to_dst[2 * i] * block_bytes,
                                        (size_t)block_bytes, hipMemcpyDefault, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return RPA_OK;
}

int rpa_validate_metadata(const rpa_desc* desc, const int32_t* kv_lens,
                          const int32_t* block_tables, const int32_t* query_start_loc,
                          const int32_t* distribution, uint32_t* slot_bits, int32_t* status,
                          void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_meta(kv_lens, block_tables, query_start_loc, distribution))) return st;
  if (!slot_bits || !status) return RPA_ERR_NULL_POINTER;
  ValidateParams p = {};
  p.kv_lens = kv_lens;
  p.block_tables = block_tables;
  p.qsl = query_start_loc;
  p.dist = distribution;
  p.slot_bits = slot_bits;
  p.status = status;
  p.slot_words = ((long long)desc->num_pages * desc->page_size + 31) / 32;
  p.max_num_seqs = desc->max_num_seqs;
  p.T = desc->total_tokens;
  p.pps = desc->pages_per_seq;
  p.page_size = desc->page_size;
  p.num_pages = desc->num_pages;
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_begin("validate", s);
  const hipError_t e = launch_validate(p, s);
  prof_end(s);
  return e == hipSuccess ? RPA_OK : hip_fail(e);
}

int rpa_workspace_bytes(const rpa_desc* desc, const rpa_options* opts, size_t* bytes) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_options(opts))) return st;
  if (!bytes) return RPA_ERR_NULL_POINTER;
  *bytes = workspace_layout(*desc, *opts).total;
  return RPA_OK;
}

}  // extern "C"

namespace {

// rpa_forward's work.  one_stream: every kernel on the caller's stream (no
// side stream, nothing created).  dry: check and trace only, launch nothing.
int forward_impl(const rpa_desc* desc, const rpa_options* opts, const void* queries,
                 const void* keys, const void* values, void* kv_cache, const int32_t* kv_lens,
                 const int32_t* block_tables, const int32_t* query_start_loc,
                 const int32_t* distribution, const float* attention_sink, void* out,
                 void* workspace, size_t workspace_bytes, hipStream_t s, bool one_stream,
                 bool dry) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_options(opts))) return st;
  if (!queries || !kv_cache || !out) return RPA_ERR_NULL_POINTER;
  if ((keys == nullptr) != (values == nullptr)) return RPA_ERR_NULL_POINTER;
  if ((st = check_meta(kv_lens, block_tables, query_start_loc, distribution))) return st;
  if (!aligned16(queries) || !aligned16(kv_cache) || !aligned16(out) ||
      (keys && (!aligned16(keys) || !aligned16(values))))
    return RPA_ERR_INVALID_SHAPE;
  const Workspace lay = workspace_layout(*desc, *opts);
  if (!workspace || workspace_bytes < lay.total || !aligned16(workspace)) return RPA_ERR_WORKSPACE;
  trace_printf("[rpa] forward total_tokens=%d max_num_seqs=%d pages_per_seq=%d num_pages=%d "
               "page_size=%d num_q_heads=%d num_kv_heads=%d head_dim=%d head_dim_padded=%d "
               "dtypes=%s/%s/%s update=%d softmax_scale=%g sliding_window=%d soft_cap=%g "
               "q_scale=%g k_scale=%g v_scale=%g sink=%d\n",
               desc->total_tokens, desc->max_num_seqs, desc->pages_per_seq, desc->num_pages,
               desc->page_size, desc->num_q_heads, desc->num_kv_heads, desc->head_dim,
               desc->head_dim_padded, dtype_name(desc->q_dtype), dtype_name(desc->kv_in_dtype),
               dtype_name(desc->cache_dtype), keys ? 1 : 0, opts->softmax_scale,
               opts->sliding_window, opts->logits_soft_cap, opts->q_scale, opts->k_scale,
               opts->v_scale, attention_sink ? 1 : 0);
  trace_printf("[rpa] workspace bytes=%zu header=%zu zeros=%zu rows=%zu items=%zu chunks=%zu "
               "merge_rows=%zu prefill_items=%zu part_ml=%zu part_acc=%zu max_rows=%d "
               "max_items=%d max_chunks=%d max_parts=%d max_merge_rows=%d max_prefill_items=%d\n",
               lay.total, lay.header, lay.zeros, lay.rows, lay.items, lay.chunks, lay.merge_rows,
               lay.pf_items, lay.part_ml, lay.part_acc, lay.max_rows, lay.max_items,
               lay.max_chunks, lay.max_parts, lay.max_merge_rows, lay.max_pf_items);
  if (desc->total_tokens == 0 || desc->max_num_seqs == 0) return RPA_OK;

  char* ws = static_cast<char*>(workspace);
  PlanParams pp = {};
  pp.kv_lens = kv_lens;
  pp.qsl = query_start_loc;
  pp.dist = distribution;
  pp.ws = ws;
  pp.lay = lay;
  pp.max_num_seqs = desc->max_num_seqs;
  pp.T = desc->total_tokens;
  pp.window = opts->sliding_window;
  pp.prefill_min_q = prefill_min_q(*desc);
  pp.Hkv = desc->num_kv_heads;
  pp.row_waves = row_waves_of(*desc, *opts);
  pp.Hq = desc->num_q_heads;
  pp.D = desc->head_dim;
  pp.kv_elem = elem_size(desc->cache_dtype);
  // More tokens than sequences means some sequence has two or more queries,
  // so the batch has prefill tiles: only then does the prefill kernel go to
  // the side stream (decode-only batches keep one stream and no fork / join).
  const bool side =
      !one_stream && prefill_supported(*desc) && desc->total_tokens > desc->max_num_seqs;
  pp.co_allowed = side ? 1 : 0;
  trace_printf("[rpa] streams %s row_waves=%d\n", side ? "caller+side" : "caller", pp.row_waves);
  // The update fused into the prefill kernel: when the new tokens are a bit
  // copy (no quantisation), the prefill kernel reads its sequences' new
  // tokens from keys / values and writes them into their pages itself; the
  // planner's launch then writes only the other sequences' tokens.
  const bool fuse = keys && prefill_supported(*desc) && desc->kv_in_dtype == desc->cache_dtype;
  // one launch: the planner, and the cache update when new tokens come along
  ScatterParams sp = {};
  if (keys) {
    sp = scatter_params(*desc, keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                        distribution, opts->k_scale, opts->v_scale);
    if (fuse) sp.skip_min_q = prefill_min_q(*desc);
  }
  trace_printf("[rpa] update %s\n", !keys ? "none" : fuse ? "fused (prefill sequences in the "
               "prefill kernel, the rest in prep_kernel)" : "prep_kernel");
  prof_begin(keys ? "plan+scatter" : "plan", s);
  hipError_t e = launch_prep(pp, keys ? &sp : nullptr, (rpa_dtype)desc->kv_in_dtype,
                             (rpa_dtype)desc->cache_dtype, s);
  prof_end(s);
  if (e != hipSuccess) return hip_fail(e);

  AttnParams ap = {};
  ap.q = queries;
  ap.cache = kv_cache;
  ap.kv_lens = kv_lens;
  ap.block_tables = block_tables;
  ap.qsl = query_start_loc;
  ap.sink = attention_sink;
  ap.out = out;
  ap.ws = ws;
  ap.lay = lay;
  ap.Hq = desc->num_q_heads;
  ap.Hkv = desc->num_kv_heads;
  ap.D = desc->head_dim;
  ap.Dpad = desc->head_dim_padded;
  ap.page_size = desc->page_size;
  ap.ps_shift = __builtin_ctz((unsigned)desc->page_size);
  ap.pps = desc->pages_per_seq;
  ap.window = opts->sliding_window;
  const float qs = opts->q_scale > 0.f ? opts->q_scale : 1.f;
  const float ks = opts->k_scale > 0.f ? opts->k_scale : 1.f;
  ap.qk_scale = opts->softmax_scale * qs * ks;
  ap.v_scale = opts->v_scale > 0.f ? opts->v_scale : 1.f;
  ap.cap = opts->logits_soft_cap;
  ap.fuse_update = fuse ? 1 : 0;
  ap.new_k = fuse ? keys : nullptr;
  ap.new_v = fuse ? values : nullptr;
  ap.in_row_bytes = (uint32_t)desc->num_kv_heads * desc->head_dim * elem_size(desc->kv_in_dtype);
  const rpa_dtype qd = (rpa_dtype)desc->q_dtype, cd = (rpa_dtype)desc->cache_dtype;

  if (!side) {
    // one stream: rows, then the prefill kernel (which first merges the
    // rows' split partials), or the stand-alone merge where the dtype has no
    // prefill kernel
    prof_begin("decode", s);
    e = launch_rows(ap, qd, cd, s);
    prof_end(s);
    if (e != hipSuccess) return hip_fail(e);
    if (prefill_supported(*desc)) {
      ap.fuse_merge = 1;
      prof_begin("prefill", s);
      e = launch_prefill(ap, qd, cd, s);
    } else {
      prof_begin("merge", s);
      e = launch_merge(ap, qd, s);
    }
    prof_end(s);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    // The rows and then the merge of their splits on the caller's stream,
    // the prefill tiles on the side stream; the caller's stream waits for
    // both.  The planner's co_run flag sizes both kernels to share the CUs
    // when the batch has enough of each kind of work.  The rows go first so
    // that their workgroups take CU slots before the persistent prefill grid
    // does: a row kernel that queues behind it starts late.
    std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
    SideStream dry_side;
    SideStream* ss = &dry_side;
    if (!dry) {
      lk.lock();
      if ((e = side_stream(s, &ss)) != hipSuccess) return hip_fail(e);
      if ((e = hipEventRecord(ss->fork, s)) != hipSuccess ||
          (e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess)
        return hip_fail(e);
    }
    ap.fuse_merge = 0;
    prof_begin("decode", s);
    e = launch_rows(ap, qd, cd, s);
    prof_end(s);
    if (e != hipSuccess) return hip_fail(e);
    prof_begin("prefill", ss->s);
    e = launch_prefill(ap, qd, cd, ss->s);
    prof_end(ss->s);
    if (e != hipSuccess) return hip_fail(e);
    if (!dry && (e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return hip_fail(e);
    prof_begin("merge", s);
    e = launch_merge(ap, qd, s);
    prof_end(s);
    if (e != hipSuccess) return hip_fail(e);
    if (!dry && (e = hipStreamWaitEvent(s, ss->join, 0)) != hipSuccess) return hip_fail(e);
  }
  if (t_trace.on && !dry && !t_no_alloc) {
    // the plan the device made (a synchronous read: tracing only, and never
    // while the stream is being captured)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    PlanHeader h = {};
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone &&
        hipMemcpyAsync(&h, ws + lay.header, sizeof h, hipMemcpyDeviceToHost, s) == hipSuccess &&
        hipStreamSynchronize(s) == hipSuccess)
      trace_printf("[rpa] plan num_seqs=%d rows=%d items=%d chunk_keys=%d chunks=%d "
                   "merge_rows=%d prefill_items=%d co_run=%d\n",
                   h.num_seqs, h.n_rows, h.n_items, h.split, h.n_chunks, h.n_merge_rows,
                   h.n_pf_items, h.co_run);
    else
      trace_printf("[rpa] plan not read back (stream capturing or not readable)\n");
  }
  return RPA_OK;
}

// Dummy device address for dry runs: aligned, never dereferenced.
void* dry_ptr() { return reinterpret_cast<void*>(uintptr_t(1) << 12); }

}  // namespace

extern "C" {

int rpa_forward(const rpa_desc* desc, const rpa_options* opts, const void* queries,
                const void* keys, const void* values, void* kv_cache, const int32_t* kv_lens,
                const int32_t* block_tables, const int32_t* query_start_loc,
                const int32_t* distribution, const float* attention_sink, void* out,
                void* workspace, size_t workspace_bytes, void* stream) {
  TraceScope ts(env_trace(), false, nullptr);
  return forward_impl(desc, opts, queries, keys, values, kv_cache, kv_lens, block_tables,
                      query_start_loc, distribution, attention_sink, out, workspace,
                      workspace_bytes, static_cast<hipStream_t>(stream), false, false);
}

}  // extern "C"

namespace {

// ---- allocation-free entry point ------------------------------------------
// The workspace of rpa_forward_noalloc: a device array of the library's own,
// one copy per GPU (its code object is loaded on each device it is used on
// and holds the array until the process ends).  In host code `scratch` names
// a host-side stand-in, not device memory: the device address of each GPU's
// copy comes from hipGetSymbolAddress with that device current, and only that
// address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = RPA_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of its copy of scratch

// The device address of the scratch array on the device of `s` (NULL: the
// current device), looked up once per device.
hipError_t scratch_address(hipStream_t s, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s) {
    hipDevice_t d = 0;
    if ((e = hipStreamGetDevice(s, &d)) != hipSuccess) return e;
    dev = d;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (dev != cur) (void)hipSetDevice(cur);
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

struct NoAllocScope {
  NoAllocScope() { t_no_alloc = true; }
  ~NoAllocScope() { t_no_alloc = false; }
};

}  // namespace

extern "C" {

int rpa_forward_noalloc(const rpa_desc* desc, const rpa_options* opts, const void* queries,
                        const void* keys, const void* values, void* kv_cache,
                        const int32_t* kv_lens, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* distribution,
                        const float* attention_sink, void* out, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_options(opts))) return st;
  if (workspace_layout(*desc, *opts).total > kNoAllocScratchBytes) return RPA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const hipError_t e = scratch_address(s, &ws);
  if (e != hipSuccess) return hip_fail(e);
  NoAllocScope na;
  TraceScope ts(env_trace(), false, nullptr);
  return forward_impl(desc, opts, queries, keys, values, kv_cache, kv_lens, block_tables,
                      query_start_loc, distribution, attention_sink, out, ws,
                      kNoAllocScratchBytes, s, true, false);
}

int rpa_trace_format(const rpa_desc* desc, const rpa_options* opts, int with_update, char* buf,
                     size_t buf_bytes, size_t* text_bytes) {
  std::string text;
  int st;
  {
    TraceScope ts(true, true, &text);
    void* d = dry_ptr();
    const int32_t* m = static_cast<const int32_t*>(d);
    st = forward_impl(desc, opts, d, with_update ? d : nullptr, with_update ? d : nullptr, d, m,
                      m, m, m, nullptr, d, d, SIZE_MAX, nullptr, false, true);
  }
  if (text_bytes) *text_bytes = text.size();
  if (buf && buf_bytes > 0) {
    const size_t n = std::min(text.size(), buf_bytes - 1);
    std::memcpy(buf, text.data(), n);
    buf[n] = 0;
  }
  return st;
}

const char* rpa_error_string(int status) {
  switch (status) {
    case RPA_OK: return "ok";
    case RPA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RPA_ERR_INVALID_SHAPE: return "invalid or inconsistent sizes, or a misaligned buffer";
    case RPA_ERR_UNSUPPORTED:
      return "unsupported configuration (head_dim 64/128, page_size 16/32/64/128, "
             "q/kv heads ratio 1/2/4/8/16, supported dtype triples only)";
    case RPA_ERR_INVALID_OPTION: return "invalid option (negative or non-finite value)";
    case RPA_ERR_WORKSPACE: return "workspace missing or smaller than rpa_workspace_bytes()";
    case RPA_ERR_HIP: {
      static thread_local std::string msg;
      msg = "HIP error: " + g_last_hip_error;
      return msg.c_str();
    }
    default: return "unknown status";
  }
}

int rpa_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return RPA_OK;
}

int rpa_profile_read(rpa_kernel_stat* stats, int max) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof_recs);
  }
  std::vector<rpa_kernel_stat> agg;
  int err = 0;
  for (auto& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      err = 1;
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (r.name == agg[i].name) break;
    if (i == agg.size()) {
      rpa_kernel_stat k = {};
      std::snprintf(k.name, sizeof(k.name), "%s", r.name.c_str());
      agg.push_back(k);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : recs) {
      g_event_pool.push_back(r.start);
      g_event_pool.push_back(r.stop);
    }
  }
  if (err) return -RPA_ERR_HIP;
  const int n = (int)std::min<size_t>(agg.size(), (size_t)std::max(max, 0));
  for (int i = 0; i < n; ++i) stats[i] = agg[i];
  return n;
}

}  // extern "C"
