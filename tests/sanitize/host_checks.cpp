// Host-side checks of the C ABI (include/rpa.h) run under ASan / UBSan, linked
// with host_stubs.cpp in place of the kernels: the same cases as
// tests/test_abi.py (status codes of invalid descriptors, options, pointers,
// workspaces; block copies and swaps; the metadata check's host checks; the
// allocation-free call's size limit), plus the dry-run trace formatter at full
// and truncated buffer sizes and every error string.  No pointer passed here
// is ever dereferenced: each call either fails its host checks or reaches the
// stubs.  Prints "host checks: N passed" and exits 0, or names the first
// failing check and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "rpa.h"

namespace {

int g_checks = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    std::fprintf(stderr, "host check failed (line %d): %s: got %d, want %d\n", line, what, got,
                 want);
    std::exit(1);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

rpa_desc good_desc() {
  rpa_desc d = {};
  d.total_tokens = 7;
  d.max_num_seqs = 3;
  d.pages_per_seq = 2;
  d.num_pages = 8;
  d.page_size = 16;
  d.num_q_heads = 4;
  d.num_kv_heads = 2;
  d.head_dim = 64;
  d.head_dim_padded = 64;
  d.q_dtype = RPA_F32;
  d.kv_in_dtype = RPA_F32;
  d.cache_dtype = RPA_F32;
  return d;
}

rpa_desc bf16_desc(int tokens, int seqs) {
  rpa_desc d = good_desc();
  d.q_dtype = d.kv_in_dtype = d.cache_dtype = RPA_BF16;
  d.num_q_heads = 32;
  d.num_kv_heads = 8;
  d.head_dim = d.head_dim_padded = 128;
  d.pages_per_seq = 128;
  d.num_pages = 20000;
  d.page_size = 64;
  d.total_tokens = tokens;
  d.max_num_seqs = seqs;
  return d;
}

rpa_options good_opts() {
  rpa_options o = {};
  o.softmax_scale = 0.125f;
  return o;
}

int ws_status(const rpa_desc& d, const rpa_options& o, size_t* n) {
  return rpa_workspace_bytes(&d, &o, n);
}

void* fake(uintptr_t a = 4096) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
  const rpa_options o = good_opts();
  size_t n = 0;
  EXPECT(ws_status(good_desc(), o, &n), RPA_OK);
  // descriptors
  {
    struct Case {
      void (*edit)(rpa_desc&);
      int code;
    };
    const Case cases[] = {
        {[](rpa_desc& d) { d.num_q_heads = 3; }, RPA_ERR_INVALID_SHAPE},
        {[](rpa_desc& d) { d.head_dim_padded = 32; }, RPA_ERR_INVALID_SHAPE},
        {[](rpa_desc& d) { d.num_kv_heads = 0; }, RPA_ERR_INVALID_SHAPE},
        {[](rpa_desc& d) { d.page_size = 0; }, RPA_ERR_INVALID_SHAPE},
        {[](rpa_desc& d) { d.head_dim = d.head_dim_padded = 96; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.page_size = 24; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.num_q_heads = 6; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.q_dtype = RPA_BF16; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.q_dtype = 7; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.cache_dtype = RPA_FP8_E4M3; }, RPA_ERR_UNSUPPORTED},
        {[](rpa_desc& d) { d.max_num_seqs = 20000; }, RPA_ERR_UNSUPPORTED},
    };
    for (const Case& c : cases) {
      rpa_desc d = good_desc();
      c.edit(d);
      EXPECT(ws_status(d, o, &n), c.code);
    }
    EXPECT(rpa_workspace_bytes(nullptr, &o, &n), RPA_ERR_NULL_POINTER);
    const rpa_desc d = good_desc();
    EXPECT(rpa_workspace_bytes(&d, nullptr, &n), RPA_ERR_NULL_POINTER);
    EXPECT(rpa_workspace_bytes(&d, &o, nullptr), RPA_ERR_NULL_POINTER);
  }
  // options
  {
    void (*edits[])(rpa_options&) = {
        [](rpa_options& x) { x.sliding_window = -1; },
        [](rpa_options& x) { x.logits_soft_cap = -1.f; },
        [](rpa_options& x) { x.logits_soft_cap = 1.f / 0.f; },
        [](rpa_options& x) { x.k_scale = 0.f / 0.f; },
        [](rpa_options& x) { x.softmax_scale = 1.f / 0.f; },
        [](rpa_options& x) { x.v_scale = -0.5f; },
        [](rpa_options& x) { x.num_queries_per_block = -2; },
    };
    for (auto e : edits) {
      rpa_options x = good_opts();
      e(x);
      EXPECT(ws_status(good_desc(), x, &n), RPA_ERR_INVALID_OPTION);
    }
    rpa_options z = good_opts();
    z.softmax_scale = 0.f;
    EXPECT(ws_status(good_desc(), z, &n), RPA_OK);
    z.softmax_scale = -0.3f;
    EXPECT(ws_status(good_desc(), z, &n), RPA_OK);
  }
  // forward: NULL and workspace errors, misaligned buffers
  {
    const rpa_desc d = good_desc();
    void* f = fake();
    const int32_t* m = static_cast<const int32_t*>(f);
    EXPECT(rpa_forward(&d, &o, nullptr, nullptr, nullptr, f, m, m, m, m, nullptr, f, f,
                       size_t(1) << 30, nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_forward(&d, &o, f, f, nullptr, f, m, m, m, m, nullptr, f, f, size_t(1) << 30,
                       nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_forward(&d, &o, f, nullptr, nullptr, f, m, m, m, m, nullptr, f, f, 16, nullptr),
           RPA_ERR_WORKSPACE);
    EXPECT(rpa_forward(&d, &o, f, nullptr, nullptr, fake(4096 + 8), m, m, m, m, nullptr, f, f,
                       size_t(1) << 30, nullptr),
           RPA_ERR_INVALID_SHAPE);
    // decode-only: every check passes and the stubs stand in for the launches
    const rpa_desc dec = bf16_desc(256, 256);
    size_t need = 0;
    EXPECT(ws_status(dec, o, &need), RPA_OK);
    EXPECT(rpa_forward(&dec, &o, f, f, f, f, m, m, m, m, nullptr, f, f, need, nullptr), RPA_OK);
    // update / slot mapping / split store
    EXPECT(rpa_update_kv_cache(&d, f, f, f, nullptr, m, m, m, 1.f, 1.f, nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_update_kv_cache(&d, f, f, f, m, m, m, m, 0.f / 0.f, 1.f, nullptr),
           RPA_ERR_INVALID_OPTION);
    EXPECT(rpa_update_kv_cache(nullptr, f, f, f, m, m, m, m, 1.f, 1.f, nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_update_kv_cache(&d, f, f, f, m, m, m, m, 1.f, 1.f, nullptr), RPA_OK);
    int64_t* sl = static_cast<int64_t*>(f);
    EXPECT(rpa_slot_mapping(&d, m, m, m, m, nullptr, nullptr), RPA_ERR_NULL_POINTER);
    EXPECT(rpa_slot_mapping(&d, nullptr, m, m, m, sl, nullptr), RPA_ERR_NULL_POINTER);
    rpa_desc ps = good_desc();
    ps.page_size = 24;
    EXPECT(rpa_slot_mapping(&ps, m, m, m, m, sl, nullptr), RPA_ERR_UNSUPPORTED);
    EXPECT(rpa_reshape_and_cache(&d, f, f, nullptr, f, sl, 1.f, 1.f, nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_reshape_and_cache(&d, f, f, f, f, sl, -1.f, 1.f, nullptr),
           RPA_ERR_INVALID_OPTION);
    EXPECT(rpa_reshape_and_cache(&d, fake(4096 + 4), f, f, f, sl, 1.f, 1.f, nullptr),
           RPA_ERR_INVALID_SHAPE);
    uint32_t* bits = static_cast<uint32_t*>(f);
    int32_t* status = static_cast<int32_t*>(f);
    EXPECT(rpa_validate_metadata(&d, m, m, m, m, bits, nullptr, nullptr), RPA_ERR_NULL_POINTER);
    EXPECT(rpa_validate_metadata(&d, m, nullptr, m, m, bits, status, nullptr),
           RPA_ERR_NULL_POINTER);
    EXPECT(rpa_validate_metadata(&ps, m, m, m, m, bits, status, nullptr), RPA_ERR_UNSUPPORTED);
  }
  // block copies and swaps
  {
    void* arr[2] = {fake(4096), fake(8192)};
    void* bad[2] = {fake(4096), fake(4096 + 8)};
    const int64_t* pairs_dev = static_cast<const int64_t*>(fake());
    EXPECT(rpa_copy_blocks(nullptr, arr, 2, 4, 64, pairs_dev, 1, nullptr), RPA_ERR_NULL_POINTER);
    EXPECT(rpa_copy_blocks(arr, arr, 65, 4, 64, pairs_dev, 1, nullptr), RPA_ERR_INVALID_SHAPE);
    EXPECT(rpa_copy_blocks(arr, arr, 2, 4, 60, pairs_dev, 1, nullptr), RPA_ERR_INVALID_SHAPE);
    EXPECT(rpa_copy_blocks(bad, arr, 2, 4, 64, pairs_dev, 1, nullptr), RPA_ERR_INVALID_SHAPE);
    EXPECT(rpa_copy_blocks(arr, arr, 2, 4, 64, pairs_dev, 0, nullptr), RPA_OK);
    const int64_t pairs[4] = {0, 1, 3, 5};
    EXPECT(rpa_swap_blocks(fake(), fake(), 4, 4, 64, pairs, 2, nullptr), RPA_ERR_INVALID_SHAPE);
    EXPECT(rpa_swap_blocks(nullptr, fake(), 4, 4, 64, pairs, 1, nullptr), RPA_ERR_NULL_POINTER);
  }
  // the allocation-free call: host checks and its size limit
  {
    void* f = fake();
    const int32_t* m = static_cast<const int32_t*>(f);
    EXPECT(rpa_forward_noalloc(nullptr, &o, f, f, f, f, m, m, m, m, nullptr, f, nullptr),
           RPA_ERR_NULL_POINTER);
    rpa_desc big = bf16_desc(4096, 4096);
    big.num_q_heads = 128;
    size_t need = 0;
    EXPECT(ws_status(big, o, &need), RPA_OK);
    EXPECT(need > RPA_NOALLOC_SCRATCH_BYTES ? 1 : 0, 1);
    EXPECT(rpa_forward_noalloc(&big, &o, f, f, f, f, m, m, m, m, nullptr, f, nullptr),
           RPA_ERR_WORKSPACE);
  }
  // dry-run trace: whole and truncated buffers, every kind of launch sequence
  {
    const rpa_desc descs[] = {good_desc(), bf16_desc(256, 256), bf16_desc(2176, 132)};
    for (const rpa_desc& d : descs) {
      for (int upd = 0; upd < 2; ++upd) {
        size_t len = 0;
        EXPECT(rpa_trace_format(&d, &o, upd, nullptr, 0, &len), RPA_OK);
        EXPECT(len > 0 ? 1 : 0, 1);
        std::vector<char> buf(len + 1);
        size_t len2 = 0;
        EXPECT(rpa_trace_format(&d, &o, upd, buf.data(), buf.size(), &len2), RPA_OK);
        EXPECT((int)(len2 == len && std::strlen(buf.data()) == len), 1);
        EXPECT((int)(std::strncmp(buf.data(), "[rpa] forward ", 14) == 0), 1);
        char small[17];
        EXPECT(rpa_trace_format(&d, &o, upd, small, sizeof small, nullptr), RPA_OK);
        EXPECT((int)std::strlen(small), 16);
      }
    }
    rpa_desc bad = good_desc();
    bad.page_size = 24;
    char buf[64];
    EXPECT(rpa_trace_format(&bad, &o, 1, buf, sizeof buf, nullptr), RPA_ERR_UNSUPPORTED);
  }
  // error strings and the profile record
  for (int code = 0; code < 7; ++code) EXPECT(std::strlen(rpa_error_string(code)) > 0 ? 1 : 0, 1);
  EXPECT((int)(std::strstr(rpa_error_string(99), "unknown") != nullptr), 1);
  rpa_kernel_stat stats[4];
  EXPECT(rpa_profile_read(stats, 4), 0);
  std::printf("host checks: %d passed\n", g_checks);
  return 0;
}
