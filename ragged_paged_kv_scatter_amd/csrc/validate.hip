// Device-side check of the metadata preconditions that rpa_update_kv_cache
// and rpa_forward rely on without checking them (rpa_validate_metadata).
// Three launches on the caller's stream, no host sync:
//   1. clear the status word and the slot bitmap (fill, no memset, so the
//      sequence can be captured in a HIP graph);
//   2. one thread per sequence: query_start_loc order, lengths, and the
//      block-table entries that cover [0, kv_len);
//   3. one thread per new token: its slot (page * page_size + offset) is
//      marked in the bitmap; a bit already set means two writes of one
//      update land on the same slot;
//   4. one workgroup per sequence: every context position [0, kv_len - q_len)
//      whose slot is marked means the update overwrites a key that a
//      sequence reads as context (the prefill kernel's fused update writes
//      new tokens while other units read context, so the two must not meet).
// Every read stays inside the documented array sizes whatever the values, so
// the check itself is safe on bad metadata.
#include "rpa.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

constexpr int kVThreads = 256;

__device__ __forceinline__ int num_seqs_of(const ValidateParams& p) {
  const long long n = (long long)p.dist[0] + p.dist[1] + p.dist[2];
  return (int)(n < 0 ? 0 : (n > p.max_num_seqs ? p.max_num_seqs : n));
}

__global__ __launch_bounds__(kVThreads) void validate_clear(ValidateParams p) {
  const long long i0 = (long long)blockIdx.x * kVThreads + threadIdx.x;
  if (i0 == 0) *p.status = 0;
  for (long long i = i0; i < p.slot_words; i += (long long)gridDim.x * kVThreads)
    p.slot_bits[i] = 0u;
}

__global__ __launch_bounds__(kVThreads) void validate_seqs(ValidateParams p) {
  const int num_seqs = num_seqs_of(p);
  const int s = blockIdx.x * kVThreads + threadIdx.x;
  int bits = 0;
  if (s == 0) {
    const long long sum = (long long)p.dist[0] + p.dist[1] + p.dist[2];
    if (p.dist[0] < 0 || p.dist[1] < 0 || p.dist[2] < 0 || sum > p.max_num_seqs)
      bits |= RPA_META_DISTRIBUTION;
    if (p.qsl[0] != 0) bits |= RPA_META_QSL;
    if (p.qsl[num_seqs] > p.T) bits |= RPA_META_QSL;
  }
  if (s < num_seqs) {
    const int q0 = p.qsl[s], q1 = p.qsl[s + 1];
    const int kv = p.kv_lens[s];
    if (q1 < q0) bits |= RPA_META_QSL;
    const int q_len = q1 - q0;
    const long long cap = (long long)p.pps * p.page_size;
    if (q_len > kv || kv < 0 || kv > cap) bits |= RPA_META_LENS;
    // entries covering [0, min(kv_len, pages_per_seq * page_size))
    const long long kv_c = kv < 0 ? 0 : (kv > cap ? cap : kv);
    const int n_pages = (int)((kv_c + p.page_size - 1) / p.page_size);
    const int32_t* bt = p.block_tables + (long long)s * p.pps;
    for (int i = 0; i < n_pages; ++i) {
      const int pg = bt[i];
      if (pg < 0 || pg >= p.num_pages) {
        bits |= RPA_META_BLOCK_TABLE;
        break;
      }
    }
  }
  if (bits) atomicOr(p.status, bits);
}

// Token t of the step belongs to the sequence s with qsl[s] <= t < qsl[s+1]
// (found by bisection; the search stays bounded even when qsl is out of
// order, which the sequence check reports).  Tokens of a sequence whose
// lengths or block table are invalid are skipped: those are reported too, and
// their slots are not defined.
__global__ __launch_bounds__(kVThreads) void validate_slots(ValidateParams p) {
  const int num_seqs = num_seqs_of(p);
  if (num_seqs == 0) return;
  const int end = min(p.qsl[num_seqs], p.T);
  for (long long t = (long long)blockIdx.x * kVThreads + threadIdx.x; t < end;
       t += (long long)gridDim.x * kVThreads) {
    int lo = 0, hi = num_seqs - 1;              // last s with qsl[s] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const int q0 = p.qsl[s], q1 = p.qsl[s + 1];
    if (t < q0 || t >= q1) continue;
    const int kv = p.kv_lens[s];
    const int q_len = q1 - q0;
    if (q_len > kv || kv > p.pps * p.page_size) continue;
    const int pos = kv - q_len + (int)(t - q0);
    const int pg = p.block_tables[(long long)s * p.pps + pos / p.page_size];
    if (pg < 0 || pg >= p.num_pages) continue;
    const long long slot = (long long)pg * p.page_size + pos % p.page_size;
    const unsigned bit = 1u << (slot & 31);
    const unsigned old = atomicOr(p.slot_bits + (slot >> 5), bit);
    if (old & bit) atomicOr(p.status, (int)RPA_META_SLOTS);
  }
}

__global__ __launch_bounds__(kVThreads) void validate_reads(ValidateParams p) {
  const int num_seqs = num_seqs_of(p);
  for (int s = blockIdx.x; s < num_seqs; s += gridDim.x) {
    const int q0 = p.qsl[s], q1 = p.qsl[s + 1];
    const int kv = p.kv_lens[s];
    const int q_len = q1 - q0;
    if (q1 < q0 || q_len > kv || kv < 0 || kv > p.pps * p.page_size) continue;
    const int ctx = kv - q_len;
    const int32_t* bt = p.block_tables + (long long)s * p.pps;
    bool hit = false;
    for (int pos = threadIdx.x; pos < ctx; pos += kVThreads) {
      const int pg = bt[pos / p.page_size];
      if (pg < 0 || pg >= p.num_pages) continue;
      const long long slot = (long long)pg * p.page_size + pos % p.page_size;
      if (p.slot_bits[slot >> 5] & (1u << (slot & 31))) hit = true;
    }
    if (hit) atomicOr(p.status, (int)RPA_META_WRITE_IN_CONTEXT);
  }
}

}  // namespace

hipError_t launch_validate(const ValidateParams& p, hipStream_t s) {
  const long long clear_wgs = std::min<long long>((p.slot_words + kVThreads - 1) / kVThreads, 4096);
  validate_clear<<<dim3((unsigned)std::max<long long>(clear_wgs, 1)), kVThreads, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  validate_seqs<<<dim3((unsigned)((p.max_num_seqs + kVThreads) / kVThreads)), kVThreads, 0, s>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long tok_wgs = std::min<long long>((p.T + kVThreads - 1) / kVThreads, 4096);
  validate_slots<<<dim3((unsigned)std::max<long long>(tok_wgs, 1)), kVThreads, 0, s>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  validate_reads<<<dim3((unsigned)std::max(std::min(p.max_num_seqs, 4096), 1)), kVThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace rpa
