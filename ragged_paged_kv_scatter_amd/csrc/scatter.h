// Paged KV-cache update: each new K/V token row is written to the slot
// (block_tables[s][pos / page_size], pos % page_size) of its sequence
// (tpu-inference v3 kernel diff, "_update_kv_cache"; ejkernel v3 interface for
// the cache shape).  A token's destination is one contiguous cache row of
// 2 * Hkv * Dpad elements (K_0 V_0 K_1 V_1 ...), so every workgroup writes
// whole rows with 16-byte stores; bf16 -> e4m3 quantisation is fused.
#pragma once

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {
namespace scatter_detail {

constexpr int kScatterRowsMax = 32;  // tokens per workgroup at most

// Element sizes by type tag.
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int size = 4; };
template <> struct Elem<uint16_t> { static constexpr int size = 2; };
template <> struct Elem<uint8_t> { static constexpr int size = 1; };

__device__ __forceinline__ int find_seq(const int32_t* qsl, int num_seqs, int tok) {
  // largest s with qsl[s] <= tok, among s in [0, num_seqs)
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 16 bytes of cache elements from new K or V elements at src: a bit copy, or
// for an e4m3 cache fed with bf16, x / scale in float32 (IEEE RNE) encoded to
// the nearest e4m3fn code (clamped to +-448, ties to even).
template <typename IN, typename C>
__device__ __forceinline__ uint4 encode_chunk(const IN* src, float scale) {
  if constexpr (sizeof(IN) == sizeof(C)) {
    return *reinterpret_cast<const uint4*>(src);
  } else {
    // bf16 -> e4m3: 16 inputs (32 bytes) -> 16 codes
    static_assert(sizeof(IN) == 2 && sizeof(C) == 1, "only bf16 -> e4m3 converts");
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src)[1];
    const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c0 = f32_to_e4m3(__fdiv_rn(bf16lo(wds[2 * k]), scale));
      const uint32_t c1 = f32_to_e4m3(__fdiv_rn(bf16hi(wds[2 * k]), scale));
      const uint32_t c2 = f32_to_e4m3(__fdiv_rn(bf16lo(wds[2 * k + 1]), scale));
      const uint32_t c3 = f32_to_e4m3(__fdiv_rn(bf16hi(wds[2 * k + 1]), scale));
      packed[k] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    return make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

// IN: element type of keys/values; C: element type of the cache.
constexpr int kSeqsInLds = 1024;   // query_start_loc is searched in LDS up to this many seqs

// Tokens [b * tpw, (b + 1) * tpw) by a workgroup of NTH threads (tpw <= kScatterRowsMax).
template <typename IN, typename C, int NTH>
__device__ __forceinline__ void scatter_body(const ScatterParams& p, int tpw, int b) {
  __shared__ long long s_row[kScatterRowsMax];  // destination cache row (element index), -1 = skip
  __shared__ int32_t s_qsl[kSeqsInLds + 1];
  const int tok0 = b * tpw;
  const int num_seqs = min(max(p.dist[0] + p.dist[1] + p.dist[2], 0), p.max_num_seqs);
  const bool qsl_in_lds = num_seqs <= kSeqsInLds;
  if (qsl_in_lds) {
    for (int i = threadIdx.x; i <= num_seqs; i += NTH) s_qsl[i] = p.qsl[i];
    __syncthreads();
  }
  const int n_valid = num_seqs > 0 ? (qsl_in_lds ? s_qsl[num_seqs] : p.qsl[num_seqs]) : 0;
  if (threadIdx.x < tpw) {
    const int tok = tok0 + threadIdx.x;
    long long row = -1;
    if (tok < n_valid && tok < p.T) {
      const int s = qsl_in_lds ? find_seq(s_qsl, num_seqs, tok) : find_seq(p.qsl, num_seqs, tok);
      const int q0 = p.qsl[s];
      const int q_len = p.qsl[s + 1] - q0;
      if (q_len < p.skip_min_q) {      // else the prefill kernel writes this token
        const int pos = p.kv_lens[s] - q_len + (tok - q0);
        const int page = p.block_tables[(long long)s * p.pps + pos / p.page_size];
        row = (long long)page * p.page_size + pos % p.page_size;
      }
    }
    s_row[threadIdx.x] = row;
  }
  __syncthreads();

  constexpr int ESZ = Elem<C>::size;
  constexpr int EPC = 16 / ESZ;                    // cache elements per 16-byte chunk
  const int chunks_per_head = p.Dpad / EPC;        // Dpad * ESZ % 16 == 0 (host-checked)
  const int chunks_per_row = 2 * p.Hkv * chunks_per_head;
  const int total = tpw * chunks_per_row;
  const IN* keys = static_cast<const IN*>(p.keys);
  const IN* values = static_cast<const IN*>(p.values);
  C* cache = static_cast<C*>(p.cache);

  for (int i = threadIdx.x; i < total; i += NTH) {
    const int lt = i / chunks_per_row;
    const long long row = s_row[lt];
    if (row < 0) continue;
    const int c = i - lt * chunks_per_row;
    const int ch = c / chunks_per_head;            // combined head: 2h = K, 2h+1 = V
    const int w = c - ch * chunks_per_head;
    const int h = ch >> 1;
    const int d0 = w * EPC;
    const long long tok = tok0 + lt;
    uint4 outv = make_uint4(0, 0, 0, 0);
    if (d0 < p.D) {                                // D * ESZ % 16 == 0: chunk all in or all pad
      const IN* src = ((ch & 1) ? values : keys) + (tok * p.Hkv + h) * p.D + d0;
      outv = encode_chunk<IN, C>(src, (ch & 1) ? p.inv_v_scale_src : p.inv_k_scale_src);
    }
    C* dst = cache + (row * (2 * p.Hkv) + ch) * p.Dpad + d0;
    *reinterpret_cast<uint4*>(dst) = outv;
  }
}

}  // namespace scatter_detail

using scatter_detail::Elem;
using scatter_detail::encode_chunk;
using scatter_detail::find_seq;
using scatter_detail::kScatterRowsMax;
using scatter_detail::scatter_body;

}  // namespace rpa
