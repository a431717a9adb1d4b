// Slot-mapping form of the cache update, into split K / V caches
// [num_blocks, block_size, Hkv, Dpad] (vLLM differential_flash_attn.py: the
// metadata builder's "Compute slot mapping" step with PAD_SLOT_ID padding, and
// populate_kv_cache's reshape_and_cache_flash on kv_cache[0] / kv_cache[1]).
// A slot is block * block_size + offset of the token's position, the same
// (page, offset) the combined-layout update writes; a store skips negative
// slots (padding) and, as a guard, slots past the pool.
#include <algorithm>

#include "scatter.h"

namespace rpa {
namespace {

constexpr int kSlotThreads = 256;

// One thread per token row.
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(SlotMapParams p) {
  const int tok = blockIdx.x * kSlotThreads + threadIdx.x;
  if (tok >= p.T) return;
  const int num_seqs = min(max(p.dist[0] + p.dist[1] + p.dist[2], 0), p.max_num_seqs);
  const int n_valid = num_seqs > 0 ? p.qsl[num_seqs] : 0;
  long long slot = -1;
  if (tok < n_valid) {
    const int s = find_seq(p.qsl, num_seqs, tok);
    const int q0 = p.qsl[s];
    const int q_len = p.qsl[s + 1] - q0;
    const int pos = p.kv_lens[s] - q_len + (tok - q0);
    const int page = p.block_tables[(long long)s * p.pps + pos / p.page_size];
    slot = (long long)page * p.page_size + pos % p.page_size;
  }
  p.slots[tok] = slot;
}

// Tokens [b * tpw, (b + 1) * tpw): each writes its K row (Hkv x Dpad) to the
// key cache and its V row to the value cache at its slot, 16 bytes a thread.
template <typename IN, typename C>
__global__ __launch_bounds__(kSlotThreads) void reshape_cache_kernel(ReshapeParams p, int tpw) {
  __shared__ long long s_slot[kScatterRowsMax];
  const int tok0 = blockIdx.x * tpw;
  if (threadIdx.x < tpw) {
    const int tok = tok0 + threadIdx.x;
    long long sl = tok < p.T ? p.slots[tok] : -1;
    if (sl >= p.num_slots) sl = -1;
    s_slot[threadIdx.x] = sl;
  }
  __syncthreads();
  constexpr int EPC = 16 / Elem<C>::size;          // cache elements per 16-byte chunk
  const int chunks_per_head = p.Dpad / EPC;        // Dpad * elem % 16 == 0 (host-checked)
  const int chunks_per_plane = p.Hkv * chunks_per_head;
  const int chunks_per_tok = 2 * chunks_per_plane;
  const int total = tpw * chunks_per_tok;
  for (int i = threadIdx.x; i < total; i += kSlotThreads) {
    const int lt = i / chunks_per_tok;
    const long long sl = s_slot[lt];
    if (sl < 0) continue;
    const int c = i - lt * chunks_per_tok;
    const int plane = c / chunks_per_plane;        // 0: K, 1: V
    const int w = c - plane * chunks_per_plane;
    const int h = w / chunks_per_head;
    const int d0 = (w - h * chunks_per_head) * EPC;
    const long long tok = tok0 + lt;
    uint4 outv = make_uint4(0, 0, 0, 0);
    if (d0 < p.D) {                                // D * elem % 16 == 0: chunk all in or all pad
      const IN* src = static_cast<const IN*>(plane ? p.values : p.keys) + (tok * p.Hkv + h) * p.D + d0;
      outv = encode_chunk<IN, C>(src, plane ? p.v_scale : p.k_scale);
    }
    C* dst = static_cast<C*>(plane ? p.value_cache : p.key_cache) + (sl * p.Hkv + h) * p.Dpad + d0;
    *reinterpret_cast<uint4*>(dst) = outv;
  }
}

constexpr int kTargetWGs = 1024;

// One workgroup per (pair, layer, plane): 16-byte chunks of the block.
__global__ __launch_bounds__(kSlotThreads) void copy_blocks_kernel(CopyBlocksParams p) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y >> 1, plane = blockIdx.y & 1;
  const long long src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
  if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) return;
  char* base = static_cast<char*>(plane ? p.v[layer] : p.k[layer]);
  const uint4* from = reinterpret_cast<const uint4*>(base + src * p.block_bytes);
  uint4* to = reinterpret_cast<uint4*>(base + dst * p.block_bytes);
  const long long n = p.block_bytes / 16;
  for (long long i = threadIdx.x; i < n; i += kSlotThreads) to[i] = from[i];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s) {
  if (p.num_pairs <= 0 || p.num_layers <= 0) return hipSuccess;
  copy_blocks_kernel<<<dim3(p.num_pairs, 2 * p.num_layers), kSlotThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const SlotMapParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  slot_mapping_kernel<<<(p.T + kSlotThreads - 1) / kSlotThreads, kSlotThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const ReshapeParams& p, rpa_dtype in_dt, rpa_dtype cache_dt,
                                    hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const int tpw = std::min(kScatterRowsMax, std::max(1, (p.T + kTargetWGs - 1) / kTargetWGs));
  const dim3 grid((p.T + tpw - 1) / tpw), block(kSlotThreads);
  if (in_dt == RPA_F32 && cache_dt == RPA_F32) {
    reshape_cache_kernel<float, float><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_BF16) {
    reshape_cache_kernel<uint16_t, uint16_t><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) {
    reshape_cache_kernel<uint16_t, uint8_t><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) {
    reshape_cache_kernel<uint8_t, uint8_t><<<grid, block, 0, s>>>(p, tpw);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rpa
