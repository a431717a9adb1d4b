// Merge of the split-KV partials written by the row kernel, by log-sum-exp:
// for a row and q head, out = v_scale * sum_j 2^(m_j - M) acc_j / L with
// M = max_j m_j (and the sink) and L = sum_j 2^(m_j - M) l_j (+ 2^(sink - M)),
// m in log2 units.  One wave merges one (row, kv head) with its G q heads: the
// lanes of a head split its d range.  The running form (M, L, acc rescaled as
// M grows) takes one pass over the partials, and the split loop is unrolled
// so that the loads of several partials are in flight at once.  A row cut
// into many parts (a long context over few rows) is merged by a whole
// workgroup instead: each of its 4 waves runs the same pass over every fourth
// part, and the four states are combined by the same rule.  Used by the
// stand-alone merge kernel and by the prefill kernel, which merges before its
// own work.
#pragma once

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {

template <typename QT>
__device__ __forceinline__ void store_out(QT* o, long long idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* o, long long idx, float v) { o[idx] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* o, long long idx, float v) {
  o[idx] = (uint16_t)f32_to_bf16(v);
}

template <int E>
__device__ __forceinline__ void load_floats(const float* src, float* dst) {
  if constexpr (E % 4 == 0) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + e);
      dst[e] = v.x;
      dst[e + 1] = v.y;
      dst[e + 2] = v.z;
      dst[e + 3] = v.w;
    }
  } else if constexpr (E == 2) {
    const float2 v = *reinterpret_cast<const float2*>(src);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = src[e];
  }
}

// Rows with at least this many parts are merged by a workgroup of 4 waves.
constexpr int kMergeWgParts = 16;
constexpr float kMergeLog2e = 1.4426950408889634f;

// Where a lane works in merge item idx = merge-row index * Hkv + kv head:
// its q head h and d slice sub, and the item's merge descriptor.
template <int D, int G>
struct MergeLane {
  static constexpr int LPH = 64 / G;    // lanes per head
  static constexpr int E = D / LPH;     // d elements per lane
  static_assert(LPH * G == 64 && E * LPH == D, "merge lane split");
  int h, sub;
  MergeDesc md;
  __device__ __forceinline__ MergeLane(const AttnParams& p, long long idx) {
    const MergeDesc* merge_rows = reinterpret_cast<const MergeDesc*>(p.ws + p.lay.merge_rows);
    const int lane = lane_id();
    const int mi = (int)(idx / p.Hkv);
    const int g = (int)(idx - (long long)mi * p.Hkv);
    h = g * G + lane / LPH;
    sub = lane % LPH;
    md = merge_rows[mi];
  }
};

// The running merge over parts j0, j0 + step, ... of the lane's item.
template <int D, int G>
__device__ __forceinline__ void merge_scan(const AttnParams& p, const MergeLane<D, G>& ml_,
                                           int j0, int step, float& M, float& L,
                                           float (&o)[MergeLane<D, G>::E]) {
  constexpr int E = MergeLane<D, G>::E;
  const float* part_ml = reinterpret_cast<const float*>(p.ws + p.lay.part_ml);
  const float* part_acc = reinterpret_cast<const float*>(p.ws + p.lay.part_acc);
  const int Hq = p.Hq, h = ml_.h, sub = ml_.sub;
  const MergeDesc& md = ml_.md;
#pragma unroll 4
  for (int j = j0; j < md.n_split; j += step) {
    const long long pb = (long long)(md.part_base + j) * Hq + h;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * pb);
    float a[E];
    load_floats<E>(part_acc + pb * D + sub * E, a);
    const float m_new = fmaxf(M, ml.x);
    const bool none = m_new == -INFINITY;           // nothing seen yet
    const float r = none ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
    const float w = none ? 0.f : __builtin_amdgcn_exp2f(ml.x - m_new);
    M = m_new;
    L = fmaf(w, ml.y, L * r);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(w, a[e], o[e] * r);
  }
}

template <typename QT, int D, int G>
__device__ __forceinline__ void merge_store(const AttnParams& p, const MergeLane<D, G>& ml_,
                                            float L, const float (&o)[MergeLane<D, G>::E]) {
  constexpr int E = MergeLane<D, G>::E;
  const float sc = p.v_scale / L;
  QT* op = static_cast<QT*>(p.out);
  const long long base = ((long long)ml_.md.token * p.Hq + ml_.h) * D + ml_.sub * E;
#pragma unroll
  for (int e = 0; e < E; ++e) store_out<QT>(op, base + e, o[e] * sc);
}

// Merge item idx by the calling wave.
template <typename QT, int D, int G>
__device__ __forceinline__ void merge_one(const AttnParams& p, long long idx) {
  constexpr int E = MergeLane<D, G>::E;
  const MergeLane<D, G> ml_(p, idx);
  // running state; the sink enters as a partial with l = 1 and acc = 0
  float M = -INFINITY, L = 0.f;
  if (p.sink) {
    M = p.sink[ml_.h] * kMergeLog2e;
    L = 1.f;
  }
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  merge_scan<D, G>(p, ml_, 0, 1, M, L, o);
  merge_store<QT, D, G>(p, ml_, L, o);
}

// LDS floats merge_one_wg needs: the states of waves 1-3.
template <int D, int G>
constexpr int merge_wg_floats() { return 3 * 64 * (MergeLane<D, G>::E + 2); }

// Merge item idx by all 4 waves of the workgroup (every thread calls it with
// the same idx); s holds merge_wg_floats<D, G>() floats of LDS and is free
// again on return.
template <typename QT, int D, int G>
__device__ __forceinline__ void merge_one_wg(const AttnParams& p, long long idx, float* s) {
  constexpr int E = MergeLane<D, G>::E;
  constexpr int S = 64 * (E + 2);                 // floats of one wave's state
  const MergeLane<D, G> ml_(p, idx);
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  float M = -INFINITY, L = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  merge_scan<D, G>(p, ml_, wave, 4, M, L, o);
  if (wave > 0) {
    float* b = s + (wave - 1) * S;
    b[lane] = M;
    b[64 + lane] = L;
#pragma unroll
    for (int e = 0; e < E; ++e) b[(2 + e) * 64 + lane] = o[e];
  }
  __syncthreads();
  if (wave == 0) {
    float Mx = M;
#pragma unroll
    for (int w = 0; w < 3; ++w) Mx = fmaxf(Mx, s[w * S + lane]);
    const float sink = p.sink ? p.sink[ml_.h] * kMergeLog2e : -INFINITY;
    Mx = fmaxf(Mx, sink);
    const float r0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mx);
    L *= r0;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= r0;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const float Mw = s[w * S + lane];
      const float rw = Mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mw - Mx);
      L = fmaf(rw, s[w * S + 64 + lane], L);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(rw, s[w * S + (2 + e) * 64 + lane], o[e]);
    }
    if (p.sink) L += __builtin_amdgcn_exp2f(sink - Mx);
    merge_store<QT, D, G>(p, ml_, L, o);
  }
  __syncthreads();
}

// Parts of merge item idx (uniform over the caller).
__device__ __forceinline__ int merge_parts(const AttnParams& p, long long idx) {
  const MergeDesc* merge_rows = reinterpret_cast<const MergeDesc*>(p.ws + p.lay.merge_rows);
  return merge_rows[idx / p.Hkv].n_split;
}

// Every merge item of the step: items with few parts one per wave (4 per
// workgroup, strided over the grid), then items with many parts one per
// workgroup.  s: merge_wg_floats<D, G>() floats of LDS.
template <typename QT, int D, int G>
__device__ __forceinline__ void merge_all(const AttnParams& p, long long total, float* s) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (long long idx = (long long)blockIdx.x * 4 + wave; idx < total;
       idx += (long long)gridDim.x * 4)
    if (merge_parts(p, idx) < kMergeWgParts) merge_one<QT, D, G>(p, idx);
  // the workgroup's items blockIdx.x + k * gridDim.x, 64 at a time: lane k
  // checks item k (one round of loads, not a chain), and every wave forms the
  // same mask, so the workgroup walks the many-part items together
  const long long stride = gridDim.x;
  for (long long base = blockIdx.x; base < total; base += 64 * stride) {
    const long long mine = base + (long long)lane_id() * stride;
    const bool many = mine < total && merge_parts(p, mine) >= kMergeWgParts;
    for (unsigned long long m = __ballot(many); m != 0; m &= m - 1)
      merge_one_wg<QT, D, G>(p, base + (long long)__builtin_ctzll(m) * stride, s);
  }
}

// The same with the group size G = Hq / Hkv read at run time.
template <typename QT, int D>
__device__ __forceinline__ void merge_all_g(const AttnParams& p, long long total, float* s) {
  switch (p.Hq / p.Hkv) {
    case 1: merge_all<QT, D, 1>(p, total, s); break;
    case 2: merge_all<QT, D, 2>(p, total, s); break;
    case 4: merge_all<QT, D, 4>(p, total, s); break;
    case 8: merge_all<QT, D, 8>(p, total, s); break;
    case 16: merge_all<QT, D, 16>(p, total, s); break;
    default: break;
  }
}

}  // namespace rpa
