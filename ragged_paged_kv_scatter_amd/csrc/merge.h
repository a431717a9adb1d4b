// Merge of the split-KV partials written by the row kernel, by log-sum-exp:
// for a row and q head, out = v_scale * sum_j 2^(m_j - M) acc_j / L with
// M = max_j m_j (and the sink) and L = sum_j 2^(m_j - M) l_j (+ 2^(sink - M)),
// m in log2 units.  One wave merges one (row, kv head) with its G q heads: the
// lanes of a head split its d range.  The running form (M, L, acc rescaled as
// M grows) takes one pass over the partials, and the split loop is unrolled
// so that the loads of several partials are in flight at once.  Used by the
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

// Merge item idx = merge-row index * Hkv + kv head, by the calling wave.
template <typename QT, int D, int G>
__device__ __forceinline__ void merge_one(const AttnParams& p, long long idx) {
  constexpr int LPH = 64 / G;           // lanes per head
  constexpr int E = D / LPH;            // d elements per lane
  constexpr float kLog2eM = 1.4426950408889634f;
  static_assert(LPH * G == 64 && E * LPH == D, "merge lane split");
  const MergeDesc* merge_rows = reinterpret_cast<const MergeDesc*>(p.ws + p.lay.merge_rows);
  const float* part_ml = reinterpret_cast<const float*>(p.ws + p.lay.part_ml);
  const float* part_acc = reinterpret_cast<const float*>(p.ws + p.lay.part_acc);
  const int lane = lane_id();
  const int hi = lane / LPH, sub = lane % LPH;
  const int Hq = p.Hq, Hkv = p.Hkv;
  const int mi = (int)(idx / Hkv);
  const int g = (int)(idx - (long long)mi * Hkv);
  const int h = g * G + hi;
  const MergeDesc md = merge_rows[mi];
  // running state; the sink enters as a partial with l = 1 and acc = 0
  float M = -INFINITY, L = 0.f;
  if (p.sink) {
    M = p.sink[h] * kLog2eM;
    L = 1.f;
  }
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
#pragma unroll 4
  for (int j = 0; j < md.n_split; ++j) {
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
  const float sc = p.v_scale / L;
  QT* op = static_cast<QT*>(p.out);
  const long long base = ((long long)md.token * Hq + h) * D + sub * E;
#pragma unroll
  for (int e = 0; e < E; ++e) store_out<QT>(op, base + e, o[e] * sc);
}

// The same with the group size G = Hq / Hkv read at run time.
template <typename QT, int D>
__device__ __forceinline__ void merge_one_g(const AttnParams& p, long long idx) {
  switch (p.Hq / p.Hkv) {
    case 1: merge_one<QT, D, 1>(p, idx); break;
    case 2: merge_one<QT, D, 2>(p, idx); break;
    case 4: merge_one<QT, D, 4>(p, idx); break;
    case 8: merge_one<QT, D, 8>(p, idx); break;
    case 16: merge_one<QT, D, 16>(p, idx); break;
    default: break;
  }
}

}  // namespace rpa
