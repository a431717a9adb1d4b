// Row (decode) kernel: attention of single query rows over their paged KV
// range, one wavefront per (row, KV split, kv head), all G = Hq/Hkv query
// heads of that kv head at once (GQA: the K/V bytes are read once for G heads).
//
// Online softmax as in the tpu-inference v3 kernel diff
// ("flash_attention_step1_qk_softmax": running max m, row sum l;
// "flash_attention_step2_pv": acc = exp(m_prev - m_cur) * acc + p @ v), with
// logits kept in the log2 domain so every exponential is one v_exp_f32.
//
// Lane layout: a token's K (or V) head row of D elements is spread over
// LPT = D / EPL lanes (EPL elements each, one vector load), so a wave reads
// TPR = 64 / LPT tokens per load instruction.  q.k partial sums are reduced
// within the LPT lanes by DPP / ds_swizzle butterflies; the softmax state and
// the accumulator are per lane and reduced across token slots once at the end.
// Pages are located through the block table: lane i keeps the page id of the
// i-th page of the current window and lanes fetch theirs with a bpermute.
#include <math.h>

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int BYTES> struct Vec;
template <> struct Vec<16> { using T = uint4; };
template <> struct Vec<8> { using T = uint2; };
template <> struct Vec<4> { using T = uint32_t; };

// Unpack EPL elements of type CT from raw words into floats.
template <typename CT, int EPL>
__device__ __forceinline__ void unpack(const uint32_t* w, float* f) {
  if constexpr (sizeof(CT) == 4) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) f[e] = __uint_as_float(w[e]);
  } else if constexpr (sizeof(CT) == 2) {
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) { f[2 * e] = bf16lo(w[e]); f[2 * e + 1] = bf16hi(w[e]); }
  } else {
#pragma unroll
    for (int e = 0; e < EPL / 4; ++e) {
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * e + b] = e4m3_to_f32((w[e] >> (8 * b)) & 0xffu);
    }
  }
}

template <typename CT, int EPL>
__device__ __forceinline__ void load_words(const CT* ptr, bool valid, uint32_t* w) {
  constexpr int BYTES = EPL * (int)sizeof(CT);
  constexpr int NW = BYTES / 4;
  using V = typename Vec<BYTES>::T;
  V v;
  if (valid) {
    v = *reinterpret_cast<const V*>(ptr);
  } else {
    uint32_t z[NW] = {};
    v = *reinterpret_cast<V*>(z);
  }
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = vw[i];
}

template <typename QT>
__device__ __forceinline__ float load_q(const QT* q, long long idx);
template <>
__device__ __forceinline__ float load_q<float>(const float* q, long long idx) { return q[idx]; }
template <>
__device__ __forceinline__ float load_q<uint16_t>(const uint16_t* q, long long idx) {
  return bf16_to_f32(q[idx]);
}

template <typename QT>
__device__ __forceinline__ void store_out(QT* o, long long idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* o, long long idx, float v) { o[idx] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* o, long long idx, float v) {
  o[idx] = (uint16_t)f32_to_bf16(v);
}

__device__ __forceinline__ float soft_cap(float s, float cap) {
  return cap * tanhf(s / cap);
}

template <typename QT, typename CT, int D, int G, int EPL, int NR>
__global__ __launch_bounds__(64 * kWavesPerWG) void row_kernel(AttnParams p) {
  constexpr int LPT = D / EPL;   // lanes per token
  constexpr int TPR = 64 / LPT;  // tokens per load instruction
  constexpr int CW = (EPL * (int)sizeof(CT) + 3) / 4;  // 32-bit words per lane per load
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0, "bad lane split");

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const RowDesc* rows = reinterpret_cast<const RowDesc*>(p.ws + p.lay.rows);
  const ItemDesc* items = reinterpret_cast<const ItemDesc*>(p.ws + p.lay.items);
  float* part_ml = reinterpret_cast<float*>(p.ws + p.lay.part_ml);
  float* part_acc = reinterpret_cast<float*>(p.ws + p.lay.part_acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int slot = lane / LPT;       // token slot within a load
  const int dl = lane % LPT;         // d-slice
  const int Hkv = p.Hkv;
  const long long total = (long long)hdr->n_items * Hkv;
  const int ps = p.page_size;
  const long long row_stride = 2LL * Hkv * p.Dpad;  // elements per cache token row
  const CT* cache = static_cast<const CT*>(p.cache);
  const QT* qp = static_cast<const QT*>(p.q);
  const bool use_cap = p.cap > 0.f;
  // logits in log2 units: fold log2(e) into q unless the cap needs natural units
  const float qmul = use_cap ? p.qk_scale : p.qk_scale * kLog2e;

  for (long long idx = (long long)blockIdx.x * kWavesPerWG + wave; idx < total;
       idx += (long long)gridDim.x * kWavesPerWG) {
    const int item_i = (int)(idx / Hkv);
    const int g = (int)(idx - (long long)item_i * Hkv);
    const ItemDesc it = items[item_i];
    const RowDesc rd = rows[it.row];
    const int seq = rd.seq;
    const int* bt = p.block_tables + (long long)seq * p.pps;

    float qv[G][EPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const long long base = ((long long)rd.token * p.Hq + g * G + i) * D + dl * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[i][e] = load_q<QT>(qp, base + e) * qmul;
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
    }

    const int last_page = (it.hi - 1) / ps;
    int pw0 = -(1 << 30);  // first page index held in the page window
    int page_reg = 0;
    const CT* kv_head = cache + 2LL * g * p.Dpad + dl * EPL;

    for (int k0 = it.lo; k0 < it.hi; k0 += NR * TPR) {
      // refresh the page window when this step reaches past it
      const int need_hi = min(k0 + NR * TPR, it.hi) - 1;
      if (need_hi / ps >= pw0 + 64 || k0 / ps < pw0) {
        pw0 = k0 / ps;
        const int pi = pw0 + lane;
        page_reg = (pi <= last_page) ? bt[pi] : 0;
      }
      uint32_t kw[NR][CW], vw[NR][CW];
      bool valid[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int tok = k0 + r * TPR + slot;
        valid[r] = tok < it.hi;
        const int rel = valid[r] ? (tok / ps - pw0) : 0;
        const int page = __shfl(page_reg, rel);
        const long long row = (long long)page * ps + (tok - (tok / ps) * ps);
        const CT* kp = kv_head + row * row_stride;
        load_words<CT, EPL>(kp, valid[r], kw[r]);
        load_words<CT, EPL>(kp + p.Dpad, valid[r], vw[r]);
      }
      // step 1: logits and softmax statistics
      float s[NR][G];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float kf[EPL];
        unpack<CT, EPL>(kw[r], kf);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qv[i][e], kf[e], d);
          d = group_sum<LPT>(d);
          if (use_cap) d = soft_cap(d, p.cap) * kLog2e;
          s[r][i] = valid[r] ? d : -INFINITY;
        }
      }
      float alpha[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float bm = s[0][i];
#pragma unroll
        for (int r = 1; r < NR; ++r) bm = fmaxf(bm, s[r][i]);
        bm = cross_max<LPT>(bm);
        const float mn = fmaxf(m[i], bm);
        alpha[i] = __builtin_amdgcn_exp2f(m[i] - mn);
        m[i] = mn;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          s[r][i] = __builtin_amdgcn_exp2f(s[r][i] - mn);
          ls += s[r][i];
        }
        l[i] = l[i] * alpha[i] + ls;
      }
      // step 2: acc = alpha * acc + p v
#pragma unroll
      for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] *= alpha[i];
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float vf[EPL];
        unpack<CT, EPL>(vw[r], vf);
#pragma unroll
        for (int i = 0; i < G; ++i) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[i][e] = fmaf(s[r][i], vf[e], acc[i][e]);
        }
      }
    }

    // reduce across token slots (l and acc are per-slot partial sums)
#pragma unroll
    for (int i = 0; i < G; ++i) {
      l[i] = cross_sum<LPT>(l[i]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = cross_sum<LPT>(acc[i][e]);
    }
    if (slot == 0) {
      const float vs = p.v_scale;
      if (it.part < 0) {
        QT* op = static_cast<QT*>(p.out);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int h = g * G + i;
          float mm = m[i], ll = l[i], f = 1.f;
          if (p.sink) {
            const float sg = p.sink[h] * kLog2e;
            const float mx = fmaxf(mm, sg);
            f = __builtin_amdgcn_exp2f(mm - mx);
            ll = ll * f + __builtin_amdgcn_exp2f(sg - mx);
          }
          const float scale = f * vs / ll;
          const long long base = ((long long)rd.token * p.Hq + h) * D + dl * EPL;
#pragma unroll
          for (int e = 0; e < EPL; ++e) store_out<QT>(op, base + e, acc[i][e] * scale);
        }
      } else if (it.part < p.lay.max_parts) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int h = g * G + i;
          const long long pb = (long long)it.part * p.Hq + h;
          if (dl == 0) {
            part_ml[2 * pb] = m[i];
            part_ml[2 * pb + 1] = l[i];
          }
#pragma unroll
          for (int e = 0; e < EPL; ++e) part_acc[pb * D + dl * EPL + e] = acc[i][e];
        }
      }
    }
  }
}

// Merge of split partials by log-sum-exp, one wave per (row, q head):
// M = max_j m_j (and the sink), L = sum_j 2^(m_j - M) l_j (+ 2^(sink - M)),
// out = v_scale * sum_j 2^(m_j - M) acc_j / L.
template <typename QT, int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const RowDesc* rows = reinterpret_cast<const RowDesc*>(p.ws + p.lay.rows);
  const int32_t* merge_rows = reinterpret_cast<const int32_t*>(p.ws + p.lay.merge_rows);
  const float* part_ml = reinterpret_cast<const float*>(p.ws + p.lay.part_ml);
  const float* part_acc = reinterpret_cast<const float*>(p.ws + p.lay.part_acc);
  constexpr int PER = (D + 63) / 64;
  const int lane = lane_id();
  const long long total = (long long)hdr->n_merge_rows * p.Hq;
  for (long long idx = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); idx < total;
       idx += (long long)gridDim.x * 4) {
    const int mi = (int)(idx / p.Hq);
    const int h = (int)(idx - (long long)mi * p.Hq);
    const RowDesc rd = rows[merge_rows[mi]];
    const int n = rd.n_split;
    float M = -INFINITY;
    for (int j = 0; j < n; ++j) M = fmaxf(M, part_ml[2 * ((long long)(rd.part_base + j) * p.Hq + h)]);
    float sg = 0.f;
    if (p.sink) { sg = p.sink[h] * kLog2e; M = fmaxf(M, sg); }
    float L = p.sink ? __builtin_amdgcn_exp2f(sg - M) : 0.f;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int j = 0; j < n; ++j) {
      const long long pb = (long long)(rd.part_base + j) * p.Hq + h;
      const float w = __builtin_amdgcn_exp2f(part_ml[2 * pb] - M);
      L += w * part_ml[2 * pb + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int d = lane + 64 * e;
        if (d < D) o[e] = fmaf(w, part_acc[pb * D + d], o[e]);
      }
    }
    const float sc = p.v_scale / L;
    QT* op = static_cast<QT*>(p.out);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = lane + 64 * e;
      if (d < D) store_out<QT>(op, ((long long)rd.token * p.Hq + h) * D + d, o[e] * sc);
    }
  }
}

constexpr int kRowGrid = 2048;  // persistent grid of the row kernel (x4 waves)

template <typename QT, typename CT, int D, int G>
hipError_t launch_rows_t(const AttnParams& p, hipStream_t s) {
  // elements per lane: one 16-byte load, at most 64 accumulators per lane
  constexpr int E16 = 16 / (int)sizeof(CT);
  constexpr int EPL = (E16 * G > 64) ? (64 / G) : E16;
  constexpr int NR = 4;
  const long long waves = (long long)p.lay.max_items * p.Hkv;
  const long long wgs = (waves + kWavesPerWG - 1) / kWavesPerWG;
  dim3 grid((unsigned)(wgs < kRowGrid ? (wgs > 0 ? wgs : 1) : kRowGrid));
  row_kernel<QT, CT, D, G, EPL, NR><<<grid, 64 * kWavesPerWG, 0, s>>>(p);
  return hipGetLastError();
}

template <typename QT, typename CT, int D>
hipError_t launch_rows_g(const AttnParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_rows_t<QT, CT, D, 1>(p, s);
    case 2: return launch_rows_t<QT, CT, D, 2>(p, s);
    case 4: return launch_rows_t<QT, CT, D, 4>(p, s);
    case 8: return launch_rows_t<QT, CT, D, 8>(p, s);
    case 16: return launch_rows_t<QT, CT, D, 16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename QT, typename CT>
hipError_t launch_rows_d(const AttnParams& p, hipStream_t s) {
  if (p.D == 64) return launch_rows_g<QT, CT, 64>(p, s);
  if (p.D == 128) return launch_rows_g<QT, CT, 128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rows(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt, hipStream_t s) {
  if (q_dt == RPA_F32 && cache_dt == RPA_F32) return launch_rows_d<float, float>(p, s);
  if (q_dt == RPA_BF16 && cache_dt == RPA_BF16) return launch_rows_d<uint16_t, uint16_t>(p, s);
  if (q_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) return launch_rows_d<uint16_t, uint8_t>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnParams& p, rpa_dtype q_dt, hipStream_t s) {
  const long long waves = (long long)p.lay.max_merge_rows * p.Hq;
  if (waves <= 0) return hipSuccess;
  long long wgs = (waves + 3) / 4;
  dim3 grid((unsigned)(wgs < 4096 ? wgs : 4096));
  if (q_dt == RPA_F32) {
    if (p.D == 64) merge_kernel<float, 64><<<grid, 256, 0, s>>>(p);
    else merge_kernel<float, 128><<<grid, 256, 0, s>>>(p);
  } else {
    if (p.D == 64) merge_kernel<uint16_t, 64><<<grid, 256, 0, s>>>(p);
    else merge_kernel<uint16_t, 128><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace rpa
