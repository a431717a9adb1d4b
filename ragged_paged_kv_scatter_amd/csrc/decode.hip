// Row (decode) kernel: attention of single query rows over their paged KV
// range, one wavefront per (row, KV split, kv head), all G = Hq/Hkv query
// heads of that kv head at once (GQA: the K/V bytes are read once for G heads).
//
// Online softmax as in the tpu-inference v3 kernel diff
// ("flash_attention_step1_qk_softmax": running max m, row sum l;
// "flash_attention_step2_pv": acc = exp(m_prev - m_cur) * acc + p @ v), with
// logits kept in log2 units so every exponential is one v_exp_f32.
//
// Lane layout: a token's K (or V) head row of D elements is spread over
// LPT = D / EPL lanes (EPL elements each, one vector load), so a wave reads
// TPR = 64 / LPT tokens per load instruction ("load row"), NR load rows per
// step, with the next step's loads in flight while the current one computes.
//
// q.k: bf16 pairs through v_dot2_f32_bf16 (e4m3 codes are widened to bf16
// pairs first, exactly); the G partial sums of a token are then reduced over
// its LPT lanes by a DPP reduce-scatter, after which lane L holds the full
// logit of ONE head, h = (L mod LPT) >> (log2 LPT - log2 G): the soft cap and
// the exponential run once per (token, head) instead of G times per lane.
// p is broadcast back to the token's lanes (DPP row_newbcast / ds_swizzle)
// for p.v, which pairs two tokens per v_dot2_f32_bf16.  fp32 caches use plain
// FMAs.  Pages are located through the block table: lane i keeps the page id
// of the i-th page of a 64-page window and lanes fetch theirs with a bpermute.
#include <math.h>

#include <utility>

#include "device_common.h"
#include "merge.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int PATTERN>
__device__ __forceinline__ float swz(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PATTERN));
}

// Partner value for a reduction step over lane bit K: any partner whose lane
// id differs in bit K (and possibly lower bits) keeps a reduction complete, so
// the cheap DPP mirrors serve bits 2 and 3 (lane ^ 7, lane ^ 15).
template <int K>
__device__ __forceinline__ float red_x(float v) {
  if constexpr (K == 0) return dppf<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (K == 1) return dppf<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (K == 2) return dppf<0x141>(v);  // row_half_mirror
  else if constexpr (K == 3) return dppf<0x140>(v);  // row_mirror
  else if constexpr (K == 4) return swz<0x401F>(v);  // lane ^ 16
  else return __shfl_xor(v, 32);
}
// Exact partner lane ^ (1 << K) (values differ across the lower bits).
template <int K>
__device__ __forceinline__ float xor_x(float v) {
  if constexpr (K == 0) return dppf<0xB1>(v);
  else if constexpr (K == 1) return dppf<0x4E>(v);
  else if constexpr (K == 2) return swz<0x101F>(v);  // lane ^ 4
  else if constexpr (K == 3) return dppf<0x128>(v);  // row_ror:8 == lane ^ 8 in a row
  else if constexpr (K == 4) return swz<0x401F>(v);
  else return __shfl_xor(v, 32);
}

// Value of lane REP of this lane's aligned group of LPT lanes.
template <int LPT, int REP>
__device__ __forceinline__ float bcast(float v) {
  if constexpr (LPT == 1) {
    return v;
  } else if constexpr (LPT == 16) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + REP, 0xF, 0xF, false));
  } else if constexpr (LPT < 16) {
    return swz<((0x1F & ~(LPT - 1)) | (REP << 5))>(v);
  } else if constexpr (LPT == 32) {
    return swz<(REP << 5)>(v);
  } else {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), REP));
  }
}

// Reduce G partial sums over the LPT = 2^B lanes of a token group; the first
// log2(G) steps scatter (each keeps half of its values), the rest add.  On
// return v[0] holds, in lane L, the full sum of head (L mod LPT) >> (B - log2 G).
template <int B, int NV>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (B > 0) {
    constexpr int K = B - 1;
    if constexpr (NV > 1) {
      const bool hi = (lane >> K) & 1;
#pragma unroll
      for (int j = 0; j < NV / 2; ++j) {
        const float send = hi ? v[j] : v[j + NV / 2];
        const float keep = hi ? v[j + NV / 2] : v[j];
        v[j] = keep + red_x<K>(send);
      }
      reduce_scatter<B - 1, NV / 2>(v, lane);
    } else {
      v[0] += red_x<K>(v[0]);
      reduce_scatter<B - 1, 1>(v, lane);
    }
  }
}

// max / sum over the token slots (lane bits B..5), exact partners
template <int B>
__device__ __forceinline__ float slots_max(float v) {
  if constexpr (B <= 5) {
    v = fmaxf(v, xor_x<B>(v));
    return slots_max<B + 1>(v);
  }
  return v;
}
template <int B>
__device__ __forceinline__ float slots_sum(float v) {
  if constexpr (B <= 5) {
    v += xor_x<B>(v);
    return slots_sum<B + 1>(v);
  }
  return v;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return a | (b << 16);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Head-row chunk of EPL cache elements -> words: fp32 words, or bf16 pairs.
template <typename CT, int EPL>
struct Chunk {
  static constexpr int BYTES = EPL * (int)sizeof(CT);
  static constexpr int NW = BYTES / 4;                           // raw words loaded
  static constexpr int NP = (sizeof(CT) == 4) ? EPL : EPL / 2;   // words after widening
};

// The cache is streamed once per call: loads are non-temporal (nt), which
// keeps them from displacing reusable lines in L2.
template <typename CT, int EPL>
__device__ __forceinline__ void load_chunk(const CT* ptr, bool valid, uint32_t* w) {
  constexpr int NW = Chunk<CT, EPL>::NW;
  typedef uint32_t words __attribute__((ext_vector_type(NW)));
  if (valid) {
    const words v = __builtin_nontemporal_load(reinterpret_cast<const words*>(ptr));
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = 0u;
  }
}

// e4m3 codes -> bf16 pairs of consecutive elements (exact widening)
template <int NW>
__device__ __forceinline__ void widen_fp8(const uint32_t* w, uint32_t* out) {
  typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    out[2 * i] = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
    out[2 * i + 1] =
        __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
  }
}

template <typename QT, typename CT, int D, int G, int EPL, int NR>
__global__ __launch_bounds__(64 * kWavesPerWG) void row_kernel(AttnParams p) {
  constexpr bool F32 = sizeof(CT) == 4;
  constexpr int LPT = D / EPL;          // lanes per token
  constexpr int TPR = 64 / LPT;         // tokens per load row
  constexpr int STEP = NR * TPR;        // tokens per step
  constexpr int B = ilog2(LPT);
  constexpr int LG = ilog2(G);
  constexpr int NW = Chunk<CT, EPL>::NW;
  constexpr int NP = Chunk<CT, EPL>::NP;
  static_assert((1 << B) == LPT && (1 << LG) == G && G <= LPT, "lane split");
  static_assert(NR % 2 == 0, "p.v pairs two load rows");

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const RowDesc* rows = reinterpret_cast<const RowDesc*>(p.ws + p.lay.rows);
  const ItemDesc* items = reinterpret_cast<const ItemDesc*>(p.ws + p.lay.items);
  float* part_ml = reinterpret_cast<float*>(p.ws + p.lay.part_ml);
  float* part_acc = reinterpret_cast<float*>(p.ws + p.lay.part_acc);

  const int lane = lane_id();
  const int slot = lane / LPT;          // token slot within a load row
  const int dl = lane % LPT;            // d-slice
  const int my_head = dl >> (B - LG);   // head whose logit this lane holds after the scatter
  const int Hkv = p.Hkv;
  const long long total = (long long)hdr->n_items * Hkv;
  const int sh = p.ps_shift;                        // page_size = 1 << sh
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * (uint32_t)sizeof(CT);  // one cache token row
  const uint32_t head_bytes = p.Dpad * (uint32_t)sizeof(CT);            // K -> V of a head
  const CT* cache = static_cast<const CT*>(p.cache);
  const bool use_cap = p.cap > 0.f;
  const float c_log2 = p.qk_scale * kLog2e;

  // The grid is the number of resident waves; wave w walks items w, w + grid,
  // ...  The planner lists full-size splits first, so every wave ends on the
  // short remainder splits and the launch has no long tail.
  const int wave = threadIdx.x >> 6;
  for (long long idx = (long long)blockIdx.x * kWavesPerWG + wave; idx < total;
       idx += (long long)gridDim.x * kWavesPerWG) {
    const int item_i = (int)(idx / Hkv);
    const int g = (int)(idx - (long long)item_i * Hkv);
    const ItemDesc it = items[item_i];
    const RowDesc rd = rows[it.row];
    const int* bt = p.block_tables + (long long)rd.seq * p.pps;

    // q of the G heads, this lane's d-slice: fp32 values or raw bf16 pairs
    uint32_t qw[G][NP];
    {
      const QT* qp = static_cast<const QT*>(p.q) + ((long long)rd.token * p.Hq + g * G) * D +
                     dl * EPL;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if constexpr (sizeof(QT) == 4) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) qw[i][e] = __float_as_uint(qp[i * D + e]);
        } else {
#pragma unroll
          for (int e = 0; e < NP; ++e)
            qw[i][e] = reinterpret_cast<const uint32_t*>(qp + i * D)[e];
        }
      }
    }

    float acc[G][EPL];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
    float m_own = -INFINITY, l_own = 0.f;  // softmax state of head my_head

    const int last_page = (it.hi - 1) >> sh;
    int pw0 = -(1 << 30);
    int page_reg = 0;
    const char* kv_head =
        reinterpret_cast<const char*>(cache + 2LL * g * p.Dpad + dl * EPL);

    uint32_t kA[NR][NW], vA[NR][NW], kB[NR][NW], vB[NR][NW];

    // Loads of one step.  Tokens past the item are clamped to its last token
    // (valid memory, masked out of the softmax), so every load is unconditional.
    auto load_step = [&](int k0, uint32_t (*kw)[NW], uint32_t (*vw)[NW]) {
      const int need_hi = min(k0 + STEP, it.hi) - 1;
      if ((need_hi >> sh) >= pw0 + 64 || (k0 >> sh) < pw0) {
        pw0 = k0 >> sh;
        const int pi = pw0 + lane;
        page_reg = (pi <= last_page) ? bt[pi] : 0;
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int tok = min(k0 + r * TPR + slot, it.hi - 1);
        const int page = __builtin_amdgcn_ds_bpermute(((tok >> sh) - pw0) << 2, page_reg);
        const uint32_t row = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
        const char* kp = kv_head + (uint64_t)row * row_bytes;
        load_chunk<CT, EPL>(reinterpret_cast<const CT*>(kp), true, kw[r]);
        load_chunk<CT, EPL>(reinterpret_cast<const CT*>(kp + head_bytes), true, vw[r]);
      }
    };

    auto compute_step = [&](int k0, uint32_t (*kw)[NW], uint32_t (*vw)[NW]) {
      // ---- step 1: logits of this lane's head for the NR load rows ----
      float s2[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float part[G];
        if constexpr (F32) {
#pragma unroll
          for (int i = 0; i < G; ++i) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(__uint_as_float(qw[i][e]), __uint_as_float(kw[r][e]), d);
            part[i] = d;
          }
        } else {
          uint32_t kp2[NP];
          if constexpr (sizeof(CT) == 1) widen_fp8<NW>(kw[r], kp2);
          else {
#pragma unroll
            for (int e = 0; e < NP; ++e) kp2[e] = kw[r][e];
          }
#pragma unroll
          for (int i = 0; i < G; ++i) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < NP; ++e) d = dot2(qw[i][e], kp2[e], d);
            part[i] = d;
          }
        }
        reduce_scatter<B, G>(part, lane);
        float s = part[0];
        s = use_cap ? p.cap * tanhf(s * p.qk_scale / p.cap) * kLog2e : s * c_log2;
        const bool valid = k0 + r * TPR + slot < it.hi;
        s2[r] = valid ? s : -INFINITY;
      }
      float bm = s2[0];
#pragma unroll
      for (int r = 1; r < NR; ++r) bm = fmaxf(bm, s2[r]);
      bm = slots_max<B>(bm);
      // lazy rescale: move the running max only when it grows by more than 2^8
      if (__any(bm > m_own + 8.f)) {
        const float m_new = fmaxf(m_own, bm);
        const float alpha = __builtin_amdgcn_exp2f(m_own - m_new);  // 0 on the first step
        m_own = m_new;
        l_own *= alpha;
        float al[G];
        [&]<int... I>(std::integer_sequence<int, I...>) {
          ((al[I] = bcast<LPT, (I << (B - LG))>(alpha)), ...);
        }(std::make_integer_sequence<int, G>{});
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[i][e] *= al[i];
      }
      float pr[NR];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(s2[r] - m_own);
        ls += pr[r];
      }
      l_own += ls;
      // ---- step 2: acc += p v, all G heads of this lane's token ----
#pragma unroll
      for (int r = 0; r < NR; r += 2) {
        float pa[G], pb[G];
        [&]<int... I>(std::integer_sequence<int, I...>) {
          ((pa[I] = bcast<LPT, (I << (B - LG))>(pr[r])), ...);
          ((pb[I] = bcast<LPT, (I << (B - LG))>(pr[r + 1])), ...);
        }(std::make_integer_sequence<int, G>{});
        if constexpr (F32) {
#pragma unroll
          for (int i = 0; i < G; ++i)
#pragma unroll
            for (int e = 0; e < EPL; ++e)
              acc[i][e] = fmaf(pb[i], __uint_as_float(vw[r + 1][e]),
                               fmaf(pa[i], __uint_as_float(vw[r][e]), acc[i][e]));
        } else {
          // pair the two tokens at every element: (v_r[e], v_r+1[e]) as bf16x2
          uint32_t vp[EPL];
          if constexpr (sizeof(CT) == 2) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
              vp[2 * w] = __builtin_amdgcn_perm(vw[r + 1][w], vw[r][w], 0x05040100u);
              vp[2 * w + 1] = __builtin_amdgcn_perm(vw[r + 1][w], vw[r][w], 0x07060302u);
            }
          } else {
            typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int w = 0; w < NW; ++w) {
              const f2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[r][w], false);
              const f2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[r][w], true);
              const f2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[r + 1][w], false);
              const f2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[r + 1][w], true);
              vp[4 * w + 0] = __builtin_amdgcn_perm(__float_as_uint(b0[0]), __float_as_uint(a0[0]), 0x07060302u);
              vp[4 * w + 1] = __builtin_amdgcn_perm(__float_as_uint(b0[1]), __float_as_uint(a0[1]), 0x07060302u);
              vp[4 * w + 2] = __builtin_amdgcn_perm(__float_as_uint(b1[0]), __float_as_uint(a1[0]), 0x07060302u);
              vp[4 * w + 3] = __builtin_amdgcn_perm(__float_as_uint(b1[1]), __float_as_uint(a1[1]), 0x07060302u);
            }
          }
#pragma unroll
          for (int i = 0; i < G; ++i) {
            const uint32_t pp = pack_bf16(pa[i], pb[i]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[i][e] = dot2(pp, vp[e], acc[i][e]);
          }
        }
      }
    };

    // software pipeline: the next step's loads are issued before this step's math
    load_step(it.lo, kA, vA);
    for (int k0 = it.lo; k0 < it.hi; k0 += 2 * STEP) {
      if (k0 + STEP < it.hi) load_step(k0 + STEP, kB, vB);
      compute_step(k0, kA, vA);
      if (k0 + 2 * STEP < it.hi) load_step(k0 + 2 * STEP, kA, vA);
      if (k0 + STEP < it.hi) compute_step(k0 + STEP, kB, vB);
    }

    // ---- combine the token slots; broadcast l, m of every head ----
    l_own = slots_sum<B>(l_own);
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = slots_sum<B>(acc[i][e]);
    float lh[G], mh[G];
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((lh[I] = bcast<LPT, (I << (B - LG))>(l_own)), ...);
      ((mh[I] = bcast<LPT, (I << (B - LG))>(m_own)), ...);
    }(std::make_integer_sequence<int, G>{});
    if (slot == 0) {
      const float vs = p.v_scale;
      if (it.part < 0) {
        QT* op = static_cast<QT*>(p.out);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int h = g * G + i;
          float ll = lh[i], f = 1.f;
          if (p.sink) {
            const float sg = p.sink[h] * kLog2e;
            const float mx = fmaxf(mh[i], sg);
            f = __builtin_amdgcn_exp2f(mh[i] - mx);
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
          const long long pb = (long long)it.part * p.Hq + g * G + i;
          if (dl == 0) {
            part_ml[2 * pb] = mh[i];
            part_ml[2 * pb + 1] = lh[i];
          }
#pragma unroll
          for (int e = 0; e < EPL; ++e) part_acc[pb * D + dl * EPL + e] = acc[i][e];
        }
      }
    }
    (void)my_head;
  }
}

// Stand-alone merge of the split partials (when no prefill kernel runs after
// the row kernel to do it): four merge items per workgroup.
template <typename QT, int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const long long total = (long long)hdr->n_merge_rows * p.Hkv;
  for (long long idx = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); idx < total;
       idx += (long long)gridDim.x * 4)
    merge_one<QT, D, G>(p, idx);
}

// Workgroups of `kernel` that fit on the device at once (occupancy x CUs).
int resident_blocks(const void* kernel, int block_threads, size_t lds) {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, lds) !=
          hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 1024;
  return per_cu * cus > 0 ? per_cu * cus : 1024;
}

template <typename QT, typename CT, int D, int G>
hipError_t launch_rows_t(const AttnParams& p, hipStream_t s) {
  // elements per lane: one 16-byte load, at most 64 accumulators per lane
  constexpr int E16 = 16 / (int)sizeof(CT);
  constexpr int EPL = (E16 * G > 64) ? (64 / G) : E16;
  constexpr int NR = 4;
  static const int cap = resident_blocks(
      reinterpret_cast<const void*>(&row_kernel<QT, CT, D, G, EPL, NR>), 64 * kWavesPerWG, 0);
  const long long waves = (long long)p.lay.max_items * p.Hkv;
  const long long wgs = (waves + kWavesPerWG - 1) / kWavesPerWG;
  dim3 grid((unsigned)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap));
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

namespace {
template <typename QT, int D>
hipError_t launch_merge_d(const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: merge_kernel<QT, D, 1><<<grid, 256, 0, s>>>(p); break;
    case 2: merge_kernel<QT, D, 2><<<grid, 256, 0, s>>>(p); break;
    case 4: merge_kernel<QT, D, 4><<<grid, 256, 0, s>>>(p); break;
    case 8: merge_kernel<QT, D, 8><<<grid, 256, 0, s>>>(p); break;
    case 16: merge_kernel<QT, D, 16><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_merge(const AttnParams& p, rpa_dtype q_dt, hipStream_t s) {
  const long long waves = (long long)p.lay.max_merge_rows * p.Hkv;
  if (waves <= 0) return hipSuccess;
  const long long wgs = (waves + 3) / 4;
  const dim3 grid((unsigned)(wgs < 4096 ? wgs : 4096));
  if (q_dt == RPA_F32) {
    return p.D == 64 ? launch_merge_d<float, 64>(p, grid, s) : launch_merge_d<float, 128>(p, grid, s);
  }
  return p.D == 64 ? launch_merge_d<uint16_t, 64>(p, grid, s)
                   : launch_merge_d<uint16_t, 128>(p, grid, s);
}

}  // namespace rpa
