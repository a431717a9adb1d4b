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

#include <cstdio>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "merge.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

// Per-wave clock stamps of the row kernels, compiled only into the
// measurement build (RPA_WAVE_TIMELINE, librpa_timeline.so): for wave w of
// a launch, its start, the end of its first step and its end on the 100 MHz
// constant clock, its step count and its CU (HW_ID) and XCD (XCC_ID).  They
// show how the waves of a launch share the chip; the library never reads
// them.
#ifdef RPA_WAVE_TIMELINE
constexpr int kTimelineWaves = 8192;
__device__ unsigned long long g_timeline[kTimelineWaves * 4];
__device__ __forceinline__ void timeline_put(long long w, unsigned long long t0,
                                             unsigned long long t1, int steps) {
  const unsigned long long t2 = __builtin_amdgcn_s_memrealtime();
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID, 32 bits
  const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID, 32 bits
  if ((threadIdx.x & 63) == 0 && w >= 0 && w < kTimelineWaves) {
    g_timeline[w * 4 + 0] = t0;
    g_timeline[w * 4 + 1] = t1;
    g_timeline[w * 4 + 2] = t2;
    g_timeline[w * 4 + 3] = ((unsigned long long)steps << 32) | ((xcc & 0xFu) << 16) | (hw & 0xFFFFu);
  }
}
#define RPA_TL_BEGIN()                                                      \
  const unsigned long long tl_t0 = __builtin_amdgcn_s_memrealtime();        \
  unsigned long long tl_t1 = 0;                                             \
  int tl_steps = 0
#define RPA_TL_STEP()                                                       \
  do {                                                                      \
    if (tl_steps++ == 0) tl_t1 = __builtin_amdgcn_s_memrealtime();         \
  } while (0)
#define RPA_TL_END(w) timeline_put((w), tl_t0, tl_t1, tl_steps)
#else
#define RPA_TL_BEGIN() static_assert(true, "")
#define RPA_TL_STEP() static_assert(true, "")
#define RPA_TL_END(w) static_assert(true, "")
#endif

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

// v and its partner across lane bit K (4: 16-lane rows, 5: 32-lane halves)
// from a permlane swap of v with itself, without a trip through LDS.  Lane by
// lane the two outputs are {v, partner}: (v, partner) where bit K of the lane
// is clear, (partner, v) where it is set.
template <int K>
__device__ __forceinline__ void swap_pair(float v, float& a, float& b) {
  static_assert(K == 4 || K == 5, "rows or halves");
  const uint32_t u = __float_as_uint(v);
  if constexpr (K == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}
template <int K>
__device__ __forceinline__ float partner_of(float v) {
  float a, b;
  swap_pair<K>(v, a, b);
  return ((__lane_id() >> K) & 1) ? a : b;
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
  else return partner_of<K>(v);                       // lane ^ 16, lane ^ 32
}
// Exact partner lane ^ (1 << K) (values differ across the lower bits).
template <int K>
__device__ __forceinline__ float xor_x(float v) {
  if constexpr (K == 0) return dppf<0xB1>(v);
  else if constexpr (K == 1) return dppf<0x4E>(v);
  else if constexpr (K == 2) return swz<0x101F>(v);  // lane ^ 4
  else if constexpr (K == 3) return dppf<0x128>(v);  // row_ror:8 == lane ^ 8 in a row
  else return partner_of<K>(v);
}

// Value of lane REP of this lane's aligned group of LPT lanes, by DPP and
// permlane moves (no trip through LDS).
template <int LPT, int REP>
__device__ __forceinline__ float bcast(float v) {
  const int x = __float_as_int(v);
  if constexpr (LPT == 1) {
    return v;
  } else if constexpr (LPT == 2) {
    // quad_perm [REP, REP, 2 + REP, 2 + REP]
    constexpr int c = REP | (REP << 2) | ((2 + REP) << 4) | ((2 + REP) << 6);
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, c, 0xF, 0xF, false));
  } else if constexpr (LPT == 4) {
    constexpr int c = REP * 0x55;  // quad_perm [REP, REP, REP, REP]
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, c, 0xF, 0xF, false));
  } else if constexpr (LPT == 8) {
    // lane REP % 4 of every quad, then row_half_mirror (lane 4 + j <- 3 - j
    // within each 8 lanes) written only into the quads (banks) not holding REP
    const int t = __builtin_amdgcn_mov_dpp(x, (REP & 3) * 0x55, 0xF, 0xF, false);
    constexpr int banks = (REP < 4) ? 0xA : 0x5;
    return __int_as_float(__builtin_amdgcn_update_dpp(t, t, 0x141, 0xF, banks, false));
  } else if constexpr (LPT == 16) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x150 + REP, 0xF, 0xF, false));
  } else if constexpr (LPT == 32) {
    // lane REP % 16 of every row, then the row of REP within the 32-lane half
    const float t =
        __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x150 + (REP & 15), 0xF, 0xF, false));
    float a, b;
    swap_pair<4>(t, a, b);           // lane by lane {t, t of the partner row}
    const bool own = ((__lane_id() >> 4) & 1) == (REP >> 4);
    const bool hi = (__lane_id() >> 4) & 1;
    return own ? t : (hi ? a : b);
  } else {
    return __int_as_float(__builtin_amdgcn_readlane(x, REP));
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
// (over bits 4 and 5 the two swap outputs are {v, partner}: the op of the
// two is v op partner in every lane, as the ops commute)
template <int B>
__device__ __forceinline__ float slots_max(float v) {
  if constexpr (B >= 4 && B <= 5) {
    float a, b;
    swap_pair<B>(v, a, b);
    return slots_max<B + 1>(fmaxf(a, b));
  } else if constexpr (B <= 5) {
    v = fmaxf(v, xor_x<B>(v));
    return slots_max<B + 1>(v);
  }
  return v;
}
template <int B>
__device__ __forceinline__ float slots_sum(float v) {
  if constexpr (B >= 4 && B <= 5) {
    float a, b;
    swap_pair<B>(v, a, b);
    return slots_sum<B + 1>(a + b);
  } else if constexpr (B <= 5) {
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

// e4m3 codes -> bf16 pairs of consecutive elements (exact widening: the
// scaled convert with scale 1 matched cvt_pk_f32_fp8 + bf16 truncation on all
// 65536 code pairs on the MI355X)
template <int NW>
__device__ __forceinline__ void widen_fp8(const uint32_t* w, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.f, false));
    out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.f, true));
  }
}

// A lane's EPL consecutive output elements v * scale as bf16 (round to
// nearest even) or fp32, with 16- or 8-byte stores (o and the slice offset
// are multiples of the store width).
template <typename QT, int EPL>
__device__ __forceinline__ void store_slice(QT* o, long long base, const float* v, float scale) {
  constexpr int BYTES = EPL * (int)sizeof(QT);
  if constexpr (sizeof(QT) == 2 && BYTES % 8 == 0) {
    constexpr int NWD = EPL / 2;
    uint32_t w[NWD];
#pragma unroll
    for (int k = 0; k < NWD; ++k)
      w[k] = f32_to_bf16(v[2 * k] * scale) | (f32_to_bf16(v[2 * k + 1] * scale) << 16);
    if constexpr (NWD % 4 == 0) {
#pragma unroll
      for (int k = 0; k < NWD; k += 4)
        *reinterpret_cast<uint4*>(o + base + 2 * k) = make_uint4(w[k], w[k + 1], w[k + 2], w[k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < NWD; k += 2)
        *reinterpret_cast<uint2*>(o + base + 2 * k) = make_uint2(w[k], w[k + 1]);
    }
  } else if constexpr (sizeof(QT) == 4 && EPL % 4 == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(o + base + e) =
          make_float4(v[e] * scale, v[e + 1] * scale, v[e + 2] * scale, v[e + 3] * scale);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) store_out<QT>(o, base + e, v[e] * scale);
  }
}

// QT: query type (float, uint16_t = bf16, or uint8_t = e4m3 codes, widened
// exactly to bf16 on load); the output is QT, or bf16 for e4m3 queries.
template <typename QT, typename CT, int D, int G, int EPL, int NR, bool CAP>
__global__ __launch_bounds__(64 * kWavesPerWG) void row_kernel(AttnParams p) {
  RPA_TL_BEGIN();
  using OT = std::conditional_t<sizeof(QT) == 1, uint16_t, QT>;
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
  // Where registers allow (two waves per SIMD kept), the next item's q and
  // first K/V loads are issued before this item's epilogue.
  constexpr bool kLean = G * NP <= 16;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const ItemDesc* items = reinterpret_cast<const ItemDesc*>(p.ws + p.lay.items);
  float* part_ml = reinterpret_cast<float*>(p.ws + p.lay.part_ml);
  float* part_acc = reinterpret_cast<float*>(p.ws + p.lay.part_acc);

  const int lane = lane_id();
  const int slot = lane / LPT;          // token slot within a load row
  const int dl = lane % LPT;            // d-slice
  const int my_head = dl >> (B - LG);   // head whose logit this lane holds after the scatter
  const int Hkv = p.Hkv;
  const int n_items = hdr->n_items;
  const int32_t* chunk_first = reinterpret_cast<const int32_t*>(p.ws + p.lay.chunks);
  const long long total = (long long)hdr->n_chunks * Hkv;  // (chunk, kv head) pairs
  const int sh = p.ps_shift;                        // page_size = 1 << sh
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * (uint32_t)sizeof(CT);  // one cache token row
  const uint32_t head_bytes = p.Dpad * (uint32_t)sizeof(CT);            // K -> V of a head
  const CT* cache = static_cast<const CT*>(p.cache);
  constexpr bool use_cap = CAP;       // logits soft cap on (p.cap > 0), chosen at launch
  const float c_log2 = p.qk_scale * kLog2e;
  const float cap_k = use_cap ? p.qk_scale * 2.f * kLog2e / p.cap : 0.f;  // x -> 2x log2 e
  const float cap_l2 = p.cap * kLog2e;

  // Wave-uniform view of a work item: (row, KV split, kv head g).
  struct Item {
    int token, seq, lo, hi, part, g;
  };
  int g = 0, i_last = 0;  // kv head and item end of the wave's current chunk
  auto desc_at = [&](int i) __attribute__((always_inline)) {
    return items[i < i_last ? i : i_last - 1];
  };
  auto make_item = [&](const ItemDesc& d) __attribute__((always_inline)) {
    Item r;
    r.token = __builtin_amdgcn_readfirstlane(d.token);
    r.seq = __builtin_amdgcn_readfirstlane(d.seq);
    r.lo = __builtin_amdgcn_readfirstlane(d.lo);
    r.hi = __builtin_amdgcn_readfirstlane(d.hi);
    r.part = __builtin_amdgcn_readfirstlane(d.part);
    r.g = g;
    return r;
  };
  // q of the G heads of item `it`, this lane's d-slice: fp32 values or bf16
  // pairs (e4m3 codes widened exactly, four per loaded word)
  auto load_q = [&](const Item& it, uint32_t (*qw)[NP]) __attribute__((always_inline)) {
    const QT* qp =
        static_cast<const QT*>(p.q) + ((long long)it.token * p.Hq + it.g * G) * D + dl * EPL;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if constexpr (sizeof(QT) == 4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qw[i][e] = __float_as_uint(qp[i * D + e]);
      } else if constexpr (sizeof(QT) == 1) {
        static_assert(EPL % 4 == 0, "whole words of e4m3 codes");
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(qp + i * D)[e];
          qw[i][2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, false));
          qw[i][2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, true));
        }
      } else {
#pragma unroll
        for (int e = 0; e < NP; ++e) qw[i][e] = reinterpret_cast<const uint32_t*>(qp + i * D)[e];
      }
    }
  };
  // Page ids of a 64-page window from page k0 >> sh on: lane i holds the i-th.
  auto load_window = [&](const Item& it, int k0, int& pw0, int& page_reg)
      __attribute__((always_inline)) {
    pw0 = k0 >> sh;
    const int pi = pw0 + lane;
    const int* bt = p.block_tables + (long long)it.seq * p.pps;
    page_reg = (pi <= ((it.hi - 1) >> sh)) ? bt[pi] : 0;
  };
  // Loads of one step of item `it`, whose tokens below `lim` lie in the page
  // window held in page_reg.  Tokens from `lim` on are clamped to lim - 1
  // (valid memory, masked out of the softmax), so every load is
  // unconditional.  No page id is loaded here: a global load inside the step
  // loop would make every step wait for all loads in flight (the wait counter
  // is in order), so windows are switched between chunks of an item instead.
  auto load_step = [&](const Item& it, int lim, int pw0, int page_reg, int k0,
                       uint32_t (*kw)[NW], uint32_t (*vw)[NW]) __attribute__((always_inline)) {
    const char* kv_head = reinterpret_cast<const char*>(cache + 2LL * it.g * p.Dpad + dl * EPL);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int tok = min(k0 + r * TPR + slot, lim - 1);
      const int page = __builtin_amdgcn_ds_bpermute(((tok >> sh) - pw0) << 2, page_reg);
      const uint32_t row = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
      const char* kp = kv_head + (uint64_t)row * row_bytes;
      load_chunk<CT, EPL>(reinterpret_cast<const CT*>(kp), true, kw[r]);
      load_chunk<CT, EPL>(reinterpret_cast<const CT*>(kp + head_bytes), true, vw[r]);
    }
  };
  // end of the chunk of `it` that starts at token c: the tokens whose pages
  // lie in the 64-page window from page c >> sh on
  auto chunk_end = [&](const Item& it, int c) __attribute__((always_inline)) {
    const long long e = ((long long)(c >> sh) + 64) << sh;
    return e < it.hi ? (int)e : it.hi;
  };

  // Wave w takes (chunk, kv head) pair w: the grid has a wave for every pair
  // (the planner makes at most row_chunks_max(resident waves, Hkv) chunks and
  // the launch has that many waves per kv head), and the chunks hold equal
  // numbers of keys, so the waves end together.  The wave walks the chunk's
  // items; they overlap: while the wave works on one, the descriptor of the
  // item after next and the first page window of the next are in flight.
  const long long ch = (long long)blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  if (ch >= total) return;
  const int c = (int)(ch / Hkv);
  g = (int)(ch - (long long)c * Hkv);
  const int i_first = min(max(__builtin_amdgcn_readfirstlane(chunk_first[c]), 0), n_items);
  i_last = min(max(__builtin_amdgcn_readfirstlane(chunk_first[c + 1]), i_first), n_items);
  if (i_first >= i_last) return;

  Item cur = make_item(desc_at(i_first));
  uint32_t qw[G][NP];
  load_q(cur, qw);
  int pw0 = 0, page_reg = 0;
  load_window(cur, cur.lo, pw0, page_reg);
  int idx_n = i_first + 1;
  ItemDesc desc_n = desc_at(idx_n);
  uint32_t kA[NR][NW], vA[NR][NW], kB[NR][NW], vB[NR][NW];
  load_step(cur, chunk_end(cur, cur.lo), pw0, page_reg, cur.lo, kA, vA);

  while (true) {
    const bool has_next = idx_n < i_last;
    const Item nxt = make_item(desc_n);  // a clamped, valid item when !has_next
    uint32_t qw_n[G][NP];
    if constexpr (kLean) load_q(nxt, qw_n);
    int pw0_n = 0, page_reg_n = 0;
    load_window(nxt, nxt.lo, pw0_n, page_reg_n);
    const int idx_nn = idx_n + 1;
    desc_n = desc_at(idx_nn);

    float acc[G][EPL];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
    float m_own = -INFINITY, l_own = 0.f;  // softmax state of head my_head

    auto compute_step = [&](int k0, int lim, uint32_t (*kw)[NW], uint32_t (*vw)[NW])
        __attribute__((always_inline)) {
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
        if constexpr (F32) {
          s = use_cap ? p.cap * tanhf(s * p.qk_scale / p.cap) * kLog2e : s * c_log2;
        } else if (use_cap) {
          // cap * tanh(x) in log2 units with tanh(x) = 1 - 2 / (e^{2x} + 1):
          // one exp2 and one reciprocal (well inside the bf16 / e4m3 bounds)
          const float e2 = __builtin_amdgcn_exp2f(s * cap_k);
          s = cap_l2 * (1.f - 2.f * __builtin_amdgcn_rcpf(e2 + 1.f));
        } else {
          s *= c_log2;
        }
        const bool valid = k0 + r * TPR + slot < lim;
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
    for (int c_lo = cur.lo;;) {
      const int c_hi = chunk_end(cur, c_lo);
      // The loads are unconditional (past the chunk they re-read its last
      // token, masked): a load issued on one path only would make the
      // following waits drain every load in flight.  A fully masked step
      // adds exactly nothing (p = 0), and the chunk's first step is never
      // empty, so the running max is finite from then on.
      for (int k0 = c_lo; k0 < c_hi; k0 += 2 * STEP) {
        load_step(cur, c_hi, pw0, page_reg, k0 + STEP, kB, vB);
        compute_step(k0, c_hi, kA, vA);
        RPA_TL_STEP();
        load_step(cur, c_hi, pw0, page_reg, k0 + 2 * STEP, kA, vA);
        compute_step(k0 + STEP, c_hi, kB, vB);
        RPA_TL_STEP();
      }
      if (c_hi >= cur.hi) break;
      c_lo = c_hi;
      load_window(cur, c_lo, pw0, page_reg);
      load_step(cur, chunk_end(cur, c_lo), pw0, page_reg, c_lo, kA, vA);
    }
    if constexpr (kLean) {
      if (has_next) load_step(nxt, chunk_end(nxt, nxt.lo), pw0_n, page_reg_n, nxt.lo, kA, vA);
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
      if (cur.part < 0) {
        OT* op = static_cast<OT*>(p.out);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int h = cur.g * G + i;
          float ll = lh[i], f = 1.f;
          if (p.sink) {
            const float sg = p.sink[h] * kLog2e;
            const float mx = fmaxf(mh[i], sg);
            f = __builtin_amdgcn_exp2f(mh[i] - mx);
            ll = ll * f + __builtin_amdgcn_exp2f(sg - mx);
          }
          const float scale = f * vs / ll;
          const long long base = ((long long)cur.token * p.Hq + h) * D + dl * EPL;
          store_slice<OT, EPL>(op, base, acc[i], scale);
        }
      } else if (cur.part < p.lay.max_parts) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const long long pb = (long long)cur.part * p.Hq + cur.g * G + i;
          if (dl == 0) {
            part_ml[2 * pb] = mh[i];
            part_ml[2 * pb + 1] = lh[i];
          }
          store_slice<float, EPL>(part_acc, pb * D + dl * EPL, acc[i], 1.f);
        }
      }
    }
    (void)my_head;
    if (!has_next) break;
    cur = nxt;
    if constexpr (kLean) {
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < NP; ++e) qw[i][e] = qw_n[i][e];
    } else {
      load_q(cur, qw);
    }
    pw0 = pw0_n;
    page_reg = page_reg_n;
    idx_n = idx_nn;
    if constexpr (!kLean) load_step(cur, chunk_end(cur, cur.lo), pw0, page_reg, cur.lo, kA, vA);
  }
  RPA_TL_END(ch);
}

// ---------------------------------------------------------------------------
// Row kernel for large GQA groups (G = 8 or 16 q heads per kv head, bf16
// queries or e4m3 ones widened exactly to bf16, bf16 or e4m3 cache) on
// v_mfma_f32_16x16x32_bf16.  With G >= 8 the
// dot products of the VALU kernel above outweigh the HBM time; here they run
// on the matrix cores and the wave keeps up with its loads.  Same plan, work
// items, split partials and output as the VALU kernel.
//
// A step covers 32 tokens, two groups of 16.  K and V rows are loaded whole
// (16 bytes per lane, as many lanes as a row needs), widened to bf16 and
// written to the wave's LDS, from which the MFMA operands are read.
// Lane l: c16 = l % 16, g4 = l / 16.
//   S = K Q^T per group (16 tokens x 16 heads): A = K, lane (token c16,
//     d 32 m + 8 g4 .. + 8) by ds_read_b128; B = Q^T, lane (head c16, the same
//     d).  S lands as lane (head c16, tokens 4 g4 .. 4 g4 + 3).
//   O += P V (16 heads x 16 d per MFMA, k = 32 tokens): A = P, lane (head c16,
//     token slots 8 g4 + j = tokens 4 g4 + j of group 0 and of group 1), i.e.
//     exactly the p of the lane's own S values; B = V, lane (d c16, the same
//     tokens), read transposed (ds_read_b64_tr_b16) from the wave's copy of
//     the step's V rows in LDS (rows padded to spread the banks).
//     O lands as lane (d c16 of the block, heads 4 g4 .. 4 g4 + 3).
// Heads past G (G = 8) have zero q and are never stored.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3)))* lds_i16x4_ptr;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename CT, int D>
struct MfCfg {
  static constexpr int ESZ = (int)sizeof(CT);
  static constexpr int E = 16 / ESZ;         // elements per 16-byte load
  static constexpr int LPTK = D * ESZ / 16;  // lanes per K (or V) row of a token
  static constexpr int TPI = 64 / LPTK;      // tokens per load instruction
  static constexpr int NLI = 32 / TPI;       // load instructions per step (K; as many for V)
  static constexpr int NMQ = D / 32;         // q.k MFMAs per 16 tokens
  static constexpr int NMP = D / 16;         // p.v MFMAs per step
  // staged bf16 rows, padded: K rows by 16 bytes (16 rows at one column hit
  // distinct banks), V rows by 32 (4 rows x 32 bytes of a transposed read do)
  static constexpr int LRK = 2 * D + 16;
  static constexpr int LRV = 2 * D + 32;
  static constexpr int LWAVE = 32 * (LRK + LRV);  // LDS bytes per wave
};

// Issue priority of the wave (0 lowest .. 3).  The CU's arbiter prefers the
// highest priority, then the oldest wave; a wave lowers its priority as it
// gets through its chunk, so the waves that started later are not starved
// of loads by the older ones and all finish together.
__device__ __forceinline__ void wave_priority(int pr) {
  switch (pr) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

__device__ __forceinline__ u32x4 nt_load16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// SH (kv heads a multiple of 4, no lane padding): the 4 waves of a workgroup
// hold 4 consecutive kv heads of one chunk (wave w = head 4j + w), so they
// walk the same items in step.  Their K and V rows are contiguous 4-head runs
// of 8 D element-bytes per token (512 bytes for e4m3 at D = 64): each wave
// loads whole runs of 8 of the step's 32 tokens and stages every 16-byte
// piece into the LDS rows of the wave whose head it holds, between two
// workgroup barriers.  Reading runs instead of each head's own 2 D bytes
// per token is what keeps the HBM reads long.
// The planner sizes its chunks by the resident waves of the form launched.
//
// Register buffers of the step stream: two (a step in LDS, two in flight)
// where they fit, one for bf16 rows at D = 128 (64 registers a step) and for
// bf16 rows at D = 64 without shared loads (K and V loaded per head).  The
// minimum of waves per SIMD keeps the count the buffers were sized for.
template <typename CT, int D, bool SH>
constexpr int mfma_row_nbuf() {
  return (sizeof(CT) == 2 && (D == 128 || !SH)) ? 1 : 2;
}
template <typename CT, int D, bool SH>
constexpr int mfma_row_min_waves() {
  return D == 64 ? (mfma_row_nbuf<CT, D, SH>() == 2 ? 3 : 4) : (mfma_row_nbuf<CT, D, SH>() == 2 ? 2 : 1);
}

template <typename CT, int D, int G, bool CAP, bool QF8, bool SH>
__global__ __launch_bounds__(64 * kWavesPerWG)
__attribute__((amdgpu_waves_per_eu(mfma_row_min_waves<CT, D, SH>()))) void mfma_row_kernel(AttnParams p) {
  constexpr int NBUF = mfma_row_nbuf<CT, D, SH>();
  RPA_TL_BEGIN();
  using Cfg = MfCfg<CT, D>;
  constexpr int ESZ = Cfg::ESZ, E = Cfg::E, LPTK = Cfg::LPTK, TPI = Cfg::TPI, NLI = Cfg::NLI,
                NMQ = Cfg::NMQ, NMP = Cfg::NMP, LRK = Cfg::LRK, LRV = Cfg::LRV;
  constexpr bool FP8 = sizeof(CT) == 1;
  static_assert(G == 8 || G == 16, "16-head MFMA columns");
  static_assert(LPTK >= 1 && TPI * NLI == 32, "load split");
  __shared__ __attribute__((aligned(16))) char s_v[kWavesPerWG * Cfg::LWAVE];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const ItemDesc* items = reinterpret_cast<const ItemDesc*>(p.ws + p.lay.items);
  float* part_ml = reinterpret_cast<float*>(p.ws + p.lay.part_ml);
  float* part_acc = reinterpret_cast<float*>(p.ws + p.lay.part_acc);
  const int32_t* chunk_first = reinterpret_cast<const int32_t*>(p.ws + p.lay.chunks);

  const int lane = lane_id();
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wave = threadIdx.x >> 6;
  char* kt = s_v + wave * Cfg::LWAVE;          // K rows of the step (bf16)
  char* vt = kt + 32 * LRK;                     // V rows of the step (bf16)
  const int Hkv = p.Hkv;
  const int n_items = hdr->n_items;
  const long long total = (long long)hdr->n_chunks * Hkv;
  const int sh = p.ps_shift;
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * (uint32_t)ESZ;
  const uint32_t head_bytes = p.Dpad * (uint32_t)ESZ;
  constexpr bool use_cap = CAP;       // logits soft cap on (p.cap > 0), chosen at launch
  const float c_log2 = p.qk_scale * kLog2e;
  const float cap_k = use_cap ? p.qk_scale * 2.f * kLog2e / p.cap : 0.f;
  const float cap_l2 = p.cap * kLog2e;

  const long long ch = (long long)blockIdx.x * kWavesPerWG + wave;
  const int c = (int)(ch / Hkv);
  const int g = (int)(ch - (long long)c * Hkv);
  // the chunk's item range is read beside the header (c clamped into the
  // table; waves past the plan's chunks leave below)
  const int cc = min(c, p.lay.max_chunks - 1);
  const int cf0 = __builtin_amdgcn_readfirstlane(chunk_first[cc]);
  const int cf1 = __builtin_amdgcn_readfirstlane(chunk_first[cc + 1]);
  if (ch >= total) return;
  const int i_first = min(max(cf0, 0), n_items);
  const int i_last = min(max(cf1, i_first), n_items);
  if (i_first >= i_last) return;
  const char* kv_head = reinterpret_cast<const char*>(p.cache) + 2LL * g * p.Dpad * ESZ;
  // SH: this workgroup's run of 4 heads, and the loads that cover it
  constexpr int RUN = 8 * D * ESZ;               // bytes of 4 heads' K and V of a token
  constexpr int NLS = RUN / 128;                 // 16-byte loads per lane per step (8 runs a wave)
  static_assert(!SH || (RUN % 1024 == 0 || 1024 % RUN == 0), "runs tile 1 KiB loads");
  const char* kv_run = reinterpret_cast<const char*>(p.cache) + 2LL * (g & ~3) * D * ESZ;
  static_assert(kWavesPerWG == 4, "SH: one wave per head of a group of 4");

  struct Desc {
    int token, seq, lo, hi, part;
  };
  auto read_desc = [&](int i) __attribute__((always_inline)) {
    const ItemDesc dsc = items[i];
    Desc r;
    r.token = __builtin_amdgcn_readfirstlane(dsc.token);
    r.seq = __builtin_amdgcn_readfirstlane(dsc.seq);
    r.lo = __builtin_amdgcn_readfirstlane(dsc.lo);
    r.hi = __builtin_amdgcn_readfirstlane(dsc.hi);
    r.part = __builtin_amdgcn_readfirstlane(dsc.part);
    return r;
  };
  // lane i: the page of the 64-page window from page pw of item d's sequence
  // (0 past the item's last page)
  auto window_pages = [&](const Desc& d, int pw) __attribute__((always_inline)) {
    const int pi = pw + lane;
    return (pi <= ((d.hi - 1) >> sh)) ? p.block_tables[(long long)d.seq * p.pps + pi] : 0;
  };
  // end of the window that holds key k of item d
  auto chunk_end = [&](const Desc& d, int k) __attribute__((always_inline)) {
    const long long e = ((long long)(k >> sh) + 64) << sh;
    return e < d.hi ? (int)e : d.hi;
  };
  // K and V rows of the 32 tokens from k0: instruction i, lane l loads 16
  // bytes of token k0 + TPI i + l / LPTK (tokens from lim on re-read lim - 1),
  // pages from the window (pw, pg)
  auto load_step = [&](int pw, int pg, int lim, int k0, u32x4* kw, u32x4* vw) __attribute__((always_inline)) {
    const uint32_t off = 16u * (uint32_t)(lane % LPTK);
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int tok = min(k0 + TPI * i + lane / LPTK, lim - 1);
      const int page = __builtin_amdgcn_ds_bpermute(((tok >> sh) - pw) << 2, pg);
      const uint32_t row = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
      const char* kp = kv_head + (uint64_t)row * row_bytes + off;
      kw[i] = nt_load16(kp);
      vw[i] = nt_load16(kp + head_bytes);
    }
  };
  // one loaded 16-byte piece -> bf16 in LDS at dst (16 or 32 bytes)
  auto stage = [&](const u32x4& w, char* dst) __attribute__((always_inline)) {
    if constexpr (FP8) {
      uint32_t x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[k], 1.f, false));
        x[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[k], 1.f, true));
      }
      *reinterpret_cast<uint4*>(dst) = make_uint4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(x[4], x[5], x[6], x[7]);
    } else {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  // the step's K and V rows -> LDS as bf16 (row = token - k0)
  auto stage_step = [&](const u32x4* kw, const u32x4* vw) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int r = TPI * i + lane / LPTK;
      const int cb = 2 * E * (lane % LPTK);
      stage(kw[i], kt + r * LRK + cb);
      stage(vw[i], vt + r * LRV + cb);
    }
  };
  // SH: the runs of tokens k0 + 8 wave .. + 7 (from lim on, lim - 1 again):
  // load i, lane l holds bytes 1024 i + 16 l of the wave's 8 runs
  auto load_runs = [&](int pw, int pg, int lim, int k0, u32x4* rw) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < (SH ? NLS : 0); ++i) {
      const int b = 1024 * i + 16 * lane;
      const int tok = min(k0 + 8 * wave + b / RUN, lim - 1);
      const int page = __builtin_amdgcn_ds_bpermute(((tok >> sh) - pw) << 2, pg);
      const uint32_t row = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
      rw[i] = nt_load16(kv_run + (uint64_t)row * row_bytes + (b % RUN));
    }
  };
  // SH: each loaded piece -> the K or V row (token - k0) of the wave that
  // owns its head, widened to bf16 as stage() does
  auto stage_runs = [&](const u32x4* rw) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < (SH ? NLS : 0); ++i) {
      const int b = 1024 * i + 16 * lane;
      const int r = 8 * wave + b / RUN;
      const int in_run = b % RUN;
      const int hl = in_run / (2 * D * ESZ);                 // head of the group
      const bool isv = (in_run % (2 * D * ESZ)) >= D * ESZ;
      const int chunk = (in_run % (D * ESZ)) / 16;
      char* base = s_v + hl * Cfg::LWAVE;
      char* dst = isv ? base + 32 * LRK + r * LRV : base + r * LRK;
      stage(rw[i], dst + 2 * E * chunk);
    }
  };

  // The wave's steps form one stream over its items and their page windows.
  // A load cursor runs NBUF steps ahead of the step being computed: each
  // step's rows go from their register buffer to LDS, the buffer is refilled
  // with the step NBUF ahead, and those loads stay in flight while this and
  // the next NBUF - 1 steps are computed.  Past the wave's last key the
  // cursor re-reads that key, so every step issues the same loads and no
  // wait drains them early.
  constexpr int NB = SH ? NLS : 2 * NLI;         // 16-byte loads per lane per step
  struct LoadCursor {
    Desc d;
    int ii, pw, pg, k0, lim;   // item, page window (first page, lane's page), step, window end
    bool done;
  };
  LoadCursor L;
  L.ii = i_first;
  L.d = read_desc(i_first);
  L.pw = L.d.lo >> sh;
  L.pg = window_pages(L.d, L.pw);
  L.k0 = L.d.lo;
  L.lim = chunk_end(L.d, L.d.lo);
  L.done = false;
  auto advance = [&]() __attribute__((always_inline)) {
    if (L.done) return;
    L.k0 += 32;
    if (L.k0 < L.lim) return;
    if (L.lim < L.d.hi) {                        // the item's next page window
      L.pw = L.lim >> sh;
      L.pg = window_pages(L.d, L.pw);
      L.k0 = L.lim;
      L.lim = chunk_end(L.d, L.k0);
    } else if (L.ii + 1 < i_last) {              // the next item
      ++L.ii;
      L.d = read_desc(L.ii);
      L.pw = L.d.lo >> sh;
      L.pg = window_pages(L.d, L.pw);
      L.k0 = L.d.lo;
      L.lim = chunk_end(L.d, L.k0);
    } else {                                     // past the end: the last key again
      L.done = true;
      L.k0 = L.lim - 1;
    }
  };
  auto issue = [&](u32x4* buf) __attribute__((always_inline)) {
    if constexpr (SH) load_runs(L.pw, L.pg, L.lim, L.k0, buf);
    else load_step(L.pw, L.pg, L.lim, L.k0, buf, buf + NLI);
  };
  auto stage_buf = [&](const u32x4* buf) __attribute__((always_inline)) {
    if constexpr (SH) stage_runs(buf);
    else stage_step(buf, buf + NLI);
  };

  // q^T operands of item d: lane (head c16, d slots of g4) per MFMA (e4m3
  // queries widened exactly to bf16)
  bf16x8 qb[NMQ];
  auto load_q = [&](const Desc& d) __attribute__((always_inline)) {
    const long long qrow = (long long)d.token * p.Hq + g * G + (c16 < G ? c16 : 0);
#pragma unroll
    for (int m = 0; m < NMQ; ++m) {
      const int d0 = 32 * m + 8 * g4;
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (QF8) {
        if (c16 < G) {
          const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(p.q) + qrow * D + d0);
          v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.f, false));
          v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.f, true));
          v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.f, false));
          v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.f, true));
        }
      } else {
        if (c16 < G) v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qrow * D + d0);
      }
      qb[m] = __builtin_bit_cast(bf16x8, v);
    }
  };

  f32x4 o[NMP];
  float m_run, l_run;   // head c16
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NMP; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  auto compute_step = [&](int k0, int lim) __attribute__((always_inline)) {
    // ---- S = K Q^T for the two groups ----
    f32x4 sg[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sg[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const char* kr = kt + (16 * t + c16) * LRK + 16 * g4;
#pragma unroll
      for (int m = 0; m < NMQ; ++m) {
        const uint4 a = *reinterpret_cast<const uint4*>(kr + 64 * m);
        sg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qb[m], sg[t], 0, 0, 0);
      }
    }
    // ---- logits of head c16 for tokens k0 + 16 t + 4 g4 + e, online softmax ----
    float x[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = sg[t][e];
        if (use_cap) {
          const float e2 = __builtin_amdgcn_exp2f(s * cap_k);
          s = cap_l2 * (1.f - 2.f * __builtin_amdgcn_rcpf(e2 + 1.f));
        } else {
          s *= c_log2;
        }
        x[4 * t + e] = (k0 + 16 * t + 4 * g4 + e < lim) ? s : -INFINITY;
      }
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bm = fmaxf(bm, x[i]);
    bm = slots_max<4>(bm);                    // over the head's four lane groups
    if (__any(bm > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, bm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first step
      m_run = m_new;
      l_run *= alpha;
      // O rows are heads 4 g4 + e: their alpha sits in lane 4 g4 + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a_e = __shfl(alpha, 4 * g4 + e);
#pragma unroll
        for (int b = 0; b < NMP; ++b) o[b][e] *= a_e;
      }
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
      l_run += pr[i];
    }
    const uint4 pw = make_uint4(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]),
                                pack_bf16(pr[4], pr[5]), pack_bf16(pr[6], pr[7]));
    const bf16x8 pa = __builtin_bit_cast(bf16x8, pw);
    // ---- O += P V: B from the transposed V rows (tokens 4 g4 + j and 16 + 4 g4 + j) ----
    const char* r1 = vt + (4 * g4 + (c16 >> 2)) * LRV + 8 * (c16 & 3);
    const char* r2 = r1 + 16 * LRV;
#pragma unroll
    for (int b = 0; b < NMP; ++b) {
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(r1 + 32 * b));
      const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(r2 + 32 * b));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 vb = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[b], 0, 0, 0);
    }
  };

  // ---- epilogue of item d: l of head c16 over its lane groups; O rows are heads 4 g4 + e ----
  auto finish = [&](const Desc& d) __attribute__((always_inline)) {
    const float l_tot = slots_sum<4>(l_run);
    const float vs = p.v_scale;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hl = 4 * g4 + e;                 // head within the group
      const float l_h = __shfl(l_tot, hl);
      const float m_h = __shfl(m_run, hl);
      if (hl >= G) continue;
      const int h = g * G + hl;
      if (d.part < 0) {
        float ll = l_h, f = 1.f;
        if (p.sink) {
          const float sgk = p.sink[h] * kLog2e;
          const float mx = fmaxf(m_h, sgk);
          f = __builtin_amdgcn_exp2f(m_h - mx);
          ll = ll * f + __builtin_amdgcn_exp2f(sgk - mx);
        }
        const float scale = f * vs / ll;
        uint16_t* op = static_cast<uint16_t*>(p.out) + ((long long)d.token * p.Hq + h) * D;
#pragma unroll
        for (int b = 0; b < NMP; ++b) op[16 * b + c16] = (uint16_t)f32_to_bf16(o[b][e] * scale);
      } else if (d.part < p.lay.max_parts) {
        const long long pb = (long long)d.part * p.Hq + h;
        if (c16 == 0) {
          part_ml[2 * pb] = m_h;
          part_ml[2 * pb + 1] = l_h;
        }
#pragma unroll
        for (int b = 0; b < NMP; ++b) part_acc[pb * D + 16 * b + c16] = o[b][e];
      }
    }
  };

  // the step being computed: item ci (d, the next one dn), keys [k0, k0 + 32) of the window ending at lim
  int ci = i_first;
  Desc d = L.d;
  Desc dn = read_desc(min(ci + 1, i_last - 1));
  int k0 = d.lo, lim = L.lim;
  const int chunk_keys = max(hdr->split, 32);
  int keys_done = 0;
  wave_priority(3);
  u32x4 b0[NB], b1[NBUF == 2 ? NB : 1];
  issue(b0);
  advance();
  if constexpr (NBUF == 2) {
    issue(b1);
    advance();
  }
  load_q(d);
  reset();
  // one step from buffer buf; false once the wave's last item is finished
  auto step = [&](u32x4* buf) __attribute__((always_inline)) {
    if constexpr (SH) {
      // All 4 waves take the same items, windows and steps: the barriers
      // match.  (A) nobody still reads the LDS rows of the previous step;
      // (B) every wave's pieces of this step are staged.
      __syncthreads();                                   // (A)
      stage_buf(buf);
      issue(buf);
      __syncthreads();                                   // (B)
    } else {
      stage_buf(buf);
      issue(buf);
    }
    RPA_TL_STEP();
    advance();
    keys_done += 32;
    wave_priority(3 - min(3, (4 * keys_done) / chunk_keys));
    compute_step(k0, lim);
    k0 += 32;
    if (k0 < lim) return true;
    if (lim < d.hi) {                                    // the item's next page window
      k0 = lim;
      lim = chunk_end(d, k0);
      return true;
    }
    finish(d);
    if (ci + 1 >= i_last) return false;
    ++ci;
    d = dn;
    dn = read_desc(min(ci + 1, i_last - 1));
    load_q(d);
    reset();
    k0 = d.lo;
    lim = chunk_end(d, k0);
    return true;
  };
  for (;;) {
    if (!step(b0)) break;
    if constexpr (NBUF == 2) {
      if (!step(b1)) break;
    }
  }
  RPA_TL_END(ch);
}

// Stand-alone merge of the split partials (when no prefill kernel runs after
// the row kernel to do it): four merge items per workgroup, or one per
// workgroup for rows with many parts.
template <typename QT, int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  __shared__ float s_merge[merge_wg_floats<D, G>()];
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  merge_all<QT, D, G>(p, (long long)hdr->n_merge_rows * p.Hkv, s_merge);
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

// Row kernel configuration for these types and sizes.
template <typename QT, typename CT, int D, int G, bool CAP>
struct RowCfg {
  // elements per lane: one 16-byte load, at most 64 accumulators per lane
  static constexpr int E16 = 16 / (int)sizeof(CT);
  static constexpr int EPL = (E16 * G > 64) ? (64 / G) : E16;
  // load rows per step: 4, or 2 where G x EPL = 64 accumulators leave no room
  // for two 4-row buffers at two waves per SIMD
  static constexpr int NR = (G * EPL >= 64 && (sizeof(CT) >= 2 || G >= 16)) ? 2 : 4;
  // bf16 or e4m3 queries with G >= 8 q heads per kv head: the MFMA kernel
  static constexpr bool MF = sizeof(QT) <= 2 && G >= 8;
  static constexpr bool QF8 = sizeof(QT) == 1;
  // sh: the MFMA kernel's shared-load form (its own register budget)
  static const void* kernel(bool sh) {
    if constexpr (MF) {
      if (sh) return reinterpret_cast<const void*>(&mfma_row_kernel<CT, D, (MF ? G : 8), CAP, QF8, true>);
      return reinterpret_cast<const void*>(&mfma_row_kernel<CT, D, (MF ? G : 8), CAP, QF8, false>);
    } else {
      return reinterpret_cast<const void*>(&row_kernel<QT, CT, D, G, EPL, NR, CAP>);
    }
  }
  static int resident(bool sh) {
    static const int cap[2] = {resident_blocks(kernel(false), 64 * kWavesPerWG, 0),
                               resident_blocks(kernel(true), 64 * kWavesPerWG, 0)};
    return cap[MF && sh ? 1 : 0];
  }
};

template <typename QT, typename CT, int D, int G, bool CAP>
hipError_t launch_rows_t(const AttnParams& p, hipStream_t s) {
  using Cfg = RowCfg<QT, CT, D, G, CAP>;
  // the 4 waves of a workgroup share their K / V loads when they hold 4 heads
  // of one chunk and rows carry no lane padding
  const bool sh = row_shared_loads(p.Hkv, p.Dpad, D);
  // one wave per (chunk, kv head) for as many chunks as the planner may make
  const long long waves =
      (long long)row_chunks_max(Cfg::resident(sh) * kWavesPerWG, p.Hkv) * p.Hkv;
  dim3 grid((unsigned)((waves + kWavesPerWG - 1) / kWavesPerWG));
  if (trace_active()) {
    char nm[96];
    if constexpr (Cfg::MF)
      std::snprintf(nm, sizeof nm, "mfma_row_kernel<%s%s,D%d,G%d%s%s>", elem_name<CT>(),
                    Cfg::QF8 ? ",q_fp8" : "", D, G, CAP ? ",cap" : "",
                    sh ? ",shared_loads" : "");
    else
      std::snprintf(nm, sizeof nm, "row_kernel<%s,%s,D%d,G%d,EPL%d,NR%d%s>", elem_name<QT>(),
                    elem_name<CT>(), D, G, Cfg::EPL, Cfg::NR, CAP ? ",cap" : "");
    if (trace_launch(nm, grid.x, 64 * kWavesPerWG, 0, s)) return hipSuccess;
  }
  if constexpr (Cfg::MF) {
    if (sh) mfma_row_kernel<CT, D, (Cfg::MF ? G : 8), CAP, Cfg::QF8, true><<<grid, 64 * kWavesPerWG, 0, s>>>(p);
    else mfma_row_kernel<CT, D, (Cfg::MF ? G : 8), CAP, Cfg::QF8, false><<<grid, 64 * kWavesPerWG, 0, s>>>(p);
  }
  else row_kernel<QT, CT, D, G, Cfg::EPL, Cfg::NR, CAP><<<grid, 64 * kWavesPerWG, 0, s>>>(p);
  return hipGetLastError();
}

template <typename QT, typename CT, int D, bool CAP>
int row_waves_g(int G, bool sh) {
  switch (G) {
    case 1: return RowCfg<QT, CT, D, 1, CAP>::resident(sh) * kWavesPerWG;
    case 2: return RowCfg<QT, CT, D, 2, CAP>::resident(sh) * kWavesPerWG;
    case 4: return RowCfg<QT, CT, D, 4, CAP>::resident(sh) * kWavesPerWG;
    case 8: return RowCfg<QT, CT, D, 8, CAP>::resident(sh) * kWavesPerWG;
    case 16: return RowCfg<QT, CT, D, 16, CAP>::resident(sh) * kWavesPerWG;
    default: return 0;
  }
}

template <typename QT, typename CT, bool CAP>
int row_waves_d(int D, int G, bool sh) {
  if (D == 64) return row_waves_g<QT, CT, 64, CAP>(G, sh);
  if (D == 128) return row_waves_g<QT, CT, 128, CAP>(G, sh);
  return 0;
}

template <typename QT, typename CT, int D, bool CAP>
hipError_t launch_rows_g(const AttnParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_rows_t<QT, CT, D, 1, CAP>(p, s);
    case 2: return launch_rows_t<QT, CT, D, 2, CAP>(p, s);
    case 4: return launch_rows_t<QT, CT, D, 4, CAP>(p, s);
    case 8: return launch_rows_t<QT, CT, D, 8, CAP>(p, s);
    case 16: return launch_rows_t<QT, CT, D, 16, CAP>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename QT, typename CT, bool CAP>
hipError_t launch_rows_d(const AttnParams& p, hipStream_t s) {
  if (p.D == 64) return launch_rows_g<QT, CT, 64, CAP>(p, s);
  if (p.D == 128) return launch_rows_g<QT, CT, 128, CAP>(p, s);
  return hipErrorInvalidValue;
}

template <bool CAP>
int row_waves_c(rpa_dtype q_dt, rpa_dtype cache_dt, int D, int G, bool sh) {
  if (q_dt == RPA_F32 && cache_dt == RPA_F32) return row_waves_d<float, float, CAP>(D, G, sh);
  if (q_dt == RPA_BF16 && cache_dt == RPA_BF16) return row_waves_d<uint16_t, uint16_t, CAP>(D, G, sh);
  if (q_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) return row_waves_d<uint16_t, uint8_t, CAP>(D, G, sh);
  if (q_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) return row_waves_d<uint8_t, uint8_t, CAP>(D, G, sh);
  return 0;
}

template <bool CAP>
hipError_t launch_rows_c(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt, hipStream_t s) {
  if (q_dt == RPA_F32 && cache_dt == RPA_F32) return launch_rows_d<float, float, CAP>(p, s);
  if (q_dt == RPA_BF16 && cache_dt == RPA_BF16) return launch_rows_d<uint16_t, uint16_t, CAP>(p, s);
  if (q_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) return launch_rows_d<uint16_t, uint8_t, CAP>(p, s);
  if (q_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) return launch_rows_d<uint8_t, uint8_t, CAP>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

// The soft cap is a template choice of the row kernels, so that the per-logit
// code of the uncapped kernels carries no test of it.
int row_waves(rpa_dtype q_dt, rpa_dtype cache_dt, int D, int Dpad, int Hkv, int G, bool cap) {
  const bool sh = row_shared_loads(Hkv, Dpad, D);
  return cap ? row_waves_c<true>(q_dt, cache_dt, D, G, sh) : row_waves_c<false>(q_dt, cache_dt, D, G, sh);
}

hipError_t launch_rows(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt, hipStream_t s) {
  return p.cap > 0.f ? launch_rows_c<true>(p, q_dt, cache_dt, s)
                     : launch_rows_c<false>(p, q_dt, cache_dt, s);
}

namespace {
template <typename QT, int D>
hipError_t launch_merge_d(const AttnParams& p, dim3 grid, hipStream_t s) {
  if (trace_active()) {
    char nm[64];
    std::snprintf(nm, sizeof nm, "merge_kernel<%s,D%d,G%d>", elem_name<QT>(), D, p.Hq / p.Hkv);
    if (trace_launch(nm, grid.x, 256, 0, s)) return hipSuccess;
  }
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

#ifdef RPA_WAVE_TIMELINE
// The row kernels' per-wave stamps of the measurement build: n words of
// (start, first step, end, steps << 32 | XCC_ID << 16 | HW_ID) per wave.
extern "C" int rpa_timeline_read(unsigned long long* host, int n) {
  if (n > rpa::kTimelineWaves * 4) n = rpa::kTimelineWaves * 4;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(rpa::g_timeline),
                                  (size_t)n * sizeof(unsigned long long), 0, hipMemcpyDeviceToHost);
}
extern "C" int rpa_timeline_clear(void) {
  static unsigned long long zero[rpa::kTimelineWaves * 4];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(rpa::g_timeline), zero, sizeof(zero), 0,
                                hipMemcpyHostToDevice);
}
#endif
