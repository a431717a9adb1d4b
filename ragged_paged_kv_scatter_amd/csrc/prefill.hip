// Prefill / mixed-chunk kernel on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// One work unit = one (sequence, tile of up to 128 query tokens, q head);
// each of the workgroup's 4 waves owns 32 query rows.  The keys the tile can
// see are walked in 64-token blocks fetched from the paged cache through the
// block table into LDS (tpu-inference v3 kernel diff, "_fetch_bkv": per page,
// copy min(page_size, left) token rows), with the online softmax of
// "flash_attention_step1_qk_softmax" / "flash_attention_step2_pv".
//
// Operand layout (32x32x16 MFMA, lane l, kg = l / 32):
//   S^T = K Q^T   A = K block  [32 keys x 16 d]  lane: key l%32, d 8kg..8kg+7 (LDS b128)
//                 B = Q^T      [16 d x 32 rows]  lane: row l%32, d 8kg..8kg+7 (registers)
//   The accumulator gives lane l 16 keys of query row l%32, so row max / sum
//   need one exchange with lane l^32 only.
//   O^T += V^T P^T A = V^T [32 d x 16 keys] via two ds_read_b64_tr_b16 (4 keys each),
//                 B = P^T  [16 keys x 32 rows] = the S^T accumulator itself,
//   with the 16 keys of a k-step ordered as the S^T accumulator holds them:
//   k-slot k -> key ((k>>2)&1)*8 + (k>>3)*4 + (k&3).
//
// LDS rows are unpadded (D bf16) with the 16-byte chunks of row r stored at
// chunk ^ swz(r), which keeps both the K reads (16 rows, one chunk) and the
// transposed V reads (4 rows, four chunks per 32 lanes) free of bank conflicts.
// bf16 caches are copied global -> LDS directly (global_load_lds, no staging
// registers) into two stages, so the next block is in flight while the
// current one is multiplied; keys outside the tile's range are read from a
// zero row.  e4m3 caches are widened to bf16 (exactly) in registers on the
// way.  k_scale is folded into the logit scale and v_scale into 1/l.
#include <math.h>

#include <algorithm>
#include <climits>
#include <cstdio>

#include <type_traits>

#include "device_common.h"
#include "merge.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

// Per-wave shader-clock counts of the prefill kernel, compiled only into the
// measurement build (RPA_WAVE_TIMELINE, librpa_timeline.so).  For wave w,
// kPfWords words: its clocks from start to end; clocks spent waiting for its
// own block copies at the top of each pipeline step, and at the step's
// barrier after that; its step count; then, summed over the steps that do
// math, the clocks from the barrier to the first q.k MFMA (copy issue and
// rescale), of the q.k part, of the p.v part, and of the row max / sum tail.
// Stamps are read back only after the next step's barrier, where the wave
// waits for its outstanding LDS and scalar loads anyway.  The library never
// reads them.
#ifdef RPA_WAVE_TIMELINE
constexpr int kPfTimelineWaves = 8192;
constexpr int kPfWords = 8;
__device__ unsigned long long g_pf_timeline[kPfTimelineWaves * kPfWords];
#define RPA_TL_PF_BEGIN()                                                   \
  const unsigned long long tlp_t0 = __builtin_amdgcn_s_memtime();           \
  unsigned long long tlp_vm = 0, tlp_bar = 0;                               \
  unsigned long long tlp_ph[4] = {0, 0, 0, 0};                              \
  unsigned long long tlp_s[5] = {0, 0, 0, 0, 0};                            \
  int tlp_steps = 0
#define RPA_TL_PF_MARK(v) const unsigned long long v = __builtin_amdgcn_s_memtime()
#define RPA_TL_PF_FOLD()                                                    \
  do {                                                                      \
    if (tlp_s[4] != 0) {                                                    \
      for (int i_ = 0; i_ < 4; ++i_) tlp_ph[i_] += tlp_s[i_ + 1] - tlp_s[i_]; \
      tlp_s[4] = 0;                                                         \
    }                                                                       \
  } while (0)
#define RPA_TL_PF_WAITS(a, b)                                               \
  do {                                                                      \
    const unsigned long long c_ = __builtin_amdgcn_s_memtime();             \
    RPA_TL_PF_FOLD();                                                       \
    tlp_vm += (b) - (a);                                                    \
    tlp_bar += c_ - (b);                                                    \
    ++tlp_steps;                                                            \
    tlp_s[0] = c_;                                                          \
  } while (0)
#define RPA_TL_PF_AT(i) tlp_s[i] = __builtin_amdgcn_s_memtime()
#define RPA_TL_PF_END()                                                     \
  do {                                                                      \
    const unsigned long long t_ = __builtin_amdgcn_s_memtime();             \
    RPA_TL_PF_FOLD();                                                       \
    const long long w_ = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); \
    if ((threadIdx.x & 63) == 0 && w_ < kPfTimelineWaves) {                 \
      unsigned long long* r_ = g_pf_timeline + w_ * kPfWords;               \
      r_[0] = t_ - tlp_t0;                                                  \
      r_[1] = tlp_vm;                                                       \
      r_[2] = tlp_bar;                                                      \
      r_[3] = (unsigned long long)tlp_steps;                                \
      for (int i_ = 0; i_ < 4; ++i_) r_[4 + i_] = tlp_ph[i_];               \
    }                                                                       \
  } while (0)
// The two-group kernel's laps: per wave, clocks in each part of its steps,
// read at once (each lap waits for its own stamp).
__device__ unsigned long long g_pp_timeline[kPfTimelineWaves * kPfWords];
#define RPA_TL_PP_BEGIN()                                                   \
  unsigned long long tlq_last = __builtin_amdgcn_s_memtime();               \
  const unsigned long long tlq_t0 = tlq_last;                               \
  unsigned long long tlq_acc[6] = {0, 0, 0, 0, 0, 0};                       \
  int tlq_steps = 0
#define RPA_TL_PP_LAP(i)                                                    \
  do {                                                                      \
    const unsigned long long t_ = __builtin_amdgcn_s_memtime();             \
    tlq_acc[i] += t_ - tlq_last;                                            \
    tlq_last = t_;                                                          \
  } while (0)
#define RPA_TL_PP_STEP() ++tlq_steps
#define RPA_TL_PP_END()                                                     \
  do {                                                                      \
    const unsigned long long t_ = __builtin_amdgcn_s_memtime();             \
    const long long w_ = (long long)blockIdx.x * (2 * NT / 64) + (threadIdx.x >> 6); \
    if ((threadIdx.x & 63) == 0 && w_ < kPfTimelineWaves) {                 \
      unsigned long long* r_ = g_pp_timeline + w_ * kPfWords;               \
      r_[0] = t_ - tlq_t0;                                                  \
      r_[1] = (unsigned long long)tlq_steps;                                \
      for (int i_ = 0; i_ < 6; ++i_) r_[2 + i_] = tlq_acc[i_];              \
    }                                                                       \
  } while (0)
#else
#define RPA_TL_PP_BEGIN() static_assert(true, "")
#define RPA_TL_PP_LAP(i) static_assert(true, "")
#define RPA_TL_PP_STEP() static_assert(true, "")
#define RPA_TL_PP_END() static_assert(true, "")
#define RPA_TL_PF_BEGIN() static_assert(true, "")
#define RPA_TL_PF_MARK(v) static_assert(true, "")
#define RPA_TL_PF_WAITS(a, b) static_assert(true, "")
#define RPA_TL_PF_AT(i) static_assert(true, "")
#define RPA_TL_PF_END() static_assert(true, "")
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int BK = 64;          // keys per block
constexpr int NT = 256;         // threads per workgroup
constexpr int kPT = 512;        // page ids cached in LDS per refill
constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kPrefillGrid = 1024;  // fallback persistent grid (multiple of 8)
constexpr int kPairPages = 8192;           // page ids the two-group kernel holds in LDS

template <typename CT> struct CacheElem;
template <> struct CacheElem<uint16_t> { static constexpr int size = 2; };
template <> struct CacheElem<uint8_t> { static constexpr int size = 1; };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// two floats -> two bf16 (RNE) in one word: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// two e4m3 codes (bytes 0/1, or 2/3 with HI) -> two bf16 packed in one word
// (exact: the scaled convert with scale 1 widens every code pair exactly)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, HI));
}

// Physical 16-byte chunk of logical chunk c in LDS row r.
// Chunk swizzle of LDS row r (LDS serves 256 bytes per cycle: 16 lanes of a
// ds_read_b128, 32 lanes of a ds_read_b64_tr_b16).
//  D = 128 (16 chunks, one row per 256 B): f(r) is a bijection on r mod 16, so
//    16 consecutive rows at one logical chunk hit 16 distinct chunks (K
//    reads); bits 2-3 of f are r & 3, so 4 consecutive rows x chunks
//    4dt..4dt+3 hit 16 distinct chunks (transposed V reads).
//  D = 64 (8 chunks, two rows per 256 B): rows of equal parity in a 16-row
//    window get distinct f; rows r, r + 2 differ in bit 2 of f.
// Rows r and r + 8 always differ by f ^ 2.
template <int D>
__device__ __forceinline__ int swz_f(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  return c ^ swz_f<D>(r);
}

// Chunk swizzle of an e4m3 K row (D bytes) in LDS, for the fp8-query kernel:
// the 16 rows a ds_read_b128 serves at one logical chunk land on 16 distinct
// 16-byte bank groups.  D = 128: two rows per 256 B, f(r) = (r >> 1) & 7
// spreads the 8 rows of one parity; D = 64: four rows per 256 B,
// f(r) = (r >> 2) & 3 spreads the 4 rows of one residue.
template <int D>
__device__ __forceinline__ int swz8_f(int r) {
  if constexpr (D == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0) (gfx9 encoding), leaving expcnt / lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// 16 bytes per lane global -> LDS at lds_base + 16 * lane (global_load_lds_dwordx4),
// from a per-lane 64-bit address.  Issued from asm so that the compiler does
// not serialise the LDS reads of the other buffers behind these loads; the
// kernel orders them itself with wait_vmem_all() + a barrier before a buffer
// is read.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_base)
               : "memory", "m0");
}

// The same from a wave-uniform base (SGPR pair) plus a per-lane 32-bit offset.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// A wave-uniform pointer, forced into an SGPR pair.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p));
}

// CAP: logits soft cap on (p.cap > 0), chosen at launch so that the
// per-logit code has no branch on it.
//
// Block pipeline (per workgroup, blocks b = 64 keys): K is fetched one block
// ahead of V, into two K buffers and two V buffers by block parity.  Step b
//   - waits for K(b+1) and V(b), then starts K(b+2) and V(b+1);
//   - exponentiates the logits of block b (computed in step b-1) while the
//     MFMAs of S(b+1) = K(b+1) Q^T run;
//   - multiplies P(b) V(b) while the row max of S(b+1) is formed.
// So MFMA and VALU work of one wave overlap, and every buffer is rewritten
// only after the barrier that follows its last reader.
//
// QF8 (e4m3 queries over an e4m3 cache): S^T = K Q^T runs on
// v_mfma_f32_32x32x64_f8f6f4 with the cached K codes copied global -> LDS as
// they are (no widening), and Q codes in registers; its 32x32 accumulator
// has the layout of the bf16 one, so the softmax and the bf16 O^T += V^T P^T
// steps are shared.  The fp8 A and B operands hold, in lane group kg of
// k-step s, the 32 bytes d = 64 s + 32 kg .. + 31 of their K row / Q row in
// the same order, so every product pairs the same d.
template <typename CT, int D, bool CAP, bool QF8>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(AttnParams p) {
  static_assert(!QF8 || sizeof(CT) == 1, "e4m3 queries go with an e4m3 cache");
  RPA_TL_PF_BEGIN();
  constexpr bool VDIRECT = sizeof(CT) == 2;        // bf16 cache: V global -> LDS directly
  constexpr bool KDIRECT = VDIRECT || QF8;         // K rows copied as stored
  constexpr int RB = D * 2;                        // LDS row bytes of V (and of bf16 K)
  constexpr int RBK = QF8 ? D : RB;                // LDS row bytes of K
  constexpr int CPR = RB / 16;                     // 16-byte LDS chunks per V row
  constexpr int CPRK = RBK / 16;                   // 16-byte LDS chunks per K row
  constexpr int BLKB = BK * RB;                    // bytes of one V block
  constexpr int BLKBK = BK * RBK;                  // bytes of one K block
  constexpr int KS = D / 16;                       // bf16 MFMA k-steps of q.k
  constexpr int KS8 = D / 64;                      // fp8 MFMA k-steps of q.k
  constexpr int DT = D / 32;                       // 32-row d tiles of O^T
  constexpr int IPW = BLKB / 1024 / 4;             // direct loads per wave per V block
  constexpr int RPI = 1024 / RB;                   // V rows per direct load instruction
  constexpr int IPWK = BLKBK / 1024 / 4;           // direct loads per wave per K block
  constexpr int RPIK = 1024 / RBK;                 // K rows per direct load instruction
  constexpr int ESZ = CacheElem<CT>::size;
  constexpr int GCPR = D * ESZ / 16;               // 16-byte chunks of a cached head row
  constexpr int PER = BK * GCPR / NT;              // staged chunks per thread (e4m3 path)
  static_assert(!VDIRECT || IPW * RPI == 16, "a wave loads 16 consecutive rows");
  static_assert(!KDIRECT || IPWK * RPIK == 16, "a wave loads 16 consecutive rows");
  static_assert(VDIRECT || (PER >= 1 && BK * GCPR % NT == 0), "staged split");
  __shared__ __attribute__((aligned(1024))) char s_k[2 * BLKBK];
  __shared__ __attribute__((aligned(1024))) char s_v[2 * BLKB];
  __shared__ int s_pt[kPT];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const PrefillItem* items = reinterpret_cast<const PrefillItem*>(p.ws + p.lay.pf_items);
  const char* zero_row = reinterpret_cast<const char*>(p.ws + p.lay.zeros);
  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const long long n_units = (long long)hdr->n_pf_items * Hq;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 5, col = lane & 31;
  const int sh = p.ps_shift;                       // page_size = 1 << sh (>= 16)
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * (uint32_t)ESZ;  // one cache token row
  const uint32_t v_bytes = (uint32_t)p.Dpad * ESZ;               // K row -> V row
  // Logits are masked before they are scaled (see logit() and expo()), which
  // needs a positive scale: a masked -inf times 0 is NaN and times a negative
  // scale turns into +inf.  The logit q.k * scale is therefore formed as
  // (sign(scale) q).k * |scale|: a negative scale flips the sign bits of the
  // bf16 q (exact), and a zero scale zeroes q and keeps a scale of 1, so every
  // visible logit is exactly 0, as the definition gives.
  const bool q_zero = p.qk_scale == 0.f;
  const uint32_t q_and = q_zero ? 0u : 0xFFFFFFFFu;
  const uint32_t q_xor = p.qk_scale < 0.f ? (QF8 ? 0x80808080u : 0x80008000u) : 0u;
  const float scale_pos = q_zero ? 1.f : fabsf(p.qk_scale);
  const float c_scale = CAP ? scale_pos : scale_pos * kLog2e;
  const float c_eff = CAP ? 1.f : c_scale;       // stored logits -> log2 units
  const float cap_k = CAP ? c_scale * 2.f * kLog2e / p.cap : 0.f;
  const float cap_l2 = CAP ? p.cap * kLog2e : 0.f;
  // With a soft cap, a block keeps r = 1 / (2^a + 1) per logit, with
  // a = q.k * cap_k = 2 x log2 e for x = q.k * scale / cap, instead of the
  // capped logit
  // cap log2 e tanh(x) = cap_l2 (1 - 2 r): the row max becomes a min over r
  // (a masked logit is r = +inf) and p = 2^(cap_l2 (1 - 2 r) - m) is one fma
  // and one exp2.
  constexpr float kRedInit = CAP ? INFINITY : -INFINITY;
  auto red = [](float a, float b) { return CAP ? fminf(a, b) : fmaxf(a, b); };
  // reduced block value -> row max in log2 units
  auto to_mx = [&](float v) { return CAP ? fmaf(v, -2.f * cap_l2, cap_l2) : v * c_eff; };

  // Direct loads: instruction j of a wave writes LDS rows 16 wave + RPI j +
  // lane / CPR, physical chunk lane % CPR, which holds logical chunk
  // (lane % CPR) ^ swz(row); the rows' source offsets from the wave's first
  // token row are fixed per lane.
  // Physical chunk -> logical chunk of LDS row r: K (e4m3 rows when QF8) or V.
  auto kchunk = [](int r, int c) { return QF8 ? (c ^ swz8_f<D>(r)) : swz_chunk<D>(r, c); };
  uint32_t dma_off[VDIRECT ? IPW : 1], dma_off_k[KDIRECT ? IPWK : 1];
#pragma unroll
  for (int j = 0; j < (VDIRECT ? IPW : 1); ++j) {
    const int r = RPI * j + lane / CPR;
    dma_off[j] = r * row_bytes + (swz_chunk<D>(r, lane % CPR) << 4);
  }
#pragma unroll
  for (int j = 0; j < (KDIRECT ? IPWK : 1); ++j) {
    const int r = RPIK * j + lane / CPRK;
    dma_off_k[j] = r * row_bytes + (kchunk(r, lane % CPRK) << 4);
  }
  // Fused update: the same rows read from the new keys / values, whose token
  // rows are in_row_bytes apart.
  const bool fused = p.fuse_update != 0;
  const uint32_t in_row = p.in_row_bytes;
  uint32_t dma_in[VDIRECT ? IPW : 1], dma_in_k[KDIRECT ? IPWK : 1];
#pragma unroll
  for (int j = 0; j < (VDIRECT ? IPW : 1); ++j) {
    const int r = RPI * j + lane / CPR;
    dma_in[j] = r * in_row + (swz_chunk<D>(r, lane % CPR) << 4);
  }
#pragma unroll
  for (int j = 0; j < (KDIRECT ? IPWK : 1); ++j) {
    const int r = RPIK * j + lane / CPRK;
    dma_in_k[j] = r * in_row + (kchunk(r, lane % CPRK) << 4);
  }

  // LDS byte offsets inside a K / V buffer (fixed per lane):
  //  K read (half hf, k-step ks): row hf*32 + col, logical chunk 2ks + kg,
  //    offset = (k_off ^ (ks << 5)) + hf * 32 * RB  (swz_f depends on row mod 16)
  //  V^T reads (k-step ks, d tile dt): rows 16ks + rr and 16ks + rr + 8,
  //    offsets = (v_off1 ^ (dt << 6)) + ks * 16 * RB and (v_off2 ^ (dt << 6)) + (16ks + 8) * RB
  const int fk = swz_f<D>(col);
  const uint32_t k_off = col * RB + ((((fk >> 1) << 1) | (kg ^ (fk & 1))) << 4);
  const int grp = lane >> 4, r16 = lane & 15;
  const int rr = (grp >> 1) * 4 + (r16 >> 2);
  const int g1 = (2 * (grp & 1) + ((r16 & 3) >> 1)) ^ swz_f<D>(rr);
  const uint32_t v_off1 = rr * RB + (g1 << 4) + (r16 & 1) * 8;
  const uint32_t v_off2 = v_off1 ^ 32u;  // row rr + 8: chunk ^ 2

  auto ld_k = [&](const char* kb, int ks, int hf) -> bf16x8 {
    const char* a = kb + ((k_off ^ (uint32_t)(ks << 5)) + hf * 32 * RB);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a));
  };
  // fp8 A operand (QF8): key row hf * 32 + col, bytes 64 ks + 32 kg .. + 31,
  // i.e. logical chunks 4 ks + 2 kg and 4 ks + 2 kg + 1 of the e4m3 row
  const int f8 = swz8_f<D>(col);
  auto ld_k8 = [&](const char* kb, int ks, int hf) -> i32x8 {
    const char* row = kb + (hf * 32 + col) * RBK;
    const int c0 = 4 * ks + 2 * kg;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + ((c0 ^ f8) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (((c0 + 1) ^ f8) << 4));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                 (int)hi.w};
  };
  // S^T accumulation step of one 32-key half: bf16 (16 d) or e4m3 (64 d)
  auto mfma_qk8 = [](i32x8 a, i32x8 b, f32x16 c) -> f32x16 {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  };
  auto ld_vt = [&](const char* vb, int ks, int dt) -> bf16x8 {
    const char* a1 = vb + ((v_off1 ^ (uint32_t)(dt << 6)) + ks * 16 * RB);
    const char* a2 = vb + ((v_off2 ^ (uint32_t)(dt << 6)) + (ks * 16 + 8) * RB);
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a1));
    const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a2));
    const i16x8 av = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
    return __builtin_bit_cast(bf16x8, av);
  };

  // Split-KV partials of the row kernel (launched before this one), by (row,
  // kv head); they touch rows this kernel does not write.  Rows with many
  // parts are merged by the whole workgroup in s_k, before any copy into it.
  static_assert(NT == 256, "the workgroup merge takes 4 waves");
  static_assert(merge_wg_floats<D, 16>() * 4 <= 2 * BLKB, "merge scratch fits in s_v");
  if (p.fuse_merge)
    merge_all_g<uint16_t, D>(p, (long long)hdr->n_merge_rows * Hkv, reinterpret_cast<float*>(s_v));

  // Persistent grid: in round k block b takes unit k * grid + b, except that
  // odd rounds reverse the order of the groups of 8 blocks (when the grid is
  // a multiple of 8).  Units come heavy first (causal tiles late in a
  // sequence see more keys), so the reversal evens out the blocks' sums of
  // work; units keep u mod 8 = b mod 8, so consecutive units sit on different
  // XCDs and the head slot -> (kv head = slot mod Hkv) mapping keeps the q
  // heads of one kv head on one XCD and L2.  Once a round's unit is past the
  // end, every later round's is too.
  //
  // When the planner runs this kernel beside the row kernel (co_run), only
  // the first (8 - kCoRowEighths) / 8 of the grid (a multiple of 8) takes
  // units, leaving the other slots of the CUs to the row kernel's waves.
  if (p.pf_pair && !hdr->co_run) return;           // the two-group kernel has the batch
  unsigned grid = gridDim.x;
  if (hdr->co_run && grid >= 64) grid = grid / 64 * (8 - kCoRowEighths) * 8;
  const bool co_pf = hdr->co_run != 0;
  if (blockIdx.x >= grid) return;
  const bool snake = (grid & 7) == 0;
  for (long long k = 0;; ++k) {
    const long long b = (snake && (k & 1)) ? (long long)(grid / 8 - 1 - blockIdx.x / 8) * 8 +
                                                 (blockIdx.x & 7)
                                           : (long long)blockIdx.x;
    const long long u = k * grid + b;
    if (u >= n_units) break;
    const int item_i = (int)(u / Hq);
    const int hh = (int)(u - (long long)item_i * Hq);
    const int g = hh % Hkv;
    const int h = g * G + hh / Hkv;
    const PrefillItem it = items[item_i];
    const int seq = it.seq;
    const int q0 = p.qsl[seq];
    const int q_len = p.qsl[seq + 1] - q0;
    const int ctx = p.kv_lens[seq] - q_len;
    const int W = p.window;
    const int kv_lo = W > 0 ? max(0, ctx + it.q_begin - W + 1) : 0;
    const int kv_hi = ctx + it.q_end;               // exclusive
    const int* bt = p.block_tables + (long long)seq * p.pps;
    const char* kv_head = static_cast<const char*>(p.cache) + 2LL * g * p.Dpad * ESZ;
    // Fused update: new tokens (positions >= ctx) come from the call's new K
    // / V rows (row q0 + pos - ctx), and the unit of the first q head of kv
    // head g writes its own tile's new tokens (positions ctx + q_begin ..
    // ctx + q_end - 1) into their cache slots.
    const char* in_k = fused ? static_cast<const char*>(p.new_k) + (long long)g * D * ESZ : nullptr;
    const char* in_v = fused ? static_cast<const char*>(p.new_v) + (long long)g * D * ESZ : nullptr;
    const int new_lo = fused ? ctx : INT_MAX;       // first key read from the new rows
    const bool writer = fused && hh < Hkv;
    const int own_lo = ctx + it.q_begin, own_hi = ctx + it.q_end;
    char* cache_w = const_cast<char*>(kv_head);

    const int row_q = it.q_begin + wave * 32 + col;  // this lane's query row (within the seq)
    const bool row_ok = row_q < it.q_end;
    const int pos = ctx + row_q;
    const bool wave_live = it.q_begin + wave * 32 < it.q_end;

    const int blk_first = kv_lo / BK;
    const int blk_end = (kv_hi + BK - 1) / BK;
    // Blocks [f_lo, f_hi) are visible in full to every row of the tile
    // (causal: last key <= first row's position; window: first key within W
    // of the last row's position); every other block is masked per logit.
    const int tpos_lo = ctx + it.q_begin, tpos_hi = kv_hi - 1;
    int f_lo = blk_first;
    if (W > 0 && tpos_hi - W >= 0) f_lo = max(f_lo, (tpos_hi - W) / BK + 1);
    f_lo = min(f_lo, blk_end);
    const int f_hi = min(max((tpos_lo + 1) / BK, f_lo), blk_end);
    // step b needs the mask for block b + 1: unmasked steps are [A, B)
    const int A = min(max(blk_first, f_lo - 1), blk_end);
    const int B = max(A, f_hi - 1);

    // page ids of the unit's key range, kPT at a time, in LDS
    int pt_base = -(1 << 30);
    auto ensure_pages = [&](int blk) {       // uniform: make the table cover block blk
      const int need_hi = (min(blk * BK + BK, kv_hi) - 1) >> sh;
      if (need_hi >= pt_base + kPT || (max(blk * BK, kv_lo) >> sh) < pt_base) {
        const int first_page = max(blk * BK, kv_lo) >> sh;
        const int last_page = (kv_hi - 1) >> sh;
        __syncthreads();                    // nobody still reads the old table
        for (int i = tid; i < kPT; i += NT) {
          const int pg = first_page + i;
          s_pt[i] = pg <= last_page ? bt[pg] : 0;
        }
        pt_base = first_page;
        __syncthreads();
      }
    };

    // ---- loads of one K or V block (vofs = 0: K rows, v_bytes: V rows) ----
    // ISK: K rows (RBK bytes in LDS), else V rows (RB bytes)
    auto issue_direct = [&](auto isk, int blk, char* buf, uint32_t vofs)
                            __attribute__((always_inline)) {
      constexpr bool K_ = decltype(isk)::value;
      constexpr int IPW_ = K_ ? IPWK : IPW, RPI_ = K_ ? RPIK : RPI, CPR_ = K_ ? CPRK : CPR;
      const int t0 = blk * BK + 16 * wave;           // the wave's first token
      const uint32_t lds0 = lds_addr(buf + wave * IPW_ * 1024);
      const char* in_base = K_ ? in_k : in_v;
      if (t0 >= kv_lo && t0 + 16 <= min(kv_hi, new_lo)) {
        // 16 cached tokens of one page (page_size >= 16): uniform base + lane offsets
        const int page = __builtin_amdgcn_readfirstlane(s_pt[(t0 >> sh) - pt_base]);
        const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(t0 & pmask);
        const char* base = uniform_ptr(kv_head + vofs + (uint64_t)crow * row_bytes);
#pragma unroll
        for (int j = 0; j < IPW_; ++j) dma16_s(base, K_ ? dma_off_k[j] : dma_off[j], lds0 + j * 1024);
      } else if (t0 >= max(kv_lo, new_lo) && t0 + 16 <= kv_hi) {
        // 16 new tokens: consecutive rows of the call's new K / V
        const char* base = uniform_ptr(in_base + (uint64_t)(q0 + t0 - ctx) * in_row);
#pragma unroll
        for (int j = 0; j < IPW_; ++j) dma16_s(base, K_ ? dma_in_k[j] : dma_in[j], lds0 + j * 1024);
      } else {
        // range edge: rows outside [kv_lo, kv_hi) come from the zero row
#pragma unroll
        for (int j = 0; j < IPW_; ++j) {
          const int r = RPI_ * j + lane / CPR_;
          const int tok = t0 + r;
          const int lc = K_ ? kchunk(r, lane % CPR_) : swz_chunk<D>(r, lane % CPR_);
          const char* src = zero_row + (lc << 4);
          if (tok >= kv_lo && tok < kv_hi) {
            if (tok >= new_lo) {
              src = in_base + (uint64_t)(q0 + tok - ctx) * in_row + (lc << 4);
            } else {
              const int page = s_pt[(tok >> sh) - pt_base];
              const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
              src = kv_head + vofs + (uint64_t)crow * row_bytes + (lc << 4);
            }
          }
          dma16(src, lds0 + j * 1024);
        }
      }
    };
    uint4 kr[KDIRECT ? 1 : PER], vr[VDIRECT ? 1 : PER];
    auto fetch_staged = [&](int blk, uint4* regs, uint32_t vofs) {   // e4m3: global -> registers
#pragma unroll
      for (int i = 0; i < (VDIRECT ? 0 : PER); ++i) {
        const int cidx = tid + NT * i;
        const int tok = blk * BK + cidx / GCPR, cc = cidx % GCPR;
        uint4 a = make_uint4(0, 0, 0, 0);
        if (tok >= kv_lo && tok < kv_hi) {
          if (tok >= new_lo) {
            const char* in_base = vofs ? in_v : in_k;
            a = *reinterpret_cast<const uint4*>(in_base + (uint64_t)(q0 + tok - ctx) * in_row + cc * 16);
          } else {
            const int page = s_pt[(tok >> sh) - pt_base];
            const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
            a = *reinterpret_cast<const uint4*>(kv_head + vofs + (uint64_t)crow * row_bytes + cc * 16);
          }
        }
        regs[i] = a;
      }
    };
    // The cache slot of key position tok (its K row; + v_bytes for V).  The
    // page id comes from the LDS table when the caller has checked that the
    // table holds it (a global read would make the writer wait for every
    // copy it has in flight).
    auto slot_row = [&](int tok, bool in_pt) -> char* {
      const int page = in_pt ? s_pt[(tok >> sh) - pt_base] : bt[tok >> sh];
      return cache_w + (uint64_t)(((uint32_t)page << sh) | (uint32_t)(tok & pmask)) * row_bytes;
    };
    // whether the LDS table holds the pages of key positions [lo, hi) (uniform)
    auto pt_holds = [&](int lo, int hi) {
      return (lo >> sh) >= pt_base && ((hi - 1) >> sh) < pt_base + kPT;
    };
    // Fused update, staged rows: the writer stores the codes of its own new
    // tokens (rows of block blk) as they were fetched, and zeroes pad lanes.
    auto write_staged = [&](const uint4* regs, int blk, uint32_t vofs) {
      if (!writer) return;
      const int lo = max(blk * BK, own_lo), hi = min(blk * BK + BK, own_hi);
      if (lo >= hi) return;
      const bool in_pt = pt_holds(lo, hi);
#pragma unroll
      for (int i = 0; i < (VDIRECT ? 0 : PER); ++i) {
        const int cidx = tid + NT * i;
        const int tok = blk * BK + cidx / GCPR, cc = cidx % GCPR;
        if (tok >= lo && tok < hi) {
          char* dst = slot_row(tok, in_pt) + vofs;
          *reinterpret_cast<uint4*>(dst + cc * 16) = regs[i];
          if (cc == 0)
            for (int pc = GCPR; pc < (int)(p.Dpad * ESZ / 16); ++pc)
              *reinterpret_cast<uint4*>(dst + pc * 16) = make_uint4(0, 0, 0, 0);
        }
      }
    };
    // Fused update, rows copied into LDS as stored (bf16 K and V, e4m3 K of
    // the fp8-query kernel): the writer stores its own new tokens of block
    // blk from the LDS buffer, pad lanes zeroed.
    auto write_lds = [&](auto isk, int blk, const char* buf) __attribute__((always_inline)) {
      constexpr bool K_ = decltype(isk)::value;
      constexpr int RB_ = K_ ? RBK : RB;
      constexpr int DCH = (K_ ? RBK : RB) / 16;        // chunks holding data
      if (!writer) return;
      const int lo = max(blk * BK, own_lo), hi = min(blk * BK + BK, own_hi);
      if (lo >= hi) return;
      const int wch = p.Dpad * ESZ / 16;               // chunks of a cache head row
      const int n = (hi - lo) * wch;
      const bool in_pt = pt_holds(lo, hi);
      for (int i = tid; i < n; i += NT) {
        const int rr = i / wch, c = i - rr * wch;
        const int tok = lo + rr, r = tok - blk * BK;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < DCH) {
          const int pc = K_ ? kchunk(r, c) : swz_chunk<D>(r, c);
          v = *reinterpret_cast<const uint4*>(buf + r * RB_ + (pc << 4));
        }
        *reinterpret_cast<uint4*>(slot_row(tok, in_pt) + (K_ ? 0u : v_bytes) + c * 16) = v;
      }
    };
    auto stage_staged = [&](const uint4* regs, char* buf) {  // e4m3 -> bf16 into swizzled rows
#pragma unroll
      for (int i = 0; i < (VDIRECT ? 0 : PER); ++i) {
        const int cidx = tid + NT * i;
        const int row = cidx / GCPR, cc = cidx % GCPR;
        const uint32_t w[4] = {regs[i].x, regs[i].y, regs[i].z, regs[i].w};
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = fp8x2_to_bf16x2<false>(w[e]);
          o[2 * e + 1] = fp8x2_to_bf16x2<true>(w[e]);
        }
        char* rb = buf + row * RB;
        *reinterpret_cast<uint4*>(rb + (swz_chunk<D>(row, 2 * cc) << 4)) =
            make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(rb + (swz_chunk<D>(row, 2 * cc + 1) << 4)) =
            make_uint4(o[4], o[5], o[6], o[7]);
      }
    };
    auto kbuf = [&](int blk) -> char* { return s_k + (blk & 1) * BLKBK; };
    auto vbuf = [&](int blk) -> char* { return s_v + (blk & 1) * BLKB; };
    auto load_k = [&](int blk) {
      if constexpr (KDIRECT) issue_direct(std::true_type{}, blk, kbuf(blk), 0);
      else fetch_staged(blk, kr, 0);
    };
    auto load_v = [&](int blk) {
      if constexpr (VDIRECT) issue_direct(std::false_type{}, blk, vbuf(blk), v_bytes);
      else fetch_staged(blk, vr, v_bytes);
    };
    // step b, first part: K(b+1), V(b) are in LDS; start K(b+2), V(b+1)
    auto begin_step = [&](int blk) __attribute__((always_inline)) {
      RPA_TL_PF_MARK(tlp_a);
      if constexpr (KDIRECT) wait_vmem_all();     // this wave's loads have landed
      RPA_TL_PF_MARK(tlp_b);
      __syncthreads();                            // everyone's; last readers are done
      RPA_TL_PF_WAITS(tlp_a, tlp_b);
      if (blk + 1 < blk_end) load_v(blk + 1);     // its pages are in the table already
      if (blk + 2 < blk_end) {
        ensure_pages(blk + 2);
        load_k(blk + 2);
      }
      // fused update: K(blk + 1) and V(blk) stay in LDS through this step
      if constexpr (KDIRECT) {
        if (blk + 1 < blk_end) write_lds(std::true_type{}, blk + 1, kbuf(blk + 1));
      }
      if constexpr (VDIRECT) write_lds(std::false_type{}, blk, vbuf(blk));
    };
    // step b, last part (e4m3): widen the fetched rows into their buffers
    auto end_step = [&](int blk) __attribute__((always_inline)) {
      if constexpr (!VDIRECT) {
        if (blk + 1 < blk_end) {
          stage_staged(vr, vbuf(blk + 1));
          write_staged(vr, blk + 1, v_bytes);
        }
      }
      if constexpr (!KDIRECT) {
        if (blk + 2 < blk_end) {
          stage_staged(kr, kbuf(blk + 2));
          write_staged(kr, blk + 2, 0);
        }
      }
    };

    // ---- per-lane state: Q^T operand, O^T accumulators, softmax state ----
    bf16x8 qreg[QF8 ? 1 : KS];   // 8 bf16 of row row_q, d = 16 ks + 8 kg .. +7
    i32x8 qreg8[QF8 ? KS8 : 1];   // QF8: 32 e4m3 of row row_q, d = 64 ks + 32 kg .. +31
    {
      const long long qrow = (long long)(q0 + (row_ok ? row_q : it.q_begin)) * Hq + h;
      auto fix = [&](uint4 v) {
        return make_uint4((v.x & q_and) ^ q_xor, (v.y & q_and) ^ q_xor, (v.z & q_and) ^ q_xor,
                          (v.w & q_and) ^ q_xor);
      };
      if constexpr (QF8) {
        const uint8_t* qp = static_cast<const uint8_t*>(p.q) + qrow * D + 32 * kg;
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks) {
          const uint4 z = make_uint4(0, 0, 0, 0);
          const uint4 lo = fix(row_ok ? *reinterpret_cast<const uint4*>(qp + 64 * ks) : z);
          const uint4 hi = fix(row_ok ? *reinterpret_cast<const uint4*>(qp + 64 * ks + 16) : z);
          qreg8[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y,
                            (int)hi.z, (int)hi.w};
        }
      } else {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + qrow * D + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 v = fix(row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks)
                                     : make_uint4(0, 0, 0, 0));
          qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
      }
    }
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    // S^T of a block (lane: 16 keys x its row), alternating between sa and sb
    // so that the steps of a pair name their buffers statically
    f32x16 sa[2], sb[2];
    float mx = -INFINITY;    // row max of the current block, log2 units

    // logit e (0..31) of the block starting at key k0: key
    // k0 + 32 (e >> 4) + 8 ((e & 15) >> 2) + 4 kg + (e & 3)
    auto logit = [&](auto masked, int k0, float s, int e) __attribute__((always_inline)) -> float {
      if constexpr (CAP) {
        // tanh(x) = 1 - 2 r with r = 1 / (e^{2x} + 1)
        s = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s * cap_k) + 1.f);
      }
      if constexpr (decltype(masked)::value) {
        // key j = k0 + 4 kg + ko with ko a constant: visible iff
        // j <= pos and (no window or j > pos - W)
        const int ko = (e >> 4) * 32 + ((e & 15) >> 2) * 8 + (e & 3);
        const int lim = pos - k0 - 4 * kg;
        const bool vis = ko <= lim && (W <= 0 || ko > lim - W);
        s = vis ? s : kRedInit;
      }
      return s;
    };

    // One pipeline step on block blk (see above): sacc holds S(blk), s2
    // receives S(blk + 1).  MASK_NEXT: block blk + 1 needs per-logit masking.
    auto step = [&](auto mask_next, int blk, f32x16(&sacc)[2], f32x16(&s2)[2])
                    __attribute__((always_inline)) {
      constexpr bool MASK_NEXT = decltype(mask_next)::value;
      begin_step(blk);
      // Lazy rescaling: the running max only moves (and acc / l are only
      // rescaled) when some row of the wave grows by more than 2^8; until
      // then p <= 2^8, harmless in fp32 sums and in bf16.
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float c_bias = cap_l2 - m_use;                 // cap path: p = 2^(c_bias - 2 cap_l2 r)
      const char* kn = kbuf(blk + 1);
      const char* vb = vbuf(blk);
      RPA_TL_PF_AT(1);
      __builtin_amdgcn_sched_barrier(0);

      // (1) P(b) = 2^(S(b) - m) packed to bf16, under the MFMAs of S(b+1)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) s2[hf][i] = 0.f;
      // p of logit e of sacc; odd e also packs the pair into pk and adds it
      // (as rounded to bf16, the values the p.v MFMAs use) to the row sum
      float pf[32];
      uint32_t pk[16];
      float ls0 = 0.f, ls1 = 0.f;
      auto expo = [&](int e) __attribute__((always_inline)) {
        pf[e] = CAP ? __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], -2.f * cap_l2, c_bias))
                    : __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c_eff, -m_use));
        if (e & 1) {
          pk[e >> 1] = pack_bf16(pf[e - 1], pf[e]);
          const bf16x2 pw = __builtin_bit_cast(bf16x2, pk[e >> 1]);
          if (e & 2) ls1 = __builtin_amdgcn_fdot2_f32_bf16(pw, kOnes2, ls1, false);
          else ls0 = __builtin_amdgcn_fdot2_f32_bf16(pw, kOnes2, ls0, false);
        }
      };
      // Source order is kept by fences: each chunk is one MFMA and its share
      // of VALU work, and the LDS reads of the next k-step are issued a chunk
      // ahead of their MFMAs.  The q.k MFMAs carry the p of logits 0..15, the
      // first half of the p.v MFMAs (k-steps 0, 1, which use only those) the
      // p of logits 16..31, the second half the mask / cap / max of S(b+1).
      constexpr int XA = QF8 ? 8 / KS8 : 8 / KS;   // logits exponentiated per q.k MFMA
      constexpr int XB = 8 / DT;          // per p.v MFMA of k-steps 0, 1
      constexpr int MB = 16 / DT;         // logits max-reduced per p.v MFMA of k-steps 2, 3
      // The two waves of a SIMD take turns: a wave in its compute part
      // outranks one at its barrier / copy part, which keeps the MFMA pipe
      // fed while the other wave catches up (measured 2-3% on long prefill).
      __builtin_amdgcn_s_setprio(1);
      if constexpr (QF8) {
        i32x8 a0 = ld_k8(kn, 0, 0), a1 = ld_k8(kn, 0, 1);
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks) {
          i32x8 n0 = a0, n1 = a1;
          if (ks + 1 < KS8) {
            n0 = ld_k8(kn, ks + 1, 0);
            n1 = ld_k8(kn, ks + 1, 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          s2[0] = mfma_qk8(a0, qreg8[ks], s2[0]);
#pragma unroll
          for (int x = 0; x < XA; ++x) expo((2 * ks) * XA + x);
          __builtin_amdgcn_sched_barrier(0);
          s2[1] = mfma_qk8(a1, qreg8[ks], s2[1]);
#pragma unroll
          for (int x = 0; x < XA; ++x) expo((2 * ks + 1) * XA + x);
          __builtin_amdgcn_sched_barrier(0);
          a0 = n0;
          a1 = n1;
        }
      } else {
        bf16x8 a0 = ld_k(kn, 0, 0), a1 = ld_k(kn, 0, 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 n0 = a0, n1 = a1;
          if (ks + 1 < KS) {
            n0 = ld_k(kn, ks + 1, 0);
            n1 = ld_k(kn, ks + 1, 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          s2[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s2[0], 0, 0, 0);
#pragma unroll
          for (int x = 0; x < XA; ++x) expo((2 * ks) * XA + x);
          __builtin_amdgcn_sched_barrier(0);
          s2[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s2[1], 0, 0, 0);
#pragma unroll
          for (int x = 0; x < XA; ++x) expo((2 * ks + 1) * XA + x);
          __builtin_amdgcn_sched_barrier(0);
          a0 = n0;
          a1 = n1;
        }
      }

      RPA_TL_PF_AT(2);
      // (2) O^T += V^T(b) P^T(b)
      const int k0n = (blk + 1) * BK;
      float m0 = kRedInit, m1 = kRedInit;
      bf16x8 va = ld_vt(vb, 0, 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, make_uint4(pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x8 vn = va;
          if (dt + 1 < DT) vn = ld_vt(vb, ks, dt + 1);
          else if (ks + 1 < 4) vn = ld_vt(vb, ks + 1, 0);
          __builtin_amdgcn_sched_barrier(0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
          const int m = ks * DT + dt;
          if (ks < 2) {
#pragma unroll
            for (int x = 0; x < XB; ++x) expo(16 + m * XB + x);
          } else {
#pragma unroll
            for (int x = 0; x < MB; ++x) {
              const int e = (m - 2 * DT) * MB + x;
              const float sv = logit(mask_next, k0n, s2[e >> 4][e & 15], e);
              s2[e >> 4][e & 15] = sv;
              if (x & 1) m1 = red(m1, sv);
              else m0 = red(m0, sv);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          va = vn;
        }
      }
      RPA_TL_PF_AT(3);
      // Beside the row kernel the wave keeps its raised priority through the
      // barrier and copy part as well: the row waves on its SIMD are older,
      // so at equal priority their loads win the VMEM issue slots, and the
      // part of a step from its barrier to its first q.k MFMA, where the
      // copies are issued, took about 4500 of 10800 clocks (mixed bf16
      // batch: 0.48 -> 0.46 ms per step with the priority kept).
      if (!co_pf) __builtin_amdgcn_s_setprio(0);
      l_run += ls0 + ls1;
      const float mr = red(m0, m1);
      mx = to_mx(red(mr, __shfl_xor(mr, 32)));
      end_step(blk);
      RPA_TL_PF_AT(4);
    };
    // steps [blk, end) in pairs; on return S(blk) is in sa again
    auto run = [&](auto mask_next, int& blk, int end) __attribute__((always_inline)) {
      for (; blk + 1 < end; blk += 2) {
        step(mask_next, blk, sa, sb);
        step(mask_next, blk + 1, sb, sa);
      }
      if (blk < end) {
        step(mask_next, blk, sa, sb);
        sa[0] = sb[0];
        sa[1] = sb[1];
        ++blk;
      }
    };

    // ---- prologue: K(b0) in, then K(b0+1) and V(b0) in flight, S(b0) ----
    const int b0 = blk_first;
    ensure_pages(b0);
    load_k(b0);
    if constexpr (!KDIRECT) {
      stage_staged(kr, kbuf(b0));
      write_staged(kr, b0, 0);
    }
    if constexpr (KDIRECT) wait_vmem_all();
    __syncthreads();
    if constexpr (KDIRECT) write_lds(std::true_type{}, b0, kbuf(b0));
    load_v(b0);
    if (b0 + 1 < blk_end) {
      ensure_pages(b0 + 1);
      load_k(b0 + 1);
    }
    if (wave_live) {
      const char* kb = kbuf(b0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[hf][i] = 0.f;
      if constexpr (QF8) {
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks) {
          sa[0] = mfma_qk8(ld_k8(kb, ks, 0), qreg8[ks], sa[0]);
          sa[1] = mfma_qk8(ld_k8(kb, ks, 1), qreg8[ks], sa[1]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_k(kb, ks, 0), qreg[ks], sa[0], 0, 0, 0);
          sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_k(kb, ks, 1), qreg[ks], sa[1], 0, 0, 0);
        }
      }
      float t = kRedInit;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float s = logit(std::true_type{}, b0 * BK, sa[e >> 4][e & 15], e);
        sa[e >> 4][e & 15] = s;
        t = red(t, s);
      }
      mx = to_mx(red(t, __shfl_xor(t, 32)));
    }
    if constexpr (!VDIRECT) {
      stage_staged(vr, vbuf(b0));
      write_staged(vr, b0, v_bytes);
    }
    if constexpr (!KDIRECT) {
      if (b0 + 1 < blk_end) {
        stage_staged(kr, kbuf(b0 + 1));
        write_staged(kr, b0 + 1, 0);
      }
    }

    // ---- the steps: masked [b0, A), unmasked [A, B), masked [B, end) ----
    if (wave_live) {
      int blk = b0;
      run(std::true_type{}, blk, A);
      run(std::false_type{}, blk, B);
      run(std::true_type{}, blk, blk_end);
    } else {
      for (int blk = b0; blk < blk_end; ++blk) {  // same barriers and loads, no math
        begin_step(blk);
        end_step(blk);
      }
    }

    // ---- finalise: combine the two half-row sums, sink, 1/l, v_scale ----
    if (wave_live) {
      float l_tot = l_run + __shfl_xor(l_run, 32);
      float f = 1.f;
      if (p.sink) {
        const float sg = p.sink[h] * kLog2e;
        const float mxs = fmaxf(m_run, sg);
        f = __builtin_amdgcn_exp2f(m_run - mxs);
        l_tot = l_tot * f + __builtin_amdgcn_exp2f(sg - mxs);
      }
      const float sc = f * p.v_scale / l_tot;
      if (row_ok) {
        uint16_t* op = static_cast<uint16_t*>(p.out) + ((long long)(q0 + row_q) * Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = dt * 32 + j * 8 + kg * 4;
            uint2 o;
            o.x = f32_to_bf16(oacc[dt][4 * j + 0] * sc) |
                  (f32_to_bf16(oacc[dt][4 * j + 1] * sc) << 16);
            o.y = f32_to_bf16(oacc[dt][4 * j + 2] * sc) |
                  (f32_to_bf16(oacc[dt][4 * j + 3] * sc) << 16);
            *reinterpret_cast<uint2*>(op + d) = o;
          }
      }
    }
    __syncthreads();  // LDS is reused by the next unit
  }
  RPA_TL_PF_END();
}

// ---------------------------------------------------------------------------
// Two-group prefill kernel: bf16 queries over a bf16 cache, an even GQA group.
//
// One workgroup of 8 waves per CU, and waves w and w + 4 share a SIMD.  A
// unit is (sequence, tile of up to 128 query tokens, pair of q heads of one
// kv head): group A (waves 0-3) takes the pair's first head, group B (waves
// 4-7) the second, each wave 32 query rows as in prefill_kernel.  Both heads
// see the same keys, so one LDS copy of each K / V block serves both groups,
// half the global -> LDS copies per FLOP of prefill_kernel, and group A's
// waves issue all of them.  Each group runs prefill_kernel's step (rescale;
// q.k of S(b+1) under the exps of S(b); p.v of block b under the max of
// S(b+1); row max and sum), but the step's workgroup barrier falls at a
// different point of it: for A before the q.k part (A then issues the
// copies), for B between the q.k and p.v parts.  The two waves of a SIMD
// therefore run half a step apart, and each one's copies, barrier and tail
// run while the other's MFMAs keep the matrix core busy.
//
// Blocks: A's step b copies V(b+1) and K(b+3).  Barrier b thus finds K(b+1),
// K(b+2) and V(b) in LDS; B computes S(b+1) before barrier b, so K(b+1) must
// have landed by barrier b - 1: three K buffers (block mod 3) and two V
// buffers (block mod 2).  The unit's page ids sit in LDS whole.
template <int D, bool CAP>
__global__ __launch_bounds__(2 * NT, 1) void prefill_pair_kernel(AttnParams p) {
  constexpr int RB = D * 2;                        // LDS row bytes (bf16 K and V)
  constexpr int CPR = RB / 16;                     // 16-byte chunks per row
  constexpr int BLKB = BK * RB;                    // bytes of one K or V block
  constexpr int KS = D / 16;                       // MFMA k-steps of q.k
  constexpr int DT = D / 32;                       // 32-row d tiles of O^T
  constexpr int IPW = BLKB / 1024 / 4;             // direct loads per A wave per block
  constexpr int RPI = 1024 / RB;                   // rows per direct load instruction
  constexpr int PDK = 2;                           // q.k MFMAs a K fragment read runs ahead
  constexpr int PDV = 1;                           // p.v MFMAs a V^T fragment read runs ahead
  static_assert(IPW * RPI == 16, "a wave loads 16 consecutive rows");
  __shared__ __attribute__((aligned(1024))) char s_k[3 * BLKB];
  __shared__ __attribute__((aligned(1024))) char s_v[2 * BLKB];
  __shared__ int s_pt[kPairPages];
  RPA_TL_PP_BEGIN();

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  // beside the row kernel (co_run) prefill_kernel takes the batch instead
  if (hdr->co_run) return;
  const PrefillItem* items = reinterpret_cast<const PrefillItem*>(p.ws + p.lay.pf_items);
  const char* zero_row = reinterpret_cast<const char*>(p.ws + p.lay.zeros);
  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, NPAIR = Hq / 2;
  const long long n_units = (long long)hdr->n_pf_items * NPAIR;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3, gtid = tid & (NT - 1);
  const int kg = lane >> 5, col = lane & 31;
  const int sh = p.ps_shift;
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * 2u;
  const uint32_t v_bytes = (uint32_t)p.Dpad * 2u;
  // non-positive scales: as in prefill_kernel
  const bool q_zero = p.qk_scale == 0.f;
  const uint32_t q_and = q_zero ? 0u : 0xFFFFFFFFu;
  const uint32_t q_xor = p.qk_scale < 0.f ? 0x80008000u : 0u;
  const float scale_pos = q_zero ? 1.f : fabsf(p.qk_scale);
  const float c_scale = CAP ? scale_pos : scale_pos * kLog2e;
  const float c_eff = CAP ? 1.f : c_scale;
  const float cap_k = CAP ? c_scale * 2.f * kLog2e / p.cap : 0.f;
  const float cap_l2 = CAP ? p.cap * kLog2e : 0.f;
  constexpr float kRedInit = CAP ? INFINITY : -INFINITY;
  auto red = [](float a, float b) { return CAP ? fminf(a, b) : fmaxf(a, b); };
  auto to_mx = [&](float v) { return CAP ? fmaf(v, -2.f * cap_l2, cap_l2) : v * c_eff; };

  uint32_t dma_off[IPW], dma_in[IPW];
  const uint32_t in_row = p.in_row_bytes;
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = RPI * j + lane / CPR;
    dma_off[j] = r * row_bytes + (swz_chunk<D>(r, lane % CPR) << 4);
    dma_in[j] = r * in_row + (swz_chunk<D>(r, lane % CPR) << 4);
  }
  const bool fused = p.fuse_update != 0;
  const int fk = swz_f<D>(col);
  const uint32_t k_off = col * RB + ((((fk >> 1) << 1) | (kg ^ (fk & 1))) << 4);
  const int grp16 = lane >> 4, r16 = lane & 15;
  const int rr = (grp16 >> 1) * 4 + (r16 >> 2);
  const int g1 = (2 * (grp16 & 1) + ((r16 & 3) >> 1)) ^ swz_f<D>(rr);
  const uint32_t v_off1 = rr * RB + (g1 << 4) + (r16 & 1) * 8;
  const uint32_t v_off2 = v_off1 ^ 32u;
  auto ld_k = [&](const char* kb, int ks, int hf) -> bf16x8 {
    const char* a = kb + ((k_off ^ (uint32_t)(ks << 5)) + hf * 32 * RB);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a));
  };
  auto ld_vt = [&](const char* vb, int ks, int dt) -> bf16x8 {
    const char* a1 = vb + ((v_off1 ^ (uint32_t)(dt << 6)) + ks * 16 * RB);
    const char* a2 = vb + ((v_off2 ^ (uint32_t)(dt << 6)) + (ks * 16 + 8) * RB);
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a1));
    const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a2));
    const i16x8 av = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
    return __builtin_bit_cast(bf16x8, av);
  };

  // persistent grid over units, as in prefill_kernel (snake order by rounds)
  const unsigned grid = gridDim.x;
  const bool snake = (grid & 7) == 0;
  for (long long k = 0;; ++k) {
    const long long b = (snake && (k & 1)) ? (long long)(grid / 8 - 1 - blockIdx.x / 8) * 8 +
                                                 (blockIdx.x & 7)
                                           : (long long)blockIdx.x;
    const long long u = k * grid + b;
    if (u >= n_units) break;
    const int item_i = (int)(u / NPAIR);
    const int pp = (int)(u - (long long)item_i * NPAIR);
    const int g = pp % Hkv;
    const int h = g * G + 2 * (pp / Hkv) + grp;
    const PrefillItem it = items[item_i];
    const int seq = it.seq;
    const int q0 = p.qsl[seq];
    const int q_len = p.qsl[seq + 1] - q0;
    const int ctx = p.kv_lens[seq] - q_len;
    const int W = p.window;
    const int kv_lo = W > 0 ? max(0, ctx + it.q_begin - W + 1) : 0;
    const int kv_hi = ctx + it.q_end;
    const int* bt = p.block_tables + (long long)seq * p.pps;
    const char* kv_head = static_cast<const char*>(p.cache) + 2LL * g * p.Dpad * 2;
    const char* in_k = fused ? static_cast<const char*>(p.new_k) + (long long)g * D * 2 : nullptr;
    const char* in_v = fused ? static_cast<const char*>(p.new_v) + (long long)g * D * 2 : nullptr;
    const int new_lo = fused ? ctx : INT_MAX;
    // the pair's first q head is kv head g's first: its group writes the new rows
    const bool writer = fused && pp < Hkv && grp == 0;
    const int own_lo = ctx + it.q_begin, own_hi = ctx + it.q_end;
    char* cache_w = const_cast<char*>(kv_head);

    const int row_q = it.q_begin + gw * 32 + col;
    const bool row_ok = row_q < it.q_end;
    const int pos = ctx + row_q;
    const bool wave_live = it.q_begin + gw * 32 < it.q_end;

    const int blk_first = kv_lo / BK;
    const int blk_end = (kv_hi + BK - 1) / BK;
    const int tpos_lo = ctx + it.q_begin, tpos_hi = kv_hi - 1;
    int f_lo = blk_first;
    if (W > 0 && tpos_hi - W >= 0) f_lo = max(f_lo, (tpos_hi - W) / BK + 1);
    f_lo = min(f_lo, blk_end);
    const int f_hi = min(max((tpos_lo + 1) / BK, f_lo), blk_end);
    const int UA = min(max(blk_first, f_lo - 1), blk_end);
    const int UB = max(UA, f_hi - 1);

    // page ids of the unit's whole key range in LDS (the host launches this
    // kernel only when a sequence's block table fits)
    const int pt_base = kv_lo >> sh;
    for (int i = tid, n = ((kv_hi - 1) >> sh) - pt_base + 1; i < n; i += 2 * NT)
      s_pt[i] = bt[pt_base + i];
    auto kbuf = [&](int blk) -> char* { return s_k + (blk % 3) * BLKB; };
    auto vbuf = [&](int blk) -> char* { return s_v + (blk & 1) * BLKB; };
    // group A's copy of a block's 16 rows per wave (vofs: 0 K rows, v_bytes V rows)
    auto copy_block = [&](int blk, char* buf, uint32_t vofs, const char* in_base)
                          __attribute__((always_inline)) {
      const int t0 = blk * BK + 16 * gw;
      const uint32_t lds0 = lds_addr(buf + gw * IPW * 1024);
      if (t0 >= kv_lo && t0 + 16 <= min(kv_hi, new_lo)) {
        const int page = __builtin_amdgcn_readfirstlane(s_pt[(t0 >> sh) - pt_base]);
        const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(t0 & pmask);
        const char* base = uniform_ptr(kv_head + vofs + (uint64_t)crow * row_bytes);
#pragma unroll
        for (int j = 0; j < IPW; ++j) dma16_s(base, dma_off[j], lds0 + j * 1024);
      } else if (t0 >= max(kv_lo, new_lo) && t0 + 16 <= kv_hi) {
        const char* base = uniform_ptr(in_base + (uint64_t)(q0 + t0 - ctx) * in_row);
#pragma unroll
        for (int j = 0; j < IPW; ++j) dma16_s(base, dma_in[j], lds0 + j * 1024);
      } else {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
          const int r = RPI * j + lane / CPR;
          const int tok = t0 + r;
          const int lc = swz_chunk<D>(r, lane % CPR);
          const char* src = zero_row + (lc << 4);
          if (tok >= kv_lo && tok < kv_hi) {
            if (tok >= new_lo) {
              src = in_base + (uint64_t)(q0 + tok - ctx) * in_row + (lc << 4);
            } else {
              const int page = s_pt[(tok >> sh) - pt_base];
              const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
              src = kv_head + vofs + (uint64_t)crow * row_bytes + (lc << 4);
            }
          }
          dma16(src, lds0 + j * 1024);
        }
      }
    };
    auto load_k = [&](int blk) { copy_block(blk, kbuf(blk), 0, in_k); };
    auto load_v = [&](int blk) { copy_block(blk, vbuf(blk), v_bytes, in_v); };
    // fused update: group A of the writer pair stores its tile's new rows of
    // block blk from the LDS buffer (pad lanes zeroed)
    auto write_lds = [&](int blk, const char* buf, uint32_t vofs) {
      if (!writer) return;
      const int lo = max(blk * BK, own_lo), hi = min(blk * BK + BK, own_hi);
      if (lo >= hi) return;
      const int wch = p.Dpad * 2 / 16;
      const int n = (hi - lo) * wch;
      for (int i = gtid; i < n; i += NT) {
        const int r2 = i / wch, c = i - r2 * wch;
        const int tok = lo + r2, r = tok - blk * BK;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < CPR) v = *reinterpret_cast<const uint4*>(buf + r * RB + (swz_chunk<D>(r, c) << 4));
        const int page = s_pt[(tok >> sh) - pt_base];  // own rows lie in the unit's range
        char* row = cache_w + (uint64_t)(((uint32_t)page << sh) | (uint32_t)(tok & pmask)) * row_bytes;
        *reinterpret_cast<uint4*>(row + vofs + c * 16) = v;
      }
    };

    bf16x8 qreg[KS];
    {
      const long long qrow = (long long)(q0 + (row_ok ? row_q : it.q_begin)) * Hq + h;
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + qrow * D + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
        v = make_uint4((v.x & q_and) ^ q_xor, (v.y & q_and) ^ q_xor, (v.z & q_and) ^ q_xor,
                       (v.w & q_and) ^ q_xor);
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 sa[2], sb[2];
    float mx = -INFINITY;
    auto logit = [&](auto masked, int k0, float sv, int e) __attribute__((always_inline)) -> float {
      if constexpr (CAP) sv = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * cap_k) + 1.f);
      if constexpr (decltype(masked)::value) {
        const int ko = (e >> 4) * 32 + ((e & 15) >> 2) * 8 + (e & 3);
        const int lim = pos - k0 - 4 * kg;
        const bool vis = ko <= lim && (W <= 0 || ko > lim - W);
        sv = vis ? sv : kRedInit;
      }
      return sv;
    };

    // One step on block blk: sacc holds S(blk), s2 receives S(blk + 1).  The
    // barrier (and for group A the copies) sits where the wave's group takes
    // it (see above).
    auto step = [&](auto mask_next, int blk, f32x16(&sacc)[2], f32x16(&s2)[2])
                    __attribute__((always_inline)) {
      constexpr bool MASK_NEXT = decltype(mask_next)::value;
      if (grp == 0) {
        wait_vmem_all();
        __syncthreads();
        if (blk + 1 < blk_end) load_v(blk + 1);
        if (blk + 3 < blk_end) load_k(blk + 3);
        if (blk + 1 < blk_end) write_lds(blk + 1, kbuf(blk + 1), 0);
        write_lds(blk, vbuf(blk), v_bytes);
      }
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float c_bias = cap_l2 - m_use;
      const char* kn = kbuf(blk + 1);
      const char* vb = vbuf(blk);
      RPA_TL_PP_LAP(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) s2[hf][i] = 0.f;
      float pf[32];
      uint32_t pk[16];
      float ls0 = 0.f, ls1 = 0.f;
      auto expo = [&](int e) __attribute__((always_inline)) {
        pf[e] = CAP ? __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], -2.f * cap_l2, c_bias))
                    : __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c_eff, -m_use));
        if (e & 1) {
          pk[e >> 1] = pack_bf16(pf[e - 1], pf[e]);
          const bf16x2 pw = __builtin_bit_cast(bf16x2, pk[e >> 1]);
          if (e & 2) ls1 = __builtin_amdgcn_fdot2_f32_bf16(pw, kOnes2, ls1, false);
          else ls0 = __builtin_amdgcn_fdot2_f32_bf16(pw, kOnes2, ls0, false);
          // kept in this chunk: group B's barrier below would otherwise let
          // these sink below the MFMAs they run under
          asm volatile("" ::"v"(pk[e >> 1]), "v"((e & 2) ? ls1 : ls0));
        }
      };
      constexpr int XA = 8 / KS, XB = 8 / DT, MB = 16 / DT;
      // A q.k fragment is read PDK MFMAs ahead of its MFMA, a V^T fragment
      // PDV MFMAs (reading further ahead measured no faster).
      {
        bf16x8 kq[2 * KS];
#pragma unroll
        for (int m = 0; m < PDK; ++m) kq[m] = ld_k(kn, m >> 1, m & 1);
#pragma unroll
        for (int m = 0; m < 2 * KS; ++m) {
          if (m + PDK < 2 * KS) kq[m + PDK] = ld_k(kn, (m + PDK) >> 1, (m + PDK) & 1);
          __builtin_amdgcn_sched_barrier(0);
          s2[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[m], qreg[m >> 1], s2[m & 1], 0, 0, 0);
#pragma unroll
          for (int x = 0; x < XA; ++x) expo(m * XA + x);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      RPA_TL_PP_LAP(1);
      if (grp != 0) __syncthreads();
      RPA_TL_PP_LAP(2);
      const int k0n = (blk + 1) * BK;
      float m0 = kRedInit, m1 = kRedInit;
      bf16x8 vq[4 * DT];
#pragma unroll
      for (int m = 0; m < PDV; ++m) vq[m] = ld_vt(vb, m / DT, m % DT);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, make_uint4(pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int m = ks * DT + dt;
          if (m + PDV < 4 * DT) vq[m + PDV] = ld_vt(vb, (m + PDV) / DT, (m + PDV) % DT);
          __builtin_amdgcn_sched_barrier(0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[m], pb, oacc[dt], 0, 0, 0);
          if (ks < 2) {
#pragma unroll
            for (int x = 0; x < XB; ++x) expo(16 + m * XB + x);
          } else {
#pragma unroll
            for (int x = 0; x < MB; ++x) {
              const int e = (m - 2 * DT) * MB + x;
              const float sv = logit(mask_next, k0n, s2[e >> 4][e & 15], e);
              s2[e >> 4][e & 15] = sv;
              if (x & 1) m1 = red(m1, sv);
              else m0 = red(m0, sv);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      RPA_TL_PP_LAP(3);
      l_run += ls0 + ls1;
      const float mr = red(m0, m1);
      mx = to_mx(red(mr, __shfl_xor(mr, 32)));
      (void)MASK_NEXT;
      RPA_TL_PP_LAP(4);
      RPA_TL_PP_STEP();
    };
    // a wave with no query rows takes the same barriers and copies, no math
    auto idle_step = [&](int blk) __attribute__((always_inline)) {
      if (grp == 0) {
        wait_vmem_all();
        __syncthreads();
        if (blk + 1 < blk_end) load_v(blk + 1);
        if (blk + 3 < blk_end) load_k(blk + 3);
        if (blk + 1 < blk_end) write_lds(blk + 1, kbuf(blk + 1), 0);
        write_lds(blk, vbuf(blk), v_bytes);
      } else {
        __syncthreads();
      }
    };
    auto run = [&](auto mask_next, int& blk, int end) __attribute__((always_inline)) {
      for (; blk + 1 < end; blk += 2) {
        step(mask_next, blk, sa, sb);
        step(mask_next, blk + 1, sb, sa);
      }
      if (blk < end) {
        step(mask_next, blk, sa, sb);
        sa[0] = sb[0];
        sa[1] = sb[1];
        ++blk;
      }
    };
    auto run_all = [&]() __attribute__((always_inline)) {
      if (wave_live) {
        int blk = blk_first;
        run(std::true_type{}, blk, UA);
        run(std::false_type{}, blk, UB);
        run(std::true_type{}, blk, blk_end);
      } else {
        for (int blk = blk_first; blk < blk_end; ++blk) idle_step(blk);
      }
    };

    // ---- prologue: K(b0), K(b0+1) in; then V(b0), K(b0+2) in flight; S(b0) ----
    const int b0 = blk_first;
    __syncthreads();  // the page table is in LDS
    if (grp == 0) {
      load_k(b0);
      if (b0 + 1 < blk_end) load_k(b0 + 1);
    }
    wait_vmem_all();
    __syncthreads();
    if (grp == 0) {
      write_lds(b0, kbuf(b0), 0);
      load_v(b0);
      if (b0 + 2 < blk_end) load_k(b0 + 2);
    }
    if (wave_live) {
      const char* kb = kbuf(b0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[hf][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_k(kb, ks, 0), qreg[ks], sa[0], 0, 0, 0);
        sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_k(kb, ks, 1), qreg[ks], sa[1], 0, 0, 0);
      }
      float t = kRedInit;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float sv = logit(std::true_type{}, b0 * BK, sa[e >> 4][e & 15], e);
        sa[e >> 4][e & 15] = sv;
        t = red(t, sv);
      }
      mx = to_mx(red(t, __shfl_xor(t, 32)));
    }
    run_all();

    // ---- finalise (as prefill_kernel) ----
    if (wave_live) {
      float l_tot = l_run + __shfl_xor(l_run, 32);
      float f = 1.f;
      if (p.sink) {
        const float sg = p.sink[h] * kLog2e;
        const float mxs = fmaxf(m_run, sg);
        f = __builtin_amdgcn_exp2f(m_run - mxs);
        l_tot = l_tot * f + __builtin_amdgcn_exp2f(sg - mxs);
      }
      const float sc = f * p.v_scale / l_tot;
      if (row_ok) {
        uint16_t* op = static_cast<uint16_t*>(p.out) + ((long long)(q0 + row_q) * Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = dt * 32 + j * 8 + kg * 4;
            uint2 o;
            o.x = f32_to_bf16(oacc[dt][4 * j + 0] * sc) |
                  (f32_to_bf16(oacc[dt][4 * j + 1] * sc) << 16);
            o.y = f32_to_bf16(oacc[dt][4 * j + 2] * sc) |
                  (f32_to_bf16(oacc[dt][4 * j + 3] * sc) << 16);
            *reinterpret_cast<uint2*>(op + d) = o;
          }
      }
    }
    wait_vmem_all();
    __syncthreads();  // LDS is reused by the next unit
    RPA_TL_PP_LAP(5);
  }
  RPA_TL_PP_END();
}

long long resident_grid(const void* kernel) {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NT, 0) != hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      per_cu * cus < 8)
    return kPrefillGrid;
  return (long long)(per_cu * cus) / 8 * 8;
}

template <typename CT, int D, bool CAP, bool QF8>
hipError_t launch_d(const AttnParams& p, long long blocks, hipStream_t s) {
  // persistent grid: the resident workgroups, rounded down to a multiple of 8
  // so that block b and its later units b + grid sit on the same XCD
  static const long long resident =
      resident_grid(reinterpret_cast<const void*>(&prefill_kernel<CT, D, CAP, QF8>));
  if (blocks > resident) blocks = resident;
  if (trace_active()) {
    char nm[80];
    std::snprintf(nm, sizeof nm, "prefill_kernel<%s%s,D%d%s>(%s%s)", elem_name<CT>(),
                  QF8 ? ",q_fp8" : "", D, CAP ? ",cap" : "",
                  p.fuse_merge ? "merge+tiles" : "tiles", p.fuse_update ? "+update" : "");
    if (trace_launch(nm, (unsigned)blocks, NT, 0, s)) return hipSuccess;
  }
  prefill_kernel<CT, D, CAP, QF8><<<dim3((unsigned)blocks), NT, 0, s>>>(p);
  return hipGetLastError();
}

template <int D, bool CAP>
hipError_t launch_pair_d(const AttnParams& p, long long blocks, hipStream_t s) {
  static const long long resident = [] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&prefill_pair_kernel<D, CAP>), 2 * NT, 0) !=
            hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu * cus < 8)
      return kPrefillGrid / 2;
    return (long long)(per_cu * cus) / 8 * 8;
  }();
  if (blocks > resident) blocks = resident;
  if (trace_active()) {
    char nm[80];
    std::snprintf(nm, sizeof nm, "prefill_pair_kernel<bf16,D%d%s>(tiles%s)", D, CAP ? ",cap" : "",
                  p.fuse_update ? "+update" : "");
    if (trace_launch(nm, (unsigned)blocks, 2 * NT, 0, s)) return hipSuccess;
  }
  prefill_pair_kernel<D, CAP><<<dim3((unsigned)blocks), 2 * NT, 0, s>>>(p);
  return hipGetLastError();
}

// The two-group kernel serves bf16 queries over a bf16 cache with an even
// GQA group, when the prefill kernel does not also merge the rows' splits
// and a sequence's block table fits in its LDS page table.
bool pair_eligible(const AttnParams& p, bool bf16_cache, bool qf8) {
  return bf16_cache && !qf8 && !p.fuse_merge && p.Hkv > 0 && (p.Hq / p.Hkv) % 2 == 0 &&
         p.Dpad == p.D && p.pps <= kPairPages;
}

template <typename CT, bool QF8>
hipError_t launch_t(const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  const long long merge_blocks =
      p.fuse_merge ? ((long long)p.lay.max_merge_rows * p.Hkv + 3) / 4 : 0;
  const long long blocks = std::max((long long)p.lay.max_pf_items * p.Hq, merge_blocks);
  if (blocks <= 0) return hipSuccess;
  const bool cap = p.cap > 0.f;
  // prefill_kernel first: when the planner runs it beside the rows (co_run)
  // it must not queue behind the two-group kernel, which needs whole CUs and
  // then exits at once
  p.pf_pair = pair_eligible(p, sizeof(CT) == 2, QF8) ? 1 : 0;
  hipError_t e;
  if (p.D == 64)
    e = cap ? launch_d<CT, 64, true, QF8>(p, blocks, s) : launch_d<CT, 64, false, QF8>(p, blocks, s);
  else
    e = cap ? launch_d<CT, 128, true, QF8>(p, blocks, s) : launch_d<CT, 128, false, QF8>(p, blocks, s);
  if (e != hipSuccess || !p.pf_pair) return e;
  const long long pblocks = (long long)p.lay.max_pf_items * (p.Hq / 2);
  if (p.D == 64)
    return cap ? launch_pair_d<64, true>(p, pblocks, s) : launch_pair_d<64, false>(p, pblocks, s);
  return cap ? launch_pair_d<128, true>(p, pblocks, s) : launch_pair_d<128, false>(p, pblocks, s);
}

}  // namespace

bool prefill_supported(const rpa_desc& d) {
  const bool bf16_q =
      d.q_dtype == RPA_BF16 && (d.cache_dtype == RPA_BF16 || d.cache_dtype == RPA_FP8_E4M3);
  const bool fp8_q = d.q_dtype == RPA_FP8_E4M3 && d.cache_dtype == RPA_FP8_E4M3;
  return (bf16_q || fp8_q) && (d.head_dim == 64 || d.head_dim == 128);
}

hipError_t launch_prefill(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt,
                          hipStream_t s) {
  if (q_dt == RPA_BF16 && cache_dt == RPA_BF16) return launch_t<uint16_t, false>(p, s);
  if (q_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) return launch_t<uint8_t, false>(p, s);
  if (q_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) return launch_t<uint8_t, true>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace rpa

#ifdef RPA_WAVE_TIMELINE
// The prefill kernel's per-wave clock counts of the measurement build: n
// words, 8 per wave (total, copy wait, barrier wait, steps, then the issue,
// q.k, p.v and tail parts of the steps).
extern "C" int rpa_pf_timeline_read(unsigned long long* host, int n) {
  if (n > rpa::kPfTimelineWaves * rpa::kPfWords) n = rpa::kPfTimelineWaves * rpa::kPfWords;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(rpa::g_pf_timeline),
                                  (size_t)n * sizeof(unsigned long long), 0, hipMemcpyDeviceToHost);
}
extern "C" int rpa_pp_timeline_read(unsigned long long* host, int n) {
  if (n > rpa::kPfTimelineWaves * rpa::kPfWords) n = rpa::kPfTimelineWaves * rpa::kPfWords;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(rpa::g_pp_timeline),
                                  (size_t)n * sizeof(unsigned long long), 0, hipMemcpyDeviceToHost);
}
extern "C" int rpa_pf_timeline_clear(void) {
  static unsigned long long zero[rpa::kPfTimelineWaves * rpa::kPfWords];
  const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(rpa::g_pp_timeline), zero, sizeof(zero), 0,
                                         hipMemcpyHostToDevice);
  if (e != hipSuccess) return (int)e;
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(rpa::g_pf_timeline), zero, sizeof(zero), 0,
                                hipMemcpyHostToDevice);
}
#endif
