// Prefill / mixed-chunk kernel on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// One workgroup = one (sequence, tile of up to 128 query tokens, q head);
// each of its 4 waves owns 32 query rows.  The key range the tile can see is
// walked in 64-token blocks fetched from the paged cache through the block
// table into LDS (tpu-inference v3 kernel diff, "_fetch_bkv": per page, copy
// min(page_size, left) token rows), with the online softmax of
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
// fp8 (e4m3) caches are widened to bf16 (exactly) while staging into LDS;
// k_scale is folded into the logit scale and v_scale into the final 1/l.
#include <math.h>

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) * lds_i16_ptr;

constexpr int BQ = kPrefillBQ;  // query rows per workgroup
constexpr int BK = 64;          // keys per block
constexpr int NT = 256;         // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <typename CT> struct CacheElem;
template <> struct CacheElem<uint16_t> { static constexpr int size = 2; };
template <> struct CacheElem<uint8_t> { static constexpr int size = 1; };

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return a | (b << 16);
}

// two e4m3 codes (bytes 0/1, or 2/3 with HI) -> two bf16 packed in one word (exact)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

template <typename CT, int D>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(AttnParams p) {
  constexpr int LS = D + 16;                       // LDS row stride (bf16 elements)
  constexpr int KS = D / 16;                       // MFMA k-steps of q.k
  constexpr int DT = D / 32;                       // 32-row d tiles of O^T
  constexpr int ESZ = CacheElem<CT>::size;
  constexpr int CPR = D * ESZ / 16;                // 16-byte chunks per cached head row
  constexpr int PER = BK * CPR / NT;               // chunks per thread per block
  static_assert(PER >= 1 && BK * CPR % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t sK[BK * LS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BK * LS];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const PrefillItem* items = reinterpret_cast<const PrefillItem*>(p.ws + p.lay.pf_items);
  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const long long b = blockIdx.x;
  if (b >= (long long)hdr->n_pf_items * Hq) return;
  const int item_i = (int)(b / Hq);
  const int hh = (int)(b - (long long)item_i * Hq);
  // consecutive blocks go to different XCDs; mapping hh -> (kv head hh % Hkv)
  // keeps every q head of one kv head on the same XCD (and its L2)
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
  const int ps = p.page_size;
  const long long row_stride = 2LL * Hkv * p.Dpad;
  const CT* kv_head = static_cast<const CT*>(p.cache) + 2LL * g * p.Dpad;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;
  const int row_q = it.q_begin + wave * 32 + col;  // this lane's query row (within the seq)
  const bool row_ok = row_q < it.q_end;
  const int pos = ctx + row_q;
  const int wave_q_lo = it.q_begin + wave * 32;
  const bool wave_live = wave_q_lo < it.q_end;
  const int wpos_lo = ctx + wave_q_lo;
  const int wpos_hi = ctx + min(it.q_end, wave_q_lo + 32) - 1;

  // Q^T operand: 8 bf16 of row row_q, d = 16 ks + 8 kg .. +7
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((long long)(q0 + (row_ok ? row_q : it.q_begin)) * Hq + h) * D + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const bool use_cap = p.cap > 0.f;
  const float c_scale = use_cap ? p.qk_scale : p.qk_scale * kLog2e;
  const float c_eff = use_cap ? 1.f : c_scale;   // multiplier from stored logits to log2 units

  // Staged loads of one key block: PER chunks of K and of V per thread.  The
  // page ids a block needs are fetched one block earlier than its data, so a
  // data load never waits on a block-table load.
  uint4 kr[PER], vr[PER];
  int pg[PER];
  auto fetch_pages = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = k0 + (tid + NT * i) / CPR;
      pg[i] = (j >= kv_lo && j < kv_hi) ? bt[j / ps] : -1;
    }
  };
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + NT * i;
      const int tok = c / CPR, cc = c - (c / CPR) * CPR;
      const int j = k0 + tok;
      uint4 a = make_uint4(0, 0, 0, 0), v = a;
      if (pg[i] >= 0) {
        const CT* src = kv_head + ((long long)pg[i] * ps + (j - (j / ps) * ps)) * row_stride +
                        cc * (16 / ESZ);
        a = *reinterpret_cast<const uint4*>(src);
        v = *reinterpret_cast<const uint4*>(src + p.Dpad);
      }
      kr[i] = a;
      vr[i] = v;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + NT * i;
      const int tok = c / CPR, cc = c - (c / CPR) * CPR;
      if constexpr (ESZ == 2) {
        *reinterpret_cast<uint4*>(&sK[tok * LS + cc * 8]) = kr[i];
        *reinterpret_cast<uint4*>(&sV[tok * LS + cc * 8]) = vr[i];
      } else {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
        const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        uint32_t ko[8], vo[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ko[2 * e] = fp8x2_to_bf16x2<false>(kw[e]);
          ko[2 * e + 1] = fp8x2_to_bf16x2<true>(kw[e]);
          vo[2 * e] = fp8x2_to_bf16x2<false>(vw[e]);
          vo[2 * e + 1] = fp8x2_to_bf16x2<true>(vw[e]);
        }
        uint4* dk = reinterpret_cast<uint4*>(&sK[tok * LS + cc * 16]);
        uint4* dv = reinterpret_cast<uint4*>(&sV[tok * LS + cc * 16]);
        dk[0] = make_uint4(ko[0], ko[1], ko[2], ko[3]);
        dk[1] = make_uint4(ko[4], ko[5], ko[6], ko[7]);
        dv[0] = make_uint4(vo[0], vo[1], vo[2], vo[3]);
        dv[1] = make_uint4(vo[4], vo[5], vo[6], vo[7]);
      }
    }
  };

  const int blk_first = kv_lo / BK;
  const int blk_end = (kv_hi + BK - 1) / BK;
  if (blk_first < blk_end) {
    fetch_pages(blk_first * BK);
    fetch(blk_first * BK);
    if (blk_first + 1 < blk_end) fetch_pages((blk_first + 1) * BK);
  }
  for (int blk = blk_first; blk < blk_end; ++blk) {
    const int k0 = blk * BK;
    __syncthreads();                      // previous block fully consumed
    stage();
    __syncthreads();                      // block visible to all waves
    if (blk + 1 < blk_end) {              // next block in flight during the math
      fetch(k0 + BK);
      if (blk + 2 < blk_end) fetch_pages(k0 + 2 * BK);
    }

    // does this wave see any key of the block, and does it need a mask?
    const bool needed = wave_live && k0 <= wpos_hi && (W <= 0 || k0 + BK - 1 > wpos_lo - W);
    if (!needed) continue;
    const bool full = (k0 + BK - 1 <= wpos_lo) && (W <= 0 || wpos_hi - k0 < W);

    // ---- S^T = K Q^T : two 32-key halves ----
    f32x16 sacc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[hf][i] = 0.f;
      const uint16_t* kp = &sK[(hf * 32 + col) * LS + 8 * kg];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + 16 * ks));
        sacc[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[hf], 0, 0, 0);
      }
    }
    // ---- logits (log2 units), mask, block max ----
    // Without a cap the scale is folded into the exponent: p = 2^(s*c - m).
    float mx = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = sacc[hf][i];
        if (use_cap) s = p.cap * tanhf(s * c_scale / p.cap) * kLog2e;
        if (!full) {
          const int j = k0 + hf * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
          const bool vis = j <= pos && (W <= 0 || pos - j < W);
          s = vis ? s : -INFINITY;
        }
        sacc[hf][i] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c_eff;
    // Lazy rescaling: the running max only moves (and acc / l are only
    // rescaled) when some row of the wave grows by more than 2^8; until then
    // p <= 2^8, harmless in fp32 sums and in bf16.
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
    float lsum = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[hf][i], c_eff, -m_use));
        sacc[hf][i] = pv;
        lsum += pv;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T over four 16-key steps ----
    const int grp = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int hf = ks >> 1, qq = ks & 1;
      uint4 pw;
      pw.x = pack_bf16(sacc[hf][8 * qq + 0], sacc[hf][8 * qq + 1]);
      pw.y = pack_bf16(sacc[hf][8 * qq + 2], sacc[hf][8 * qq + 3]);
      pw.z = pack_bf16(sacc[hf][8 * qq + 4], sacc[hf][8 * qq + 5]);
      pw.w = pack_bf16(sacc[hf][8 * qq + 6], sacc[hf][8 * qq + 7]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
      const int tb = 16 * ks + (grp >> 1) * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d0 = dt * 32 + (grp & 1) * 16;
        uint16_t* a1 = &sV[(tb + (r16 >> 2)) * LS + d0 + 4 * (r16 & 3)];
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16_ptr)(a1));
        const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16_ptr)(a1 + 8 * LS));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 av = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                           oacc[dt], 0, 0, 0);
      }
    }
  }

  // ---- finalise: combine the two half-row sums, sink, 1/l, v_scale ----
  if (!wave_live) return;
  float l_tot = l_run + __shfl_xor(l_run, 32);
  float f = 1.f;
  if (p.sink) {
    const float sg = p.sink[h] * kLog2e;
    const float mx = fmaxf(m_run, sg);
    f = __builtin_amdgcn_exp2f(m_run - mx);
    l_tot = l_tot * f + __builtin_amdgcn_exp2f(sg - mx);
  }
  const float sc = f * p.v_scale / l_tot;
  if (!row_ok) return;
  uint16_t* op = static_cast<uint16_t*>(p.out) + ((long long)(q0 + row_q) * Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = dt * 32 + j * 8 + kg * 4;
      uint2 o;
      o.x = f32_to_bf16(oacc[dt][4 * j + 0] * sc) | (f32_to_bf16(oacc[dt][4 * j + 1] * sc) << 16);
      o.y = f32_to_bf16(oacc[dt][4 * j + 2] * sc) | (f32_to_bf16(oacc[dt][4 * j + 3] * sc) << 16);
      *reinterpret_cast<uint2*>(op + d) = o;
    }
}

template <typename CT>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  const long long blocks = (long long)p.lay.max_pf_items * p.Hq;
  if (blocks <= 0) return hipSuccess;
  if (p.D == 64) prefill_kernel<CT, 64><<<dim3((unsigned)blocks), NT, 0, s>>>(p);
  else prefill_kernel<CT, 128><<<dim3((unsigned)blocks), NT, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(const rpa_desc& d) {
  return d.q_dtype == RPA_BF16 && (d.cache_dtype == RPA_BF16 || d.cache_dtype == RPA_FP8_E4M3) &&
         (d.head_dim == 64 || d.head_dim == 128);
}

hipError_t launch_prefill(const AttnParams& p, rpa_dtype q_dt, rpa_dtype cache_dt,
                          hipStream_t s) {
  if (q_dt != RPA_BF16) return hipErrorInvalidValue;
  if (cache_dt == RPA_BF16) return launch_t<uint16_t>(p, s);
  if (cache_dt == RPA_FP8_E4M3) return launch_t<uint8_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace rpa
