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

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;

constexpr int BK = 64;          // keys per block
constexpr int NT = 256;         // threads per workgroup
constexpr int NS = 2;           // LDS stages (bf16 caches)
constexpr int kPT = 512;        // page ids cached in LDS per refill
constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kPrefillGrid = 1024;  // fallback persistent grid (multiple of 8)

template <typename CT> struct CacheElem;
template <> struct CacheElem<uint16_t> { static constexpr int size = 2; };
template <> struct CacheElem<uint8_t> { static constexpr int size = 1; };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (RNE) in one word: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// two e4m3 codes (bytes 0/1, or 2/3 with HI) -> two bf16 packed in one word (exact)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
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

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0) (gfx9 encoding), leaving expcnt / lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// 16 bytes per lane global -> LDS at lds_base + 16 * lane (global_load_lds_dwordx4).
// Issued from asm so that the compiler does not serialise the LDS reads of the
// other stage behind these loads; the kernel orders them itself with
// wait_vmem_all() + a barrier before the stage is read.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_base)
               : "memory", "m0");
}

template <typename CT, int D>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(AttnParams p) {
  constexpr bool DIRECT = sizeof(CT) == 2;         // bf16 cache: global -> LDS directly
  constexpr int RB = D * 2;                        // LDS row bytes (bf16)
  constexpr int CPR = RB / 16;                     // 16-byte LDS chunks per row
  constexpr int BLKB = BK * RB;                    // bytes of one K (or V) block
  constexpr int KS = D / 16;                       // MFMA k-steps of q.k
  constexpr int DT = D / 32;                       // 32-row d tiles of O^T
  constexpr int IPW = BLKB / 1024 / 4;             // direct loads per wave per K (or V) block
  constexpr int RPI = 1024 / RB;                   // rows per direct load instruction
  constexpr int ESZ = CacheElem<CT>::size;
  constexpr int GCPR = D * ESZ / 16;               // 16-byte chunks of a cached head row
  constexpr int PER = BK * GCPR / NT;              // staged chunks per thread (e4m3 path)
  constexpr int NSTAGE = DIRECT ? NS : 1;
  static_assert(!DIRECT || IPW >= 1, "direct split");
  static_assert(DIRECT || (PER >= 1 && BK * GCPR % NT == 0), "staged split");
  // stage buffers are distinct objects so the compiler can tell that the
  // loads streaming into one stage do not alias the reads of the other
  __shared__ __attribute__((aligned(1024))) char smem[2 * BLKB];
  __shared__ __attribute__((aligned(1024))) char smem1[DIRECT ? 2 * BLKB : 16];
  __shared__ int s_pt[kPT];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(p.ws + p.lay.header);
  const PrefillItem* items = reinterpret_cast<const PrefillItem*>(p.ws + p.lay.pf_items);
  const uint16_t* zero_row = reinterpret_cast<const uint16_t*>(p.ws + p.lay.zeros);
  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const long long n_units = (long long)hdr->n_pf_items * Hq;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 5, col = lane & 31;
  const int sh = p.ps_shift;                       // page_size = 1 << sh
  const int pmask = (1 << sh) - 1;
  const uint32_t row_bytes = 2u * Hkv * p.Dpad * (uint32_t)ESZ;  // one cache token row
  const bool use_cap = p.cap > 0.f;
  const float c_scale = use_cap ? p.qk_scale : p.qk_scale * kLog2e;
  const float c_eff = use_cap ? 1.f : c_scale;   // stored logits -> log2 units

  // Persistent grid (a multiple of 8 blocks): block b takes units b, b + grid,
  // ...  Consecutive units sit on different XCDs; the head slot -> (kv head =
  // slot mod Hkv) mapping keeps the q heads of one kv head on one XCD and L2.
  for (long long u = blockIdx.x; u < n_units; u += gridDim.x) {
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
    const CT* kv_head = static_cast<const CT*>(p.cache) + 2LL * g * p.Dpad;

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

    const int blk_first = kv_lo / BK;
    const int blk_end = (kv_hi + BK - 1) / BK;

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

    // ---- loads of one block ----
    auto issue_direct = [&](int blk, char* stage) {  // bf16: global -> LDS, IPW x 2 per wave
      const int k0 = blk * BK;
      char* ks_ = stage;
      char* vs_ = stage + BLKB;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int inst = wave * IPW + j;
        const int row = inst * RPI + lane / CPR;
        const int c = swz_chunk<D>(row, lane % CPR);
        const int tok = k0 + row;
        const uint16_t* ksrc = zero_row + c * 8;
        const uint16_t* vsrc = ksrc;
        if (tok >= kv_lo && tok < kv_hi) {
          const int page = s_pt[(tok >> sh) - pt_base];
          const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
          ksrc = reinterpret_cast<const uint16_t*>(
              reinterpret_cast<const char*>(kv_head) + (uint64_t)crow * row_bytes + c * 16);
          vsrc = ksrc + p.Dpad;
        }
        const uint32_t kdst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ks_ + inst * 1024));
        const uint32_t vdst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(vs_ + inst * 1024));
        dma16(ksrc, kdst);
        dma16(vsrc, vdst);
      }
    };
    uint4 kr[DIRECT ? 1 : PER], vr[DIRECT ? 1 : PER];
    auto fetch_staged = [&](int blk) {       // e4m3: global -> registers
#pragma unroll
      for (int i = 0; i < (DIRECT ? 0 : PER); ++i) {
        const int cidx = tid + NT * i;
        const int tok = blk * BK + cidx / GCPR, cc = cidx % GCPR;
        uint4 a = make_uint4(0, 0, 0, 0), v = a;
        if (tok >= kv_lo && tok < kv_hi) {
          const int page = s_pt[(tok >> sh) - pt_base];
          const uint32_t crow = ((uint32_t)page << sh) | (uint32_t)(tok & pmask);
          const CT* src = reinterpret_cast<const CT*>(
              reinterpret_cast<const char*>(kv_head) + (uint64_t)crow * row_bytes + cc * 16);
          a = *reinterpret_cast<const uint4*>(src);
          v = *reinterpret_cast<const uint4*>(src + p.Dpad);
        }
        kr[i] = a;
        vr[i] = v;
      }
    };
    auto stage_staged = [&]() {              // e4m3 -> bf16 into the swizzled rows
#pragma unroll
      for (int i = 0; i < (DIRECT ? 0 : PER); ++i) {
        const int cidx = tid + NT * i;
        const int row = cidx / GCPR, cc = cidx % GCPR;
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
        char* kb = smem + row * RB;
        char* vb = smem + BLKB + row * RB;
        *reinterpret_cast<uint4*>(kb + (swz_chunk<D>(row, 2 * cc) << 4)) =
            make_uint4(ko[0], ko[1], ko[2], ko[3]);
        *reinterpret_cast<uint4*>(kb + (swz_chunk<D>(row, 2 * cc + 1) << 4)) =
            make_uint4(ko[4], ko[5], ko[6], ko[7]);
        *reinterpret_cast<uint4*>(vb + (swz_chunk<D>(row, 2 * cc) << 4)) =
            make_uint4(vo[0], vo[1], vo[2], vo[3]);
        *reinterpret_cast<uint4*>(vb + (swz_chunk<D>(row, 2 * cc + 1) << 4)) =
            make_uint4(vo[4], vo[5], vo[6], vo[7]);
      }
    };

    // ---- the math on one block held in LDS ----
    // Per-lane LDS byte offsets inside a stage (fixed for the kernel):
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
    auto ld_vt = [&](const char* vb, int ks, int dt) -> bf16x8 {
      const char* a1 = vb + ((v_off1 ^ (uint32_t)(dt << 6)) + ks * 16 * RB);
      const char* a2 = vb + ((v_off2 ^ (uint32_t)(dt << 6)) + (ks * 16 + 8) * RB);
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a1));
      const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(a2));
      const i16x8 av = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
      return __builtin_bit_cast(bf16x8, av);
    };

    auto compute = [&](int k0, const char* kb, const char* vb) {
      const bool needed = wave_live && k0 <= wpos_hi && (W <= 0 || k0 + BK - 1 > wpos_lo - W);
      if (!needed) return;
      const bool full = (k0 + BK - 1 <= wpos_lo) && (W <= 0 || wpos_hi - k0 < W);
      // S^T = K Q^T: two independent 32-key chains, K fragments read one k-step ahead
      f32x16 sacc[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[hf][i] = 0.f;
      bf16x8 a0 = ld_k(kb, 0, 0), a1 = ld_k(kb, 0, 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 n0 = a0, n1 = a1;
        if (ks + 1 < KS) {
          n0 = ld_k(kb, ks + 1, 0);
          n1 = ld_k(kb, ks + 1, 1);
        }
        // keep the next k-step's reads ahead of this k-step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], sacc[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        a0 = n0;
        a1 = n1;
      }
      // first V^T fragment of p.v: independent of p, in flight during the softmax
      bf16x8 va = ld_vt(vb, 0, 0);
      // logits (log2 units after c_eff), mask, block max
      float mx = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sacc[hf][i];
          if (use_cap) {
            // cap * tanh(s * scale / cap) in log2 units, tanh(x) = 1 - 2 / (e^{2x} + 1)
            const float e2 = __builtin_amdgcn_exp2f(s * (c_scale * 2.f * kLog2e / p.cap));
            s = p.cap * kLog2e * (1.f - 2.f * __builtin_amdgcn_rcpf(e2 + 1.f));
          }
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
      // O^T += V^T P^T over four 16-key steps, V^T fragments one step ahead
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int hf = ks >> 1, qq = ks & 1;
        uint4 pw;
        pw.x = pack_bf16(sacc[hf][8 * qq + 0], sacc[hf][8 * qq + 1]);
        pw.y = pack_bf16(sacc[hf][8 * qq + 2], sacc[hf][8 * qq + 3]);
        pw.z = pack_bf16(sacc[hf][8 * qq + 4], sacc[hf][8 * qq + 5]);
        pw.w = pack_bf16(sacc[hf][8 * qq + 6], sacc[hf][8 * qq + 7]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x8 vn = va;
          if (dt + 1 < DT) vn = ld_vt(vb, ks, dt + 1);
          else if (ks + 1 < 4) vn = ld_vt(vb, ks + 1, 0);
          __builtin_amdgcn_sched_barrier(0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          va = vn;
        }
      }
    };

    if constexpr (DIRECT) {
      // two LDS stages: block blk + 1 streams in while block blk is multiplied
      // (unrolled by two so each half names its stage buffer statically)
      if (blk_first < blk_end) {
        ensure_pages(blk_first);
        issue_direct(blk_first, smem);
      }
      for (int blk = blk_first; blk < blk_end; blk += 2) {
        wait_vmem_all();                    // this wave's part of block blk has landed
        __syncthreads();                    // all parts landed; block blk - 1 fully consumed
        if (blk + 1 < blk_end) {
          ensure_pages(blk + 1);
          issue_direct(blk + 1, smem1);
        }
        compute(blk * BK, smem, smem + BLKB);
        if (blk + 1 < blk_end) {
          wait_vmem_all();
          __syncthreads();
          if (blk + 2 < blk_end) {
            ensure_pages(blk + 2);
            issue_direct(blk + 2, smem);
          }
          compute((blk + 1) * BK, smem1, smem1 + BLKB);
        }
      }
    } else {
      if (blk_first < blk_end) {
        ensure_pages(blk_first);
        fetch_staged(blk_first);
      }
      for (int blk = blk_first; blk < blk_end; ++blk) {
        __syncthreads();                    // previous block fully consumed
        stage_staged();
        __syncthreads();                    // block visible to all waves
        if (blk + 1 < blk_end) {
          ensure_pages(blk + 1);
          fetch_staged(blk + 1);
        }
        compute(blk * BK, smem, smem + BLKB);
      }
    }

    // ---- finalise: combine the two half-row sums, sink, 1/l, v_scale ----
    if (wave_live) {
      float l_tot = l_run + __shfl_xor(l_run, 32);
      float f = 1.f;
      if (p.sink) {
        const float sg = p.sink[h] * kLog2e;
        const float mx = fmaxf(m_run, sg);
        f = __builtin_amdgcn_exp2f(m_run - mx);
        l_tot = l_tot * f + __builtin_amdgcn_exp2f(sg - mx);
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

template <typename CT>
hipError_t launch_t(const AttnParams& p, hipStream_t s) {
  long long blocks = (long long)p.lay.max_pf_items * p.Hq;
  if (blocks <= 0) return hipSuccess;
  // persistent grid: the resident workgroups, rounded down to a multiple of 8
  // so that block b and its later units b + grid sit on the same XCD
  static const long long cap64 =
      resident_grid(reinterpret_cast<const void*>(&prefill_kernel<CT, 64>));
  static const long long cap128 =
      resident_grid(reinterpret_cast<const void*>(&prefill_kernel<CT, 128>));
  const long long cap = p.D == 64 ? cap64 : cap128;
  if (blocks > cap) blocks = cap;
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
