// The MFMA-beside-VALU probe (include/rpa_probes.h, rpa_probe_mix and
// rpa_probe_mix_vgpr_acc), shared by probes.hip and probes_vacc.hip: the
// latter is compiled with MFMA accumulators forced into VGPRs, as in the
// attention kernels, where the compiler keeps them in AGPRs here.  Included
// inside each file's anonymous namespace, after its kT, bf16x8 and f32x16.
#ifndef RPA_PROBES_MIX_H_
#define RPA_PROBES_MIX_H_

// MFMA beside VALU work in the same wave, in the shape of the prefill
// kernel's chunks: each of 4 independent v_mfma_f32_32x32x16_bf16 chains is
// followed by NV VALU pairs (v_fma_f32 feeding v_exp_f32 when EXP, else a
// second v_fma_f32) on chains of their own, with scheduling fences keeping
// that order.  4 * iters MFMAs and 8 * NV * iters VALU instructions per wave;
// clocks as in mfma_probe.
template <int NV, bool EXP>
__device__ __forceinline__ void mix_valu(float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float y = fmaf(x[j], 0.999f, -0.5f);
    x[j] = EXP ? __builtin_amdgcn_exp2f(y) : fmaf(y, 0.998f, 0.25f);
  }
}

template <int NV, bool EXP>
__global__ __launch_bounds__(kT) void mix_probe(float* __restrict__ sink,
                                                int64_t* __restrict__ clocks, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int i = 0; i < 16; ++i) c0[i] = c1[i] = c2[i] = c3[i] = 0.f;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.25f + 0.01f * (float)((lane + j) & 31);
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int k = 0; k < iters; ++k) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    mix_valu<NV, EXP>(x);
    __builtin_amdgcn_sched_barrier(0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    mix_valu<NV, EXP>(x);
    __builtin_amdgcn_sched_barrier(0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    mix_valu<NV, EXP>(x);
    __builtin_amdgcn_sched_barrier(0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    mix_valu<NV, EXP>(x);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float* o = sink + ((size_t)blockIdx.x * kT + threadIdx.x) * 16;
  float xs = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) xs += x[j];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = c0[i] + c1[i] + c2[i] + c3[i] + xs;
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + threadIdx.x / 64;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

inline int launch_mix(float* sink, int64_t* clocks, int nv, int exp, int iters, int blocks,
                      void* stream) {
  if (!sink || !clocks || blocks <= 0 || iters < 0 || nv < 0 || nv > 4 || exp < 0 || exp > 1)
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  using K = void (*)(float*, int64_t*, int);
  static const K table[2][5] = {
      {mix_probe<0, false>, mix_probe<1, false>, mix_probe<2, false>, mix_probe<3, false>,
       mix_probe<4, false>},
      {mix_probe<0, true>, mix_probe<1, true>, mix_probe<2, true>, mix_probe<3, true>,
       mix_probe<4, true>}};
  table[exp][nv]<<<blocks, kT, 0, s>>>(sink, clocks, iters);
  return (int)hipGetLastError();
}

#endif  // RPA_PROBES_MIX_H_
