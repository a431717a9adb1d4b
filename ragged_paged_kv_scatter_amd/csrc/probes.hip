// Measurement probes (include/rpa_probes.h): HBM streaming read and copy,
// a dense bf16 MFMA burn with shader-clock counters, and VALU issue-rate
// chains.  They give the roofline figures of the attention kernels a measured
// ceiling beside the published peaks; the attention path never calls them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa_probes.h"

namespace {

constexpr int kT = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kT) void read_probe(const u32x4* __restrict__ src, size_t n16,
                                                 uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kT;
  size_t i = (size_t)blockIdx.x * kT + threadIdx.x;
  uint32_t acc = 0;
  // four loads in flight per lane
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(size_t)blockIdx.x * kT + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kT) void copy_probe(const u32x4* __restrict__ src,
                                                 u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kT;
  size_t i = (size_t)blockIdx.x * kT + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kT) void mfma_probe(float* __restrict__ sink,
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
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int k = 0; k < iters; ++k) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float* o = sink + ((size_t)blockIdx.x * kT + threadIdx.x) * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + threadIdx.x / 64;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(kT) void valu_probe(float* __restrict__ sink, int op, int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.01f * (float)((threadIdx.x + j) & 31);
  if (op == 0) {
    // x -> 2^-x: a stable chain of one v_exp_f32 (the negation is a free modifier)
    for (int k = 0; k < iters; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  } else if (op == 1) {
    for (int k = 0; k < iters; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_rcpf(x[j]);
  } else {
    for (int k = 0; k < iters; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], 0.999f, 0.001f);
  }
  float* o = sink + ((size_t)blockIdx.x * kT + threadIdx.x) * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = x[j];
}

int done() { return (int)hipGetLastError(); }

}  // namespace

extern "C" {

int rpa_probe_read(const void* src, size_t n16, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || blocks <= 0) return (int)hipErrorInvalidValue;
  read_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), n16, sink);
  return done();
}

int rpa_probe_copy(const void* src, void* dst, size_t n16, int blocks, void* stream) {
  if (!src || !dst || blocks <= 0) return (int)hipErrorInvalidValue;
  copy_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return done();
}

int rpa_probe_mfma(float* sink, int64_t* clocks, int iters, int blocks, void* stream) {
  if (!sink || !clocks || blocks <= 0 || iters < 0) return (int)hipErrorInvalidValue;
  mfma_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(sink, clocks, iters);
  return done();
}

int rpa_probe_valu(float* sink, int op, int iters, int blocks, void* stream) {
  if (!sink || blocks <= 0 || iters < 0 || op < 0 || op > 2) return (int)hipErrorInvalidValue;
  valu_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(sink, op, iters);
  return done();
}

}  // extern "C"
