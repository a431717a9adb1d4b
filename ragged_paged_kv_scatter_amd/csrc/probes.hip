// Measurement probes (include/rpa_probes.h): HBM streaming read and copy,
// a dense bf16 MFMA burn with shader-clock counters, VALU issue-rate chains,
// LDS read / transposed read / write rates and the global -> LDS copy rate.
// They give the roofline figures of the attention kernels a measured ceiling
// beside the published peaks; the attention path never calls them.
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

#include "probes_mix.h"

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

// LDS throughput.  Each wave owns 8 KiB of its workgroup's 32 KiB and runs
// `iters` rounds of 8 instructions over it:
//   op 0: ds_read_b128         lane offset 16 lane + 1024 j   (1 KiB each)
//   op 1: ds_read_b64_tr_b16   lane offset 8 lane + 512 j     (512 B each)
//   op 2: ds_write_b128        lane offset 16 lane + 1024 j   (1 KiB each)
// Contiguous lane addresses, so no bank conflicts.  Read values are kept by
// empty asm statements that take them as operands (no VALU work), and the
// wave's base offset passes through one each round so no access is hoisted
// or merged across rounds.  Clocks as in mfma_probe.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;
typedef u32x4 __attribute__((address_space(3))) * lds_u32x4_ptr;

__global__ __launch_bounds__(kT) void lds_probe(uint32_t* __restrict__ sink,
                                                int64_t* __restrict__ clocks, int op, int iters) {
  __shared__ __attribute__((aligned(1024))) char buf[32768];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 32768 / 16; i += kT)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{(uint32_t)i, (uint32_t)i + 1, (uint32_t)i + 2, (uint32_t)i + 3};
  __syncthreads();
  __attribute__((address_space(3))) char* lds = (__attribute__((address_space(3))) char*)(buf);
  uint32_t off = wave * 8192 + (op == 1 ? lane * 8 : lane * 16);
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  if (op == 0) {
    for (int k = 0; k < iters; ++k) {
      asm volatile("" : "+v"(off));
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *(lds_u32x4_ptr)(lds + off + 1024 * j);
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
    }
  } else if (op == 1) {
    for (int k = 0; k < iters; ++k) {
      asm volatile("" : "+v"(off));
      i16x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(lds + off + 512 * j));
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
    }
  } else {
    const u32x4 val = {(uint32_t)lane, (uint32_t)wave, 7u, 9u};
    for (int k = 0; k < iters; ++k) {
      asm volatile("" : "+v"(off));
#pragma unroll
      for (int j = 0; j < 8; ++j) *(lds_u32x4_ptr)(lds + off + 1024 * j) = val;
      asm volatile("" ::: "memory");
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  __syncthreads();
  sink[(size_t)blockIdx.x * kT + threadIdx.x] = reinterpret_cast<const uint32_t*>(buf)[threadIdx.x * 4];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + wave;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// Global -> LDS copy rate (global_load_lds_dwordx4, the attention kernels'
// block copy).  Each wave copies 8 KiB per round into its own 8 KiB of LDS,
// 8 instructions of 1 KiB, from a source window of `window` bytes that it
// walks round by round, then waits for the round's copies (as a pipeline
// step of the prefill kernel waits for its block).  A window that fits in L2
// measures the L2 -> LDS path.
__global__ __launch_bounds__(kT) void dma_probe(const char* __restrict__ src, uint32_t window_kib,
                                                uint32_t* __restrict__ sink,
                                                int64_t* __restrict__ clocks, int iters) {
  __shared__ __attribute__((aligned(1024))) char buf[32768];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(buf)) + wave * 8192;
  uint32_t kib = (uint32_t)(blockIdx.x * 4 + wave) * 8u % window_kib;
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int k = 0; k < iters; ++k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const char* g = src + (size_t)((kib + j) % window_kib) * 1024 + lane * 16;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(g), "s"(lds0 + j * 1024)
                   : "memory", "m0");
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    kib = (kib + 8) % window_kib;
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  __syncthreads();
  sink[(size_t)blockIdx.x * kT + threadIdx.x] = reinterpret_cast<const uint32_t*>(buf)[threadIdx.x * 4];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + wave;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// MFMA fed from LDS, in the prefill kernel's two patterns, at the residency
// it runs at (launch 2 workgroups of 256 threads per CU):
//   mode 0 (q.k): each v_mfma_f32_32x32x16_bf16 takes its A operand from one
//     ds_read_b128 issued two MFMAs ahead, B from registers, and alternates
//     between 2 accumulators;
//   mode 1 (p.v): each MFMA takes A from two ds_read_b64_tr_b16 issued one
//     MFMA ahead and cycles through 4 accumulators;
//   mode 2: mode 0's pattern with no LDS reads (A from registers);
//   mode 3: mode 0 with 4 accumulators.
// Every wave reads 16 KiB of its workgroup's 32 KiB at contiguous lane
// addresses.  16 MFMAs per round, `iters` rounds; clocks as in mfma_probe.
template <int MODE>
__global__ __launch_bounds__(kT) void lds_mfma_probe(float* __restrict__ sink,
                                                     int64_t* __restrict__ clocks, int iters) {
  __shared__ __attribute__((aligned(1024))) char buf[32768];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 32768 / 16; i += kT)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{0x3c003c00u, 0x3c003c00u, 0u, (uint32_t)i};
  __syncthreads();
  __attribute__((address_space(3))) char* lds = (__attribute__((address_space(3))) char*)(buf);
  uint32_t off = (wave & 1) * 16384 + lane * 16;
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(0.002f * (float)(lane - i));
  f32x16 c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[k][i] = 0.f;
  auto rd128 = [&](int j) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *(lds_u32x4_ptr)(lds + off + ((j & 15) << 10)));
  };
  auto rdtr = [&](int j) -> bf16x8 {
    const uint32_t a = off + ((j & 15) << 10);
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(lds + (a & ~15u)));
    const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(lds + (a & ~15u) + 8));
    const i16x8 v = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a0 = b, a1 = b, a2 = b;
  if constexpr (MODE == 0 || MODE == 3) { a0 = rd128(0); a1 = rd128(1); }
  if constexpr (MODE == 1) a0 = rdtr(0);
  for (int k = 0; k < iters; ++k) {
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      constexpr int NC = (MODE == 1 || MODE == 3) ? 4 : 2;
      if constexpr (MODE == 0 || MODE == 3) {
        a2 = rd128(m + 2);
        __builtin_amdgcn_sched_barrier(0);
        c[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, c[m % NC], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        a0 = a1;
        a1 = a2;
      } else if constexpr (MODE == 1) {
        a1 = rdtr(m + 1);
        __builtin_amdgcn_sched_barrier(0);
        c[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, c[m % NC], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        a0 = a1;
      } else {
        c[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, c[m % NC], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float* o = sink + ((size_t)blockIdx.x * kT + threadIdx.x) * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = c[0][i] + c[1][i] + c[2][i] + c[3][i] + (float)a0[i & 7];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + wave;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// LDS reads beside global -> LDS copies, as in the prefill kernel's steps:
// in every workgroup of 256 threads, waves 0 and 1 run rounds of 8
// ds_read_b128 over their own 8 KiB (mode bit 0) and waves 2 and 3 rounds of
// 8 KiB global -> LDS copies into theirs, from a source window of window_kib
// KiB (mode bit 1).  Every active wave runs rounds until `ticks` of the 100
// MHz constant clock have passed, then writes its round count and shader
// clocks to counts[2 w], counts[2 w + 1].  The read rate with and without
// the copies beside it shows how much the copies' LDS writes slow the reads.
__global__ __launch_bounds__(kT) void lds_dma_probe(const char* __restrict__ src, uint32_t window_kib,
                                                    uint32_t* __restrict__ sink,
                                                    int64_t* __restrict__ counts, int mode,
                                                    int64_t ticks) {
  __shared__ __attribute__((aligned(1024))) char buf[32768];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = threadIdx.x; i < 32768 / 16; i += kT)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const bool reader = wave < 2;
  const bool active = reader ? (mode & 1) != 0 : (mode & 2) != 0;
  int64_t rounds = 0;
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  if (active && reader) {
    __attribute__((address_space(3))) char* lds = (__attribute__((address_space(3))) char*)(buf);
    uint32_t off = wave * 8192 + lane * 16;
    while (__builtin_amdgcn_s_memrealtime() - r0 < ticks) {
      asm volatile("" : "+v"(off));
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *(lds_u32x4_ptr)(lds + off + 1024 * j);
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
      ++rounds;
    }
  } else if (active) {
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(buf)) + wave * 8192;
    uint32_t kib = (uint32_t)(blockIdx.x * 4 + wave) * 8u % window_kib;
    while (__builtin_amdgcn_s_memrealtime() - r0 < ticks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const char* g = src + (size_t)((kib + j) % window_kib) * 1024 + lane * 16;
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(g), "s"(lds0 + j * 1024)
                     : "memory", "m0");
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      kib = (kib + 8) % window_kib;
      ++rounds;
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  sink[(size_t)blockIdx.x * kT + threadIdx.x] = reinterpret_cast<const uint32_t*>(buf)[threadIdx.x * 4];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kT / 64) + wave;
    counts[2 * w] = rounds;
    counts[2 * w + 1] = t1 - t0;
  }
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

int rpa_probe_lds(uint32_t* sink, int64_t* clocks, int op, int iters, int blocks, void* stream) {
  if (!sink || !clocks || blocks <= 0 || iters < 0 || op < 0 || op > 2)
    return (int)hipErrorInvalidValue;
  lds_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(sink, clocks, op, iters);
  return done();
}

int rpa_probe_dma(const void* src, size_t window_bytes, uint32_t* sink, int64_t* clocks, int iters,
                  int blocks, void* stream) {
  if (!src || !sink || !clocks || blocks <= 0 || iters < 0 || window_bytes < 8192 ||
      window_bytes % 1024 != 0 || window_bytes / 1024 > 0xFFFFFFFFull)
    return (int)hipErrorInvalidValue;
  dma_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(src), (uint32_t)(window_bytes / 1024), sink, clocks, iters);
  return done();
}

int rpa_probe_lds_dma(const void* src, size_t window_bytes, uint32_t* sink, int64_t* counts,
                      int mode, int64_t ticks, int blocks, void* stream) {
  if (!src || !sink || !counts || blocks <= 0 || mode < 1 || mode > 3 || ticks <= 0 ||
      window_bytes < 8192 || window_bytes % 1024 != 0 || window_bytes / 1024 > 0xFFFFFFFFull)
    return (int)hipErrorInvalidValue;
  lds_dma_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(src), (uint32_t)(window_bytes / 1024), sink, counts, mode, ticks);
  return done();
}

int rpa_probe_mix(float* sink, int64_t* clocks, int nv, int exp, int iters, int blocks,
                  void* stream) {
  return launch_mix(sink, clocks, nv, exp, iters, blocks, stream);
}

int rpa_probe_lds_mfma(float* sink, int64_t* clocks, int mode, int iters, int blocks,
                       void* stream) {
  if (!sink || !clocks || blocks <= 0 || iters < 0 || mode < 0 || mode > 3)
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  using K = void (*)(float*, int64_t*, int);
  static const K table[4] = {lds_mfma_probe<0>, lds_mfma_probe<1>, lds_mfma_probe<2>,
                             lds_mfma_probe<3>};
  table[mode]<<<blocks, kT, 0, s>>>(sink, clocks, iters);
  return done();
}

int rpa_probe_valu(float* sink, int op, int iters, int blocks, void* stream) {
  if (!sink || blocks <= 0 || iters < 0 || op < 0 || op > 2) return (int)hipErrorInvalidValue;
  valu_probe<<<blocks, kT, 0, static_cast<hipStream_t>(stream)>>>(sink, op, iters);
  return done();
}

}  // extern "C"
