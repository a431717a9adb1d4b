// Device helpers: element conversions and wavefront reductions for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpa {

// ---- element types --------------------------------------------------------
// bf16 and e4m3 values travel as raw bits (uint16_t / uint8_t).

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Low / high bf16 of a packed 32-bit word.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even; NaN stays a quiet NaN of the same sign.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP e4m3fn code -> float (exact).  Exponent bias 7, subnormals m/8 * 2^-6,
// code 0x7F / 0xFF is NaN, there is no infinity.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t em = c & 0x7fu;
  if (em == 0x7fu) return __uint_as_float(s | 0x7fc00000u);
  if (em < 8u) {  // subnormal: m * 2^-9
    return __uint_as_float(s | __float_as_uint((float)em * 0.001953125f));
  }
  // normal: rebias exponent 7 -> 127 (add 120) and widen the mantissa 3 -> 23 bits
  return __uint_as_float(s | ((em + (120u << 3)) << 20));
}

// float (the already-scaled y = x / scale) -> e4m3fn code: clamp to +-448 then
// round to nearest, ties to even.  NaN -> 0x7F with the sign of the input.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;         // |y| >= 448 (incl. inf): clamp
  if (a < 0x3c800000u) {                             // |y| < 2^-6: subnormal grid m * 2^-9
    float q = __uint_as_float(a) * 512.0f;           // exact (power-of-two scaling)
    uint32_t m = (uint32_t)__builtin_rintf(q);       // round half to even; 8 = min normal
    return sign | m;
  }
  int32_t e = (int32_t)(a >> 23) - 127;              // -6 .. 8
  uint32_t mant = a & 0x7fffffu;
  uint32_t r = mant >> 20;                           // top 3 mantissa bits
  uint32_t rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  uint32_t code = ((uint32_t)(e + 7) << 3) + r;      // a carry out of r bumps the exponent
  if (code > 0x7eu) code = 0x7eu;                    // cannot exceed 448 after the clamp
  return sign | code;
}

// ---- wavefront exchange ---------------------------------------------------
// Value of lane (lane ^ mask) for a power-of-two mask < 64.
template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(MASK > 0 && MASK < 64 && (MASK & (MASK - 1)) == 0, "power of two");
  if constexpr (MASK == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  } else if constexpr (MASK == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  } else if constexpr (MASK == 4 || MASK == 8 || MASK == 16) {
    // ds_swizzle bit mode: and_mask 0x1F, xor_mask = MASK (within 32-lane halves)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (MASK << 10)));
  } else {
    return __shfl_xor(v, 32);
  }
}

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// the group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += lane_xor<1>(v);
  if constexpr (N >= 4) v += lane_xor<2>(v);
  if constexpr (N >= 8) v += lane_xor<4>(v);
  if constexpr (N >= 16) v += lane_xor<8>(v);
  if constexpr (N >= 32) v += lane_xor<16>(v);
  if constexpr (N >= 64) v += lane_xor<32>(v);
  return v;
}

// Sum / max across lanes that differ only in bits [log2(FROM), 6) of the lane id
// (i.e. over the 64/FROM groups of FROM lanes), result in every lane.
template <int FROM>
__device__ __forceinline__ float cross_sum(float v) {
  if constexpr (FROM <= 1) v += lane_xor<1>(v);
  if constexpr (FROM <= 2) v += lane_xor<2>(v);
  if constexpr (FROM <= 4) v += lane_xor<4>(v);
  if constexpr (FROM <= 8) v += lane_xor<8>(v);
  if constexpr (FROM <= 16) v += lane_xor<16>(v);
  if constexpr (FROM <= 32) v += lane_xor<32>(v);
  return v;
}

template <int FROM>
__device__ __forceinline__ float cross_max(float v) {
  if constexpr (FROM <= 1) v = fmaxf(v, lane_xor<1>(v));
  if constexpr (FROM <= 2) v = fmaxf(v, lane_xor<2>(v));
  if constexpr (FROM <= 4) v = fmaxf(v, lane_xor<4>(v));
  if constexpr (FROM <= 8) v = fmaxf(v, lane_xor<8>(v));
  if constexpr (FROM <= 16) v = fmaxf(v, lane_xor<16>(v));
  if constexpr (FROM <= 32) v = fmaxf(v, lane_xor<32>(v));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace rpa
