// Device helpers shared by the gfx950 kernels of the MoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a
// quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP FP8 E4M3 byte -> fp32 (exact).  Bit 7 sign, bits 6..3 exponent field
// (bias 7), bits 2..0 mantissa; field 0 holds the subnormals m * 2^-9; the
// all-ones magnitude 0x7F is NaN (the format has no infinities).  One
// formula for both kinds, without branches: (8 [field > 0] + m) *
// 2^(max(field, 1) - 10), the integer converted exactly and scaled by ldexp.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t field = (b >> 3) & 15u, m = b & 7u;
  const float mag = __builtin_amdgcn_ldexpf((float)(m + 8u * min(field, 1u)),
                                            (int)max(field, 1u) - 10);
  const uint32_t bits = (b & 0x7Fu) == 0x7Fu ? 0x7FC00000u : __float_as_uint(mag);
  return __uint_as_float(bits | ((b & 0x80u) << 24));
}

// Clamped SwiGLU on fp32 pre-activations: the gate is bounded from above
// only, the up projection on both sides; silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu_clamped(float g, float u, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g / (1.0f + expf(-g)) * u;
}

// The same with the hardware exponential and reciprocal (about 1 ulp each):
// e^-g = 2^(-g log2 e); a gate far below zero gives 2^+inf = inf, 1/inf = 0.
__device__ __forceinline__ float swiglu_clamped_fast(float g, float u, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Butterfly (xor) reductions: addition is commutative, so every lane ends
// with the same bits, and the order is fixed, so runs repeat exactly.

// 64-bit wave-wide max (every lane ends with the max).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, MOE_WAVE);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, MOE_WAVE);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}
