// Device helpers shared by the libmoeq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;

// ------------------------------------------------------------ bit casts ----
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// bfloat16 <-> fp32.  fp32 -> bf16 rounds to nearest even (finite inputs).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return u2f(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = f2u(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// fp32 -> OCP E4M3 byte: round to nearest even, saturate to +-448 (E4M3 has no
// infinity), keep the sign (a negative value rounding to zero gives 0x80).
// Finite inputs only.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = f2u(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a >= 0x43E00000u) {                 // |f| >= 448
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {           // |f| < 2^-6: subnormal grid of 2^-9
    mag = uint32_t(rintf(u2f(a) * 512.0f));   // exact scaling, RNE; 8 -> 0x08 = 2^-6
  } else {                                // normal: keep 3 of the 23 mantissa bits, RNE
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    mag = r - (120u << 3);                // rebias exponent 127 -> 7
  }
  return sign | mag;
}

// ----------------------------------------------------- wave reductions ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

}  // namespace moeq
