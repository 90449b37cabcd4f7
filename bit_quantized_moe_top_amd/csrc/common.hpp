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

// 8 bf16 values (16 bytes, little-endian) -> fp32
__device__ __forceinline__ void bf16x8_to_f32(const uint4& u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = u2f(w[i] << 16);
    v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
  }
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
// Cross-lane steps use DPP (a VALU operand modifier, no LDS round trip):
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror combine within
// each 16-lane row; row_bcast15 / row_bcast31 (restricted to rows 1,3 / 2,3)
// carry rows into rows; lane 63 then holds the wave-wide result, which
// readlane broadcasts.  Lanes a step does not write return `old`.
constexpr int kDppQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppRowShr = 0x110;         // + n: row_shr:n

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float src) {
  return __builtin_bit_cast(float, dpp<CTRL, ROW_MASK>(__builtin_bit_cast(int, old),
                                                       __builtin_bit_cast(int, src)));
}
__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// wave-wide combine of op over all 64 lanes (ident: op's identity), result in
// every lane; the combination order is fixed, so results are deterministic
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op, T ident) {
  v = op(v, dpp<kDppQuadSwap1>(ident, v));
  v = op(v, dpp<kDppQuadSwap2>(ident, v));
  v = op(v, dpp<kDppRowHalfMirror>(ident, v));
  v = op(v, dpp<kDppRowMirror>(ident, v));
  v = op(v, dpp<kDppRowBcast15, 0xA>(ident, v));
  v = op(v, dpp<kDppRowBcast31, 0xC>(ident, v));
  return readlane(v, 63);
}
__device__ __forceinline__ float wave_max(float v) {   // for v >= 0 (magnitudes)
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); }, 0.0f);
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; }, 0.0f);
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp<kDppRowShr + 1>(0, v);
  v += dpp<kDppRowShr + 2>(0, v);
  v += dpp<kDppRowShr + 4>(0, v);
  v += dpp<kDppRowShr + 8>(0, v);
  v += dpp<kDppRowBcast15, 0xA>(0, v);
  v += dpp<kDppRowBcast31, 0xC>(0, v);
  return v;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------ FP8 (E4M3) codes ----
// scale = fp32(amax / 448) (IEEE division)
__device__ __forceinline__ float fp8_scale(float amax) { return __fdiv_rn(amax, 448.0f); }

// E4M3 codes of four values in [-448, 448], packed little-endian: the gfx950
// conversion (round to nearest even, sign kept) equals f32_to_e4m3 there.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// True where E4M3 rounding of a value within a few ulp of q may differ from
// that of q: within 8 ulp of a rounding midpoint (the 20 fp32 mantissa bits
// below E4M3's 3 are near 0x80000) or in E4M3's subnormal range (|q| < 2^-6).
// (Bitwise operators, not && / ||: the test is evaluated for every value and
// must not turn into branches.)
__device__ __forceinline__ bool e4m3_rounding_close(float q) {
  const uint32_t a = f2u(q) & 0x7FFFFFFFu;
  return ((a - 1u) < 0x3C7FFFFFu) | (((a & 0xFFFFFu) - 0x7FFF8u) <= 0x10u);
}

// 8 codes of x / s packed little-endian: E4M3 (round to nearest even,
// saturating) of the IEEE fp32 quotient fl32(x / s).  The quotients are formed
// as x * (1 / s) with the hardware reciprocal, within 3 ulp of fl32(x / s);
// where that could round to a different code (e4m3_rounding_close) the lane
// takes the IEEE division instead, so the codes always equal those of the
// division.  s <= 0 gives zeros.
__device__ __forceinline__ uint2 fp8_codes8(const float (&v)[8], float s) {
  if (!(s > 0.0f)) return make_uint2(0u, 0u);
  float q[8];
  bool exact = !(s >= 0x1p-120f && s <= 0x1p120f);   // reciprocal normal and accurate
  if (!exact) {
    const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      q[i] = v[i] * rs;
      exact = exact | e4m3_rounding_close(q[i]);
    }
  }
  if (exact) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __fdiv_rn(v[i], s);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(q[i], -448.0f), 448.0f);
  return make_uint2(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]));
}


// E4M3 code (low byte) of x / s, exactly as fp8_codes8 for one value.
__device__ __forceinline__ uint32_t fp8_code1(float v, float s) {
  if (!(s > 0.0f)) return 0u;
  float q;
  if (s >= 0x1p-120f && s <= 0x1p120f) {
    q = v * __builtin_amdgcn_rcpf(s);
    if (e4m3_rounding_close(q)) q = __fdiv_rn(v, s);
  } else {
    q = __fdiv_rn(v, s);
  }
  q = fminf(fmaxf(q, -448.0f), 448.0f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false)) & 0xFFu;
}


}  // namespace moeq
