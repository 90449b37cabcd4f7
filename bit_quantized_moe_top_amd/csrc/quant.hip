// quant_fp8_per_token kernel: one 256-thread workgroup per row.
//
// Pass 1 reads the row and reduces max|x| (wave shuffles, then 4 partials in
// LDS); pass 2 re-reads the row (now in cache), divides by the scale with an
// IEEE division and encodes E4M3 with round-to-nearest-even.  Each thread moves
// 8 elements (16 B of bf16 / 32 B of fp32) per step and writes 8 codes (8 B).
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

template <typename T>
struct Load8;

template <>
struct Load8<uint16_t> {
  static __device__ __forceinline__ void run(const uint16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = u2f(w[i] << 16);
      v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
  }
};

template <>
struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T>
__global__ void __launch_bounds__(256)
quant_fp8_kernel(const T* __restrict__ x, int K, int64_t ld_x, uint8_t* __restrict__ q,
                 float* __restrict__ scale) {
  __shared__ float part[4];
  const int64_t m = blockIdx.x;
  const T* row = x + m * ld_x;
  uint8_t* qrow = q + m * int64_t(K);
  float amax = 0.0f;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    Load8<T>::run(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = __fdiv_rn(amax, 448.0f);
  if (threadIdx.x == 0) scale[m] = s;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    uint32_t lo = 0, hi = 0;
    if (s > 0.0f) {
      float v[8];
      Load8<T>::run(row + c, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= f32_to_e4m3(__fdiv_rn(v[i], s)) << (8 * i);
        hi |= f32_to_e4m3(__fdiv_rn(v[4 + i], s)) << (8 * i);
      }
    }
    *reinterpret_cast<uint2*>(qrow + c) = make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_quant_fp8(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x,
                            uint8_t* q, float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // grid.x holds up to 2^31-1 workgroups; larger M is split into several launches
  const int64_t kMaxGrid = 0x7FFFFFFF;
  for (int64_t m0 = 0; m0 < M; m0 += kMaxGrid) {
    const int64_t rows = (M - m0 < kMaxGrid) ? (M - m0) : kMaxGrid;
    if (x_dtype == MOEQ_BF16) {
      hipLaunchKernelGGL(quant_fp8_kernel<uint16_t>, dim3(unsigned(rows)), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(x) + m0 * ld_x, K, ld_x, q + m0 * K,
                         scale + m0);
    } else {
      hipLaunchKernelGGL(quant_fp8_kernel<float>, dim3(unsigned(rows)), dim3(256), 0, stream,
                         static_cast<const float*>(x) + m0 * ld_x, K, ld_x, q + m0 * K,
                         scale + m0);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moeq
