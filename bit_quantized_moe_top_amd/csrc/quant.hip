// quant_fp8_per_token kernel: one 256-thread workgroup per row.
//
// Pass 1 reads the row and reduces max|x| (wave shuffles, then 4 partials in
// LDS); pass 2 re-reads the row (now in cache), divides by the scale with an
// IEEE division and encodes E4M3 with round-to-nearest-even (fp8_scale and
// fp8_codes8 in front.hpp, shared with the fused front-end kernel).  Each
// thread moves 8 elements per step and writes 8 codes (8 B).
#include "front.hpp"

namespace moeq {

namespace {

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
    load8(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = fp8_scale(amax);
  if (threadIdx.x == 0) scale[m] = s;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    load8(row + c, v);
    *reinterpret_cast<uint2*>(qrow + c) = fp8_codes8(v, s);
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
