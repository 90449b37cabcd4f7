// quant_fp8_per_token kernels.
//
// Rows of up to 4096 elements: one wave per row (four rows per 256-thread
// workgroup).  The wave loads the whole row into registers (RowQuant in
// front.hpp, 8 elements per chunk, up to 8 chunks per lane), reduces max|x|
// with DPP, and encodes from the registers, so every element is read once.
// Longer rows: one 256-thread workgroup per row, two passes over the row (the
// second from cache).  Both use fp8_scale and fp8_codes8 (common.hpp):
// scale = max|x| / 448 with an IEEE division, codes = RNE(x / scale) to E4M3,
// the same arithmetic as the fused front-end and expert-MLP kernels.
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

template <typename T, int CPL>
__global__ void __launch_bounds__(256)
quant_fp8_wave_kernel(const T* __restrict__ x, int64_t M, int K, int64_t ld_x,
                      uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t m = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (m >= M) return;                                   // wave-uniform
  RowQuant<T, CPL> rq;
  rq.run(x + m * ld_x, K, lane);
  rq.store(q + m * int64_t(K), K, lane);
  if (lane == 0) scale[m] = rq.scale;
}

template <typename T>
hipError_t launch_rows(const T* x, int64_t M, int K, int64_t ld_x, uint8_t* q, float* scale,
                       hipStream_t stream) {
  if (row_quant_cpl(K) != 0) {
    return with_row_quant_cpl(K, [&](auto cpl) {
      constexpr int CPL = decltype(cpl)::value;
      // grid.x holds up to 2^31-1 workgroups of four rows
      const int64_t kMaxRows = int64_t(0x7FFFFFFF) * 4;
      for (int64_t m0 = 0; m0 < M; m0 += kMaxRows) {
        const int64_t rows = (M - m0 < kMaxRows) ? (M - m0) : kMaxRows;
        hipLaunchKernelGGL((quant_fp8_wave_kernel<T, CPL>), dim3(unsigned((rows + 3) / 4)),
                           dim3(256), 0, stream, x + m0 * ld_x, rows, K, ld_x, q + m0 * K,
                           scale + m0);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
      }
      return hipSuccess;
    });
  }
  const int64_t kMaxGrid = 0x7FFFFFFF;
  for (int64_t m0 = 0; m0 < M; m0 += kMaxGrid) {
    const int64_t rows = (M - m0 < kMaxGrid) ? (M - m0) : kMaxGrid;
    hipLaunchKernelGGL(quant_fp8_kernel<T>, dim3(unsigned(rows)), dim3(256), 0, stream,
                       x + m0 * ld_x, K, ld_x, q + m0 * K, scale + m0);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_quant_fp8(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x,
                            uint8_t* q, float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (x_dtype == MOEQ_BF16)
    return launch_rows(static_cast<const uint16_t*>(x), M, K, ld_x, q, scale, stream);
  return launch_rows(static_cast<const float*>(x), M, K, ld_x, q, scale, stream);
}

}  // namespace moeq
