// quant_fp8_per_token kernels.
//
// Rows of up to 4096 elements: one wave per row (four rows per 256-thread
// workgroup); where K is a multiple of 1024 (and q 16-byte aligned) each lane
// takes pairs of adjacent chunks and stores 16 bytes at a time
// (quant_fp8_pair_kernel: 18.6 against 20.7 us for 12288 rows of 2048).  The wave loads the whole row into registers (RowQuant in
// front.hpp, 8 elements per chunk, up to 8 chunks per lane), reduces max|x|
// with DPP, and encodes from the registers, so every element is read once.
// Longer rows: one 256-thread workgroup per row, two passes over the row (the
// second from cache).  Both use fp8_scale and fp8_codes8 (common.hpp):
// scale = max|x| / 448 with an IEEE division, codes = RNE(x / scale) to E4M3,
// the same arithmetic as the fused front-end and expert-MLP kernels.
//
// Also here: the conversion of row-scaled E4M3FNUZ expert weights to row-scaled
// OCP E4M3 (moe_requant_fp8_fnuz), the same row quantization applied to the
// weights fl32(s * fnuz(b)).
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

// One wave per row with each lane taking pairs of adjacent 8-element chunks
// (K % 1024 == 0, K <= 4096): a lane's codes for 16 consecutive elements leave
// in one 16-byte store, against two 8-byte stores when chunks are interleaved.
template <typename T, int PPL>
__global__ void __launch_bounds__(256)
quant_fp8_pair_kernel(const T* __restrict__ x, int64_t M, int K, int64_t ld_x,
                      uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t m = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (m >= M) return;                                   // wave-uniform
  const T* row = x + m * ld_x;
  XChunk<T> xc[2 * PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    const int e0 = (lane + kWave * i) * 16;
    xc[2 * i].load(row + e0);
    xc[2 * i + 1].load(row + e0 + 8);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 2 * PPL; ++i) {
    float v[8];
    xc[i].values(v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  const float s = fp8_scale(wave_max(amax));
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    float v0[8], v1[8];
    xc[2 * i].values(v0);
    xc[2 * i + 1].values(v1);
    const uint2 c0 = fp8_codes8(v0, s), c1 = fp8_codes8(v1, s);
    *reinterpret_cast<uint4*>(q + m * int64_t(K) + (lane + kWave * i) * 16) =
        make_uint4(c0.x, c0.y, c1.x, c1.y);
  }
  if (lane == 0) scale[m] = s;
}

template <typename T>
hipError_t launch_rows(const T* x, int64_t M, int K, int64_t ld_x, uint8_t* q, float* scale,
                       hipStream_t stream) {
  if (K % 1024 == 0 && K <= 4096 && (reinterpret_cast<uintptr_t>(q) & 15) == 0) {
    const int64_t kMaxRows = int64_t(0x7FFFFFFF) * 4;
    for (int64_t m0 = 0; m0 < M; m0 += kMaxRows) {
      const int64_t rows = (M - m0 < kMaxRows) ? (M - m0) : kMaxRows;
      const dim3 grid(unsigned((rows + 3) / 4));
      switch (K / 1024) {
        case 1: hipLaunchKernelGGL((quant_fp8_pair_kernel<T, 1>), grid, dim3(256), 0, stream,
                                   x + m0 * ld_x, rows, K, ld_x, q + m0 * K, scale + m0); break;
        case 2: hipLaunchKernelGGL((quant_fp8_pair_kernel<T, 2>), grid, dim3(256), 0, stream,
                                   x + m0 * ld_x, rows, K, ld_x, q + m0 * K, scale + m0); break;
        case 3: hipLaunchKernelGGL((quant_fp8_pair_kernel<T, 3>), grid, dim3(256), 0, stream,
                                   x + m0 * ld_x, rows, K, ld_x, q + m0 * K, scale + m0); break;
        default: hipLaunchKernelGGL((quant_fp8_pair_kernel<T, 4>), grid, dim3(256), 0, stream,
                                    x + m0 * ld_x, rows, K, ld_x, q + m0 * K, scale + m0); break;
      }
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  }
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

// ------------------------------------------- E4M3FNUZ rows -> OCP E4M3 rows
// Value of an E4M3FNUZ byte (exponent bias 8, no negative zero); 0x80, the
// format's only NaN, is read as +0.  Normal bytes become an fp32 with the
// exponent rebiased (+119) and the 3 mantissa bits at the top of the fp32
// mantissa; subnormal bytes are m * 2^-10.  Exact.
__device__ __forceinline__ float fnuz_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  const float mag = e ? u2f(((e + 119u) << 23) | (m << 20)) : float(m) * 0x1p-10f;
  return ((b & 0x80u) && (b & 0x7Fu)) ? -mag : mag;
}

// the 8 weights of chunk `raw`: fl32(s * fnuz(b)), one rounding each
__device__ __forceinline__ void fnuz_weights8(const uint2& raw, float s, float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = s * fnuz_value((raw.x >> (8 * j)) & 0xFFu);
    v[4 + j] = s * fnuz_value((raw.y >> (8 * j)) & 0xFFu);
  }
}

// one wave per row (K <= 4096): the row's bytes stay in registers
template <int CPL>
__global__ void __launch_bounds__(256)
requant_fnuz_wave_kernel(const uint8_t* __restrict__ wf, const float* __restrict__ sf, int64_t rows,
                         int K, uint8_t* __restrict__ wq, float* __restrict__ sq) {
  const int lane = threadIdx.x & 63;
  const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                                // wave-uniform
  const int chunks = K >> 3;
  const float s = sf[r];
  uint2 raw[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    if (lane + kWave * i < chunks)
      raw[i] = *reinterpret_cast<const uint2*>(wf + r * K + (lane + kWave * i) * 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (lane + kWave * i < chunks) {
      float v[8];
      fnuz_weights8(raw[i], s, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
  }
  const float s2 = fp8_scale(wave_max(amax));
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (lane + kWave * i < chunks) {
      float v[8];
      fnuz_weights8(raw[i], s, v);
      *reinterpret_cast<uint2*>(wq + r * K + (lane + kWave * i) * 8) = fp8_codes8(v, s2);
    }
  }
  if (lane == 0) sq[r] = s2;
}

// longer rows: one workgroup per row, two passes
__global__ void __launch_bounds__(256)
requant_fnuz_kernel(const uint8_t* __restrict__ wf, const float* __restrict__ sf, int K,
                    uint8_t* __restrict__ wq, float* __restrict__ sq) {
  __shared__ float part[4];
  const int64_t r = blockIdx.x;
  const float s = sf[r];
  float amax = 0.0f;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    fnuz_weights8(*reinterpret_cast<const uint2*>(wf + r * K + c), s, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  const float s2 = fp8_scale(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])));
  if (threadIdx.x == 0) sq[r] = s2;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    fnuz_weights8(*reinterpret_cast<const uint2*>(wf + r * K + c), s, v);
    *reinterpret_cast<uint2*>(wq + r * K + c) = fp8_codes8(v, s2);
  }
}

}  // namespace

hipError_t launch_requant_fnuz(const uint8_t* w_fnuz, const float* s_fnuz, int64_t rows, int K,
                               uint8_t* w_ocp, float* s_ocp, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (row_quant_cpl(K) != 0) {
    return with_row_quant_cpl(K, [&](auto cpl) {
      constexpr int CPL = decltype(cpl)::value;
      const int64_t kMaxRows = int64_t(0x7FFFFFFF) * 4;
      for (int64_t r0 = 0; r0 < rows; r0 += kMaxRows) {
        const int64_t n = (rows - r0 < kMaxRows) ? (rows - r0) : kMaxRows;
        hipLaunchKernelGGL((requant_fnuz_wave_kernel<CPL>), dim3(unsigned((n + 3) / 4)), dim3(256),
                           0, stream, w_fnuz + r0 * K, s_fnuz + r0, n, K, w_ocp + r0 * K,
                           s_ocp + r0);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
      }
      return hipSuccess;
    });
  }
  const int64_t kMaxGrid = 0x7FFFFFFF;
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
    const int64_t n = (rows - r0 < kMaxGrid) ? (rows - r0) : kMaxGrid;
    hipLaunchKernelGGL(requant_fnuz_kernel, dim3(unsigned(n)), dim3(256), 0, stream,
                       w_fnuz + r0 * K, s_fnuz + r0, K, w_ocp + r0 * K, s_ocp + r0);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_quant_fp8(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x,
                            uint8_t* q, float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (x_dtype == MOEQ_BF16)
    return launch_rows(static_cast<const uint16_t*>(x), M, K, ld_x, q, scale, stream);
  return launch_rows(static_cast<const float*>(x), M, K, ld_x, q, scale, stream);
}

}  // namespace moeq
