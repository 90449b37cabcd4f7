// moe_route_topk kernel: one wave64 per token (the per-token routine is
// route_token_wave in front.hpp).
//
// moe_router_logits kernels: logits[t, e] = sum_h x[t, h] * Wr[e, h] with fp32
// accumulation (fused multiply-adds).
//  * T <= kRouterGemvT (decode): one wave per expert; lane l accumulates the
//    4-element pieces h = 4 (l + 64 i) for every token in registers, then a DPP
//    wave sum per token.  The router weights (E x H fp32) are streamed once.
//  * larger T: 64 x 64 output tiles per 256-thread workgroup, 16-wide K chunks
//    staged in LDS (transposed, so a thread reads its 4 rows / 4 columns as one
//    16-byte word), the next chunk's global loads in flight during the current
//    chunk's FMAs; each thread owns a 4 x 4 block and sums k in order.
#include "front.hpp"

namespace moeq {

namespace {

template <int NS>
__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
                  int k, int renormalize, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                   // whole wave exits together
  route_token_wave<NS>(logits + int64_t(t) * E, bias, E, k, renormalize, ids + int64_t(t) * k,
                       w + int64_t(t) * k, lane);
}

constexpr int kRouterGemvT = 16;

template <typename XT>
__device__ __forceinline__ float4 load4(const XT* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(u2f(u.x << 16), u2f(u.x & 0xFFFF0000u), u2f(u.y << 16), u2f(u.y & 0xFFFF0000u));
}

template <typename XT>
__global__ void __launch_bounds__(256)
router_gemv_kernel(const XT* __restrict__ x, int T, int H, const float* __restrict__ wr, int E,
                   float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;                                   // wave-uniform
  const float* wrow = wr + int64_t(e) * H;
  float acc[kRouterGemvT];
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) acc[t] = 0.0f;
  for (int h = 4 * lane; h < H; h += 4 * kWave) {
    const float4 w4 = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int t = 0; t < kRouterGemvT; ++t) {
      if (t < T) {
        const float4 x4 = load4(x + int64_t(t) * H + h);
        acc[t] = fmaf(x4.x, w4.x, acc[t]);
        acc[t] = fmaf(x4.y, w4.y, acc[t]);
        acc[t] = fmaf(x4.z, w4.z, acc[t]);
        acc[t] = fmaf(x4.w, w4.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) logits[int64_t(t) * E + e] = v;
    }
  }
}

constexpr int kRtTile = 64, kRtK = 16, kRtPad = 4;

template <typename XT>
__global__ void __launch_bounds__(256)
router_gemm_kernel(const XT* __restrict__ x, int T, int H, const float* __restrict__ wr, int E,
                   float* __restrict__ logits) {
  __shared__ __align__(16) float Xs[kRtK][kRtTile + kRtPad];
  __shared__ __align__(16) float Ws[kRtK][kRtTile + kRtPad];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRtTile, e0 = blockIdx.y * kRtTile;
  // loader: thread -> (row tid / 4, k piece 4 (tid % 4)) of the 64 x 16 chunk
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const bool x_ok = t0 + lr < T, w_ok = e0 + lr < E;
  const XT* xsrc = x + int64_t(x_ok ? t0 + lr : 0) * H + lk;
  const float* wsrc = wr + int64_t(w_ok ? e0 + lr : 0) * H + lk;
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 xn = x_ok ? load4(xsrc) : zero;
  float4 wn = w_ok ? *reinterpret_cast<const float4*>(wsrc) : zero;
  // compute: thread -> rows 4 (tid / 16) .., columns 4 (tid % 16) ..
  const int cr = (tid >> 4) * 4, cc = (tid & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < H; k0 += kRtK) {
    Xs[lk][lr] = xn.x; Xs[lk + 1][lr] = xn.y; Xs[lk + 2][lr] = xn.z; Xs[lk + 3][lr] = xn.w;
    Ws[lk][lr] = wn.x; Ws[lk + 1][lr] = wn.y; Ws[lk + 2][lr] = wn.z; Ws[lk + 3][lr] = wn.w;
    __syncthreads();
    if (k0 + kRtK < H) {                               // next chunk in flight
      xn = x_ok ? load4(xsrc + k0 + kRtK) : zero;
      wn = w_ok ? *reinterpret_cast<const float4*>(wsrc + k0 + kRtK) : zero;
    }
#pragma unroll
    for (int k = 0; k < kRtK; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&Xs[k][cr]);
      const float4 b = *reinterpret_cast<const float4*>(&Ws[k][cc]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + cr + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + cc + j < E) logits[int64_t(t) * E + e0 + cc + j] = acc[i][j];
  }
}

template <typename XT>
hipError_t launch_router_typed(const XT* x, int T, int H, const float* wr, int E, float* logits,
                               hipStream_t stream) {
  if (T <= kRouterGemvT) {
    hipLaunchKernelGGL(router_gemv_kernel<XT>, dim3((E + 3) / 4), dim3(256), 0, stream, x, T, H,
                       wr, E, logits);
  } else {
    const dim3 grid(unsigned((T + kRtTile - 1) / kRtTile), unsigned((E + kRtTile - 1) / kRtTile));
    hipLaunchKernelGGL(router_gemm_kernel<XT>, grid, dim3(256), 0, stream, x, T, H, wr, E,
                       logits);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const void* x, int x_dtype, int T, int H, const float* wr, int E,
                                float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (x_dtype == MOEQ_BF16)
    return launch_router_typed(static_cast<const uint16_t*>(x), T, H, wr, E, logits, stream);
  return launch_router_typed(static_cast<const float*>(x), T, H, wr, E, logits, stream);
}

hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int renormalize, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  with_route_slots(E, [&](auto ns) {
    hipLaunchKernelGGL(route_topk_kernel<decltype(ns)::value>, dim3((T + 3) / 4), dim3(256), 0,
                       stream, logits, bias, T, E, k, renormalize, ids, w);
    return 0;
  });
  return hipGetLastError();
}

}  // namespace moeq
