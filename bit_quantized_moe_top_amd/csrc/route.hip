// moe_route_topk kernel: one wave64 per token (the per-token routine is
// route_token_wave in front.hpp).
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

}  // namespace

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
