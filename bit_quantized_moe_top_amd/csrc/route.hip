// moe_route_topk kernel: one wave64 per token.
//
// Each lane keeps up to E/64 scores in registers (expert e lives in lane e % 64,
// slot e / 64).  k rounds of a wave-wide argmax select the experts best first;
// the comparison orders by score descending and expert index ascending, so ties
// go to the lower index and the result is independent of reduction order.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

constexpr int kMaxSlots = MOEQ_MAX_EXPERTS / kWave;   // 16

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
                  int k, int renormalize, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                   // whole wave exits together
  const float* row = logits + int64_t(t) * E;
  float s[kMaxSlots];
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    const int e = j * kWave + lane;
    float v = -INFINITY;
    if (e < E) {
      v = row[e];
      if (bias) v = v + bias[e];
    }
    s[j] = v;
  }
  uint32_t used = 0;                                    // slots already selected (bit j)
  float sel_v[MOEQ_MAX_TOPK];
  int sel_e[MOEQ_MAX_TOPK];
#pragma unroll
  for (int r = 0; r < MOEQ_MAX_TOPK; ++r) {
    sel_v[r] = -INFINITY;
    sel_e[r] = 0;
    if (r >= k) continue;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      const int e = j * kWave + lane;
      if (e < E && !((used >> j) & 1u) && better(s[j], e, bv, bi)) { bv = s[j]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
    sel_v[r] = bv;
    sel_e[r] = bi;
  }
  const float smax = sel_v[0];
  float den = 0.0f;
  if (renormalize) {
#pragma unroll
    for (int r = 0; r < MOEQ_MAX_TOPK; ++r)
      if (r < k) den += expf(sel_v[r] - smax);
  } else {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j)
      if (j * kWave + lane < E) part += expf(s[j] - smax);
    den = wave_sum(part);
  }
  float v = sel_v[0];
  int e = sel_e[0];
#pragma unroll
  for (int r = 1; r < MOEQ_MAX_TOPK; ++r)
    if (r == lane) { v = sel_v[r]; e = sel_e[r]; }
  if (lane < k) {
    ids[int64_t(t) * k + lane] = e;
    w[int64_t(t) * k + lane] = expf(v - smax) / den;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int renormalize, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(256), 0, stream, logits, bias, T, E, k,
                     renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace moeq
