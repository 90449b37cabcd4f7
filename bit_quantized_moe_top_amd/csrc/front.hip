// moe_route_quant_permute: the layer's front end (routing, FP8 quantization of
// x, permutation plan and gather) as one launch for small batches.
//
// At decode-sized T the four separate launches are almost pure latency (a few
// microseconds each for a few kilobytes of work).  One 1024-thread workgroup
// does all of it: waves route one token each, 16/T waves quantize each token's
// row, the workgroup builds
// the plan from the expert ids it keeps in LDS, and the waves then copy the
// routed rows into plan order.  The arithmetic is the shared front.hpp code, so
// the results are bit-identical to the separate calls.
#include "front.hpp"

namespace moeq {

namespace {

template <typename XT>
__global__ void __launch_bounds__(kPlanThreads)
front_small_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
                   int k, int renormalize, const XT* __restrict__ x, int H, int32_t* ids, float* w,
                   uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, int32_t* plan) {
  extern __shared__ int smem[];           // plan_build_workgroup's E * 17 ints, then R ids
  int* s_ids = smem + E * (1 + kPlanWaves);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;

  for (int t = wave; t < T; t += kPlanWaves) {
    const int e = route_token_wave(logits + int64_t(t) * E, bias, E, k, renormalize,
                                   ids + int64_t(t) * k, w + int64_t(t) * k, lane);
    if (lane < k) s_ids[t * k + lane] = e;
  }
  __shared__ float s_part[kPlanWaves];
  quant_rows_workgroup<XT>(x, T, H, x_q, x_s, s_part);
  __threadfence_block();
  __syncthreads();

  plan_build_workgroup([&](int r) { return s_ids[r]; }, T, k, E, plan, smem);
  __threadfence_block();
  __syncthreads();

  // gather: wave-strided over the placed rows, 16 bytes per lane per step
  const PlanView pv = plan_view(plan, E, R);
  const int n_rows = pv.offsets[E];
  for (int p = wave; p < n_rows; p += kPlanWaves) {
    const int t = pv.sorted_rows[p] / k;
    const uint4* src = reinterpret_cast<const uint4*>(x_q + int64_t(t) * H);
    uint4* dst = reinterpret_cast<uint4*>(xp_q + int64_t(p) * H);
    for (int c = lane; c < H / 16; c += kWave) dst[c] = src[c];
    if (lane == 0) xp_s[p] = x_s[t];
  }
}

}  // namespace

hipError_t launch_front(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, const void* x, int x_dtype, int H, int32_t* ids, float* w,
                        uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, void* plan,
                        hipStream_t stream) {
  hipError_t err;
  if (T > kFrontSmallT) {
    if ((err = launch_route_topk(logits, bias, T, E, k, renormalize, ids, w, stream)) != hipSuccess)
      return err;
    if ((err = launch_quant_fp8(x, x_dtype, T, H, H, x_q, x_s, stream)) != hipSuccess) return err;
    return launch_permute(ids, T, k, E, x_q, x_s, H, xp_q, xp_s, plan, stream);
  }
  const size_t lds = (size_t(E) * (1 + kPlanWaves) + size_t(T) * k) * sizeof(int);
  int32_t* p = static_cast<int32_t*>(plan);
  if (x_dtype == MOEQ_BF16) {
    auto fn = front_small_kernel<uint16_t>;
    if (lds > 64 * 1024 &&
        (err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(lds))) != hipSuccess)
      return err;
    hipLaunchKernelGGL(fn, dim3(1), dim3(kPlanThreads), lds, stream, logits, bias, T, E, k,
                       renormalize, static_cast<const uint16_t*>(x), H, ids, w, x_q, x_s, xp_q, xp_s,
                       p);
  } else {
    auto fn = front_small_kernel<float>;
    if (lds > 64 * 1024 &&
        (err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(lds))) != hipSuccess)
      return err;
    hipLaunchKernelGGL(fn, dim3(1), dim3(kPlanThreads), lds, stream, logits, bias, T, E, k,
                       renormalize, static_cast<const float*>(x), H, ids, w, x_q, x_s, xp_q, xp_s, p);
  }
  return hipGetLastError();
}

}  // namespace moeq
