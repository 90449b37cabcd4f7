// moe_combine kernel: one thread per 8 consecutive hidden columns of one token.
// y[t, c] = bf16( sum_j w[t, j] * o[row_pos[t*k + j], c] + shared[t, c] ), fp32
// accumulation in slot order j = 0..k-1, then the shared-expert addend.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

__device__ __forceinline__ void bf16x8_to_f32(const uint4& u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = u2f(w[i] << 16);
    v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
  }
}

__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ o, const int32_t* __restrict__ plan,
               const float* __restrict__ w, const uint16_t* __restrict__ shared, int T, int k,
               int H, uint16_t* __restrict__ y) {
  // token t = blockIdx.x, 2048-column block blockIdx.y: no division by a
  // kernel argument, so every argument load goes out in one round
  const int t = blockIdx.x;
  const int R = T * k;
  const int c_raw = (blockIdx.y * 256 + threadIdx.x) * 8;
  const bool live = c_raw < H;
  const int c = live ? c_raw : 0;
  // row_pos leads the plan after its header: no dependent read of E.  Lane j of
  // each wave loads slot j's position and weight (lanes past k re-read slot
  // k - 1 and are ignored), which reach every lane by readlane: one round trip
  // for all the slots, then one for every slot's row of o (a row that is not
  // there reads row 0 and is dropped).  (As scalar loads, the sixteen values
  // came back in two rounds or, under per-slot branches, in sixteen.)
  const int32_t* row_pos = plan + kPlanHeader;
  const int lane = threadIdx.x & 63;
  const int slot = t * k + min(lane, k - 1);
  const int pos_l = row_pos[slot];
  const float w_l = w[slot];
  int pos[MOEQ_MAX_TOPK];
  float wt[MOEQ_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOEQ_MAX_TOPK; ++j) {
    pos[j] = readlane(pos_l, j);
    wt[j] = readlane(w_l, j);
  }
  uint4 raw[MOEQ_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOEQ_MAX_TOPK; ++j)
    raw[j] = *reinterpret_cast<const uint4*>(o + int64_t(min(max(pos[j], 0), R - 1)) * H + c);
  uint4 sh = {};
  if (shared) sh = *reinterpret_cast<const uint4*>(shared + int64_t(t) * H + c);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < MOEQ_MAX_TOPK; ++j) {
    // slots past k, rows dropped by the permute (and positions outside o, which
    // only a plan built for other sizes holds)
    if (j >= k || pos[j] < 0 || pos[j] >= R) continue;
    float v[8];
    bf16x8_to_f32(raw[j], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], v[i], acc[i]);
  }
  if (shared) {
    float v[8];
    bf16x8_to_f32(sh, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  uint4 out;
  out.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
  out.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
  out.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
  out.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
  if (live) *reinterpret_cast<uint4*>(y + int64_t(t) * H + c) = out;
}

}  // namespace

hipError_t launch_combine(const uint16_t* o, const void* plan, const float* w,
                          const uint16_t* shared, int T, int k, int H, uint16_t* y,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  dim3 grid(unsigned(T), unsigned((H / 8 + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, o, static_cast<const int32_t*>(plan),
                     w, shared, T, k, H, y);
  return hipGetLastError();
}

}  // namespace moeq
