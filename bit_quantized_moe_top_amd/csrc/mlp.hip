// The routed experts' MLP: gate/up GEMM with the SiLU-gated product, per-row
// FP8 quantization of h, down GEMM -- three launches on one stream.
//
// A down GEMM that quantizes h itself (each workgroup re-quantizing its tile's
// rows of h into LDS, saving the quantization launch) is slower with the
// K-split wave units: every one of the four times more workgroups then pays
// two dependent reads of h and a barrier before its first MFMA, which costs
// more than the small quantization launch it removes.
#include "kernels.hpp"

namespace moeq {

hipError_t launch_expert_mlp(int wfmt, const uint8_t* xp_q, const float* xp_s, const void* plan,
                             int E, int R, const uint8_t* w13, const void* s13, const uint8_t* w2,
                             const void* s2, int H, int I, uint16_t* h, uint8_t* h_q, float* h_s,
                             uint16_t* o, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipError_t err = launch_grouped_gemm(wfmt, xp_q, xp_s, plan, E, R, w13, s13, 2 * I, H,
                                       MOEQ_EPI_SILU_MUL, h, MOEQ_BF16, stream);
  if (err != hipSuccess) return err;
  if ((err = launch_quant_fp8(h, MOEQ_BF16, R, I, I, h_q, h_s, stream)) != hipSuccess) return err;
  return launch_grouped_gemm(wfmt, h_q, h_s, plan, E, R, w2, s2, H, I, MOEQ_EPI_NONE, o, MOEQ_BF16,
                             stream);
}

}  // namespace moeq
