// The routed experts' MLP -- gate/up GEMM with the SiLU-gated product, per-row
// FP8 quantization of h, down GEMM -- in two launches for few routed rows
// (R <= kMlpMaxRows, e.g. decode) instead of three.
//
// The down GEMM quantizes h itself.  Its workgroups hold four consecutive wave
// units (tile, 32 weight rows) of one tile; each first issues its first weight
// loads, then quantizes the tile's rows of h (wave w takes rows w, w + 4, ...:
// max |h|, scale, E4M3 codes -- quant_fp8_per_token's arithmetic) into LDS,
// meets the other three at a barrier, and runs its sweep with the activations
// read from LDS.  h comes from the previous launch, so nothing crosses waves
// inside a launch except through LDS.  The quantization repeats in each of
// the tile's workgroups (a few microseconds of VALU work overlapped with the
// weight loads already in flight); the workgroup with the tile's first units
// also writes the codes and scales out (h_q, h_s).  This removes the
// quantization launch and one launch gap.
//
// Used when the LDS for a tile's rows fits three workgroups per CU; otherwise
// the three launches.  The arithmetic is the wave kernel's and
// quant_fp8_per_token's, so h, its codes and scales, and o are bit-identical to
// the three separate calls.
#include "gemm.hpp"

namespace moeq {

namespace {

constexpr int kLdsPad = 16;                     // LDS row padding (bank spread)
constexpr size_t kLdsPerWorkgroup = 53 * 1024;  // three workgroups per CU

__host__ __device__ inline int lds_stride(int I) { return I + kLdsPad; }

// Down GEMM (EPI_NONE, bf16 out) that quantizes its tile's rows of h into LDS.
template <int WFMT, int GS>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
down_quant_kernel(const uint16_t* h, const int32_t* plan, int E, int R, const uint8_t* w2,
                  const ScaleT<WFMT>* s2, int H, int I, uint8_t* h_q, float* h_s, uint16_t* o) {
  extern __shared__ __align__(16) uint8_t s_codes[];   // [rows][lds_stride(I)] E4M3
  __shared__ float s_scale[kMlpMaxRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int upt = H >> 5;                               // a multiple of 4
  const int tile = blockIdx.x * (kThreads / 64) / upt;  // one tile per workgroup
  const int u = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + wave) - tile * upt;
  if (tile >= plan[kPlanTiles]) return;                 // workgroup-uniform
  const TileInfo ti = tile_info(plan, E, R, tile);
  const int stride = lds_stride(I);
  const bool writer = u < kThreads / 64;                // the tile's first workgroup

  auto quantize_rows = [&] {
    for (int r = wave; r < ti.rows; r += kThreads / 64) {
      const int p = ti.row0 + r;
      const uint16_t* hr = h + int64_t(p) * I;
      float amax = 0.0f;
      for (int c = lane; c < (I >> 3); c += kWave) {
        float v[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(hr + c * 8), v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
      const float scale = fp8_scale(wave_max(amax));
      for (int c = lane; c < (I >> 3); c += kWave) {
        float v[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(hr + c * 8), v);
        const uint2 q = fp8_codes8(v, scale);
        *reinterpret_cast<uint2*>(s_codes + r * stride + c * 8) = q;
        if (writer) *reinterpret_cast<uint2*>(h_q + int64_t(p) * I + c * 8) = q;
      }
      if (lane == 0) {
        s_scale[r] = scale;
        if (writer) h_s[p] = scale;
      }
    }
    __syncthreads();
  };

  int col[2];
  unit_columns<MOEQ_EPI_NONE>(H, u, col);
  const uint8_t* wrow[2];
  const ScaleT<WFMT>* srow[2];
  weight_rows<WFMT>(w2, s2, ti.e, H, I, col, ln, wrow, srow);
  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    v4f acc[2];
    wave_sweep<WFMT, 2, GS, true, kALds>(
        acc, s_codes, I, ti.row0, ti.rows, rb, wrow, srow, ln, kb,
        [&] {
          if (rb == 0) quantize_rows();
        },
        stride);
    store_block<WFMT, MOEQ_EPI_NONE>(acc, rb, ti.row0, ti.rows,
                                     [&](int p) { return s_scale[p - ti.row0]; }, srow, col, ln,
                                     kb, H, o, 0);
  }
}

template <int WFMT, int GS>
hipError_t launch_down_quant(const uint16_t* h, const void* plan, int E, int R, const uint8_t* w2,
                             const ScaleT<WFMT>* s2, int H, int I, uint8_t* h_q, float* h_s,
                             uint16_t* o,
                             size_t lds, hipStream_t stream) {
  auto fn = down_quant_kernel<WFMT, GS>;
  hipError_t err;
  if (lds > 64 * 1024 &&
      (err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds))) != hipSuccess)
    return err;
  const int64_t units = int64_t(plan_max_tiles(E, R)) * (H >> 5);
  hipLaunchKernelGGL(fn, dim3(unsigned(units / 4)), dim3(kThreads), lds, stream, h,
                     static_cast<const int32_t*>(plan), E, R, w2, s2, H, I, h_q, h_s, o);
  return hipGetLastError();
}

template <int WFMT>
hipError_t launch_down_quant_shape(const uint16_t* h, const void* plan, int E, int R,
                                   const uint8_t* w2, const ScaleT<WFMT>* s2, int H, int I,
                                   uint8_t* h_q,
                                   float* h_s, uint16_t* o, size_t lds, hipStream_t stream) {
  if (I == 2048)
    return launch_down_quant<WFMT, 16>(h, plan, E, R, w2, s2, H, I, h_q, h_s, o, lds, stream);
  return launch_down_quant<WFMT, 0>(h, plan, E, R, w2, s2, H, I, h_q, h_s, o, lds, stream);
}

}  // namespace

hipError_t launch_expert_mlp(int wfmt, const uint8_t* xp_q, const float* xp_s, const void* plan,
                             int E, int R, const uint8_t* w13, const void* s13, const uint8_t* w2,
                             const void* s2, int H, int I, uint16_t* h, uint8_t* h_q, float* h_s,
                             uint16_t* o, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipError_t err = launch_grouped_gemm(wfmt, xp_q, xp_s, plan, E, R, w13, s13, 2 * I, H,
                                       MOEQ_EPI_SILU_MUL, h, MOEQ_BF16, stream);
  if (err != hipSuccess) return err;
  const int max_rows = R < kMlpMaxRows ? R : kMlpMaxRows;     // rows of one tile
  const size_t lds = size_t(max_rows) * lds_stride(I);
  if (R <= kMlpMaxRows && lds <= kLdsPerWorkgroup) {
    switch (wfmt) {
      case kW4G128:
        return launch_down_quant_shape<kW4G128>(h, plan, E, R, w2, static_cast<const float*>(s2),
                                                H, I, h_q, h_s, o, lds, stream);
      case kW4G128Bf16:
        return launch_down_quant_shape<kW4G128Bf16>(h, plan, E, R, w2,
                                                    static_cast<const uint16_t*>(s2), H, I, h_q,
                                                    h_s, o, lds, stream);
      default:
        return launch_down_quant_shape<kFp8Row>(h, plan, E, R, w2, static_cast<const float*>(s2),
                                                H, I, h_q, h_s, o, lds, stream);
    }
  }
  if ((err = launch_quant_fp8(h, MOEQ_BF16, R, I, I, h_q, h_s, stream)) != hipSuccess) return err;
  return launch_grouped_gemm(wfmt, h_q, h_s, plan, E, R, w2, s2, H, I, MOEQ_EPI_NONE, o, MOEQ_BF16,
                             stream);
}

}  // namespace moeq
