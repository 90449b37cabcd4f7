// The routed experts' MLP: gate/up GEMM with the SiLU-gated product, per-row
// FP8 quantization of h, down GEMM.
//
// For few routed rows (R <= kWaveMaxRows, the decode regime) and I <= 2048 the down GEMM
// quantizes h itself, so the MLP is two launches instead of three.  It runs
// the grouped GEMM's K-split units (one workgroup per (tile, 32 weight rows),
// wave q sweeping K quarter q).  Before its weight loads each wave loads its
// quarter of the block's rows of h (one 16-byte load per lane and row; the
// quarter is at most 512 elements); after issuing them it takes max |h| of
// each row over its quarter, the four partial maxima meet in LDS at one
// barrier, and each wave encodes its quarter with the row's scale into LDS,
// from where its sweep reads the activations.  The maximum of the partial
// maxima is the row maximum, and the scale and codes are quant_fp8_per_token's
// arithmetic, so h_q, h_s and o are bit-identical to the three separate calls.
// The tile's first workgroup also stores the codes and scales (h_q, h_s).
// Larger R or I take the three launches.
#include "gemm.hpp"

namespace moeq {

namespace {

constexpr int kHqRows = 16;                 // rows of a 16-row block
constexpr int kHqMaxQuarter = 512;          // elements of h per wave and row (I <= 2048)
constexpr int kHqStride = kHqMaxQuarter + 16;

__device__ __forceinline__ uint4 load_h8(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int WFMT, int GS>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
down_hq_kernel(const uint16_t* h, const int32_t* plan, int E, int R, const uint8_t* w2,
               const ScaleT<WFMT>* s2, int H, int I, uint8_t* h_q, float* h_s, uint16_t* o) {
  static_assert(GS % 4 == 0, "quarters of a compile-time sweep must be whole groups");
  constexpr int GQ = GS / 4;
  __shared__ __align__(16) uint8_t a_stage[4][kHqRows][kHqStride];   // E4M3 codes
  __shared__ float s_part[4][kHqRows];          // per-quarter max |h| of each row
  __shared__ float s_scale[kHqRows];
  __shared__ v4f red[3 * 2 * kWave];           // quarter sums of waves 1..3
  const int lane = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, kb = lane >> 4;
  const int upt = H >> 5;                       // units per tile
  const int tile = blockIdx.x / upt;
  const int u = blockIdx.x - tile * upt;
  TileInfo ti;
  const bool active = tile_info(plan, E, R, tile, ti);
  // the kernel arguments used after the exit test are loaded ahead of it, with
  // the ones the lookup needs (an asm statement ahead of the plan loads would
  // turn them into vector loads)
  asm volatile("" ::"s"(h), "s"(w2), "s"(s2), "s"(h_q), "s"(h_s), "s"(o));
  if (!active) return;                          // workgroup-uniform
  const bool writer = u == 0;                   // the tile's first workgroup stores h_q, h_s

  int col[2];
  unit_columns<MOEQ_EPI_NONE>(H, u, col);
  const uint8_t* wblk[2];
  const ScaleT<WFMT>* srow[2];
  uint32_t wlane;
  weight_rows<WFMT>(w2, s2, ti.e, H, I, col, ln, kb, wblk, srow, wlane);
  const int G = I >> 7;
  const int g0 = quarter_g0(G, q);
  quarter_rows<WFMT, 2>(g0, wblk, srow);
  const int kq = (GS > 0 ? GQ : quarter_groups(G, q)) * 128;   // <= kHqMaxQuarter
  const int c0 = g0 * 128 + lane * 8;           // this lane's 8 elements of the quarter
  const bool on = lane * 8 < kq;
  uint8_t* stage = &a_stage[q][0][0];

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    const int rrows = min(kHqRows, ti.rows - 16 * rb);
    const int64_t p0 = ti.row0 + 16 * rb;       // plan row of the block's first row
    const uint16_t* hb = h + p0 * I + c0;
    // rows 0..3 loaded ahead of the weights (scalars: an array captured by the
    // lambda below would stay in scratch); further rows, rare, in the hook
    uint4 v0 = {}, v1 = {}, v2 = {}, v3 = {};
    if (on) {
      v0 = load_h8(hb);
      if (rrows > 1) v1 = load_h8(hb + I);
      if (rrows > 2) v2 = load_h8(hb + 2 * int64_t(I));
      if (rrows > 3) v3 = load_h8(hb + 3 * int64_t(I));
    }
    auto quantize = [&] {
      auto part = [&](int r, const uint4& raw) {
        float v[8];
        bf16x8_to_f32(raw, v);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        m = wave_max(m);
        if (lane == 0) s_part[q][r] = m;
      };
      auto encode = [&](int r, const uint4& raw) {
        const float scale = fp8_scale(fmaxf(fmaxf(s_part[0][r], s_part[1][r]),
                                            fmaxf(s_part[2][r], s_part[3][r])));
        float v[8];
        bf16x8_to_f32(raw, v);
        const uint2 c = fp8_codes8(v, scale);
        if (on) {
          *reinterpret_cast<uint2*>(stage + r * kHqStride + lane * 8) = c;
          if (writer) *reinterpret_cast<uint2*>(h_q + (p0 + r) * I + c0) = c;
        }
        if (q == 0 && lane == 0) {
          s_scale[r] = scale;
          if (writer) h_s[p0 + r] = scale;
        }
      };
      const uint4 zero = {};
      part(0, v0);
      if (rrows > 1) part(1, v1);
      if (rrows > 2) part(2, v2);
      if (rrows > 3) part(3, v3);
      for (int r = 4; r < rrows; ++r) part(r, on ? load_h8(hb + r * int64_t(I)) : zero);
      __syncthreads();
      encode(0, v0);
      if (rrows > 1) encode(1, v1);
      if (rrows > 2) encode(2, v2);
      if (rrows > 3) encode(3, v3);
      for (int r = 4; r < rrows; ++r) encode(r, on ? load_h8(hb + r * int64_t(I)) : zero);
    };
    v4f acc[2];
    wave_sweep<WFMT, 2, GQ, true, kALds>(acc, stage, kq, 0, rrows, 0, wblk, srow, wlane, ln, kb,
                                         quantize, kHqStride);
    quarter_reduce<2>(acc, red, q, lane, rb + 1 < nrb);
    if (q == 0)
      store_block<WFMT, MOEQ_EPI_NONE>(acc, rb, ti.row0, ti.rows,
                                       [&](int p, int) { return s_scale[p - p0]; }, srow, col, ln, kb,
                                       H, o, 0);
    // the next block rewrites s_part after every wave has passed this block's
    // reduction barrier (all reads of s_part precede it); s_scale is written
    // and read by wave 0 alone
  }
}

template <int WFMT>
hipError_t launch_down_hq(const uint16_t* h, const void* plan, int E, int R, const uint8_t* w2,
                          const ScaleT<WFMT>* s2, int H, int I, uint8_t* h_q, float* h_s,
                          uint16_t* o, hipStream_t stream) {
  const int64_t units = int64_t(plan_max_tiles(E, R)) * (H >> 5);
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (I == 2048)
    hipLaunchKernelGGL((down_hq_kernel<WFMT, 16>), dim3(unsigned(units)), dim3(kThreads), 0,
                       stream, h, p, E, R, w2, s2, H, I, h_q, h_s, o);
  else
    hipLaunchKernelGGL((down_hq_kernel<WFMT, 0>), dim3(unsigned(units)), dim3(kThreads), 0,
                       stream, h, p, E, R, w2, s2, H, I, h_q, h_s, o);
  return hipGetLastError();
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
  if (R <= kWaveMaxRows && I <= 4 * kHqMaxQuarter) {
    switch (wfmt) {
      case kW4G128:
        return launch_down_hq<kW4G128>(h, plan, E, R, w2, static_cast<const float*>(s2), H, I,
                                       h_q, h_s, o, stream);
      case kW4G128Bf16:
        return launch_down_hq<kW4G128Bf16>(h, plan, E, R, w2, static_cast<const uint16_t*>(s2), H,
                                           I, h_q, h_s, o, stream);
      default:
        return launch_down_hq<kFp8Row>(h, plan, E, R, w2, static_cast<const float*>(s2), H, I,
                                       h_q, h_s, o, stream);
    }
  }
  if ((err = launch_quant_fp8(h, MOEQ_BF16, R, I, I, h_q, h_s, stream)) != hipSuccess) return err;
  return launch_grouped_gemm(wfmt, h_q, h_s, plan, E, R, w2, s2, H, I, MOEQ_EPI_NONE, o, MOEQ_BF16,
                             stream);
}

}  // namespace moeq
