// Grouped GEMM over NVFP4 expert weights (the hot experts of the NVFP4 + AQLM
// hybrid checkpoint): E2M1 codes, two per byte with the low nibble first, one
// E4M3 scale per 16 consecutive K and one fp32 scale2 per expert:
//   W[n, k] = e2m1(code) * e4m3(scale[n, k / 16]) * scale2
// with per-token FP8 (E4M3) activations:
//   out[p, n] = epilogue( a_s[p] * scale2[e] * sum_k e4m3(a_q[p, k]) * e2m1(c) * s_b )
//
// The block size (16) is smaller than any FP8 MFMA's K, so the block scale is
// folded into the weights before the MFMA instead of being applied to partial
// sums: each code becomes f16 with v_cvt_scalef32_pk_f16_fp4 (scale 1; that
// instruction applies only the exponent of its scale operand) and is multiplied
// by its block scale with v_pk_mul_f16.  e2m1 values carry at most 2 significant
// bits and E4M3 scales 4, so the product (<= 6 bits, |.| <= 2688, >= 2^-10) is
// exact in f16.  Activations become f16 exactly with v_cvt_scalef32_pk_f16_fp8
// (scale 1).  v_mfma_f32_16x16x32_f16 then forms exact products accumulated in
// fp32 over all of K; scale2 and the activation scale are applied once at the
// end.  One dequantization instruction per weight pair plus one multiply: no
// per-block partial sums and no per-group FMAs.
//
// slab_of (optional, [E]): weight slab of each routed expert, -1 for experts
// stored in another format (the hybrid card keeps hot experts as NVFP4 slabs
// listed by hot_ids and cold ones as AQLM); tiles of such experts are skipped,
// so the rows they own are left to the other format's kernel.
//
// Structure: the K-split units of the INT4 path's wave kernel (gemm.hip) -- one
// workgroup per (plan tile, 32 weight rows), wave q sweeping K quarter q in
// 128-K chunks through a register ring, the quarters summed in LDS in a fixed
// order and stored by wave 0 (a few hot experts make few units: splitting K
// puts four times the loads in flight); lane (n, kb)
// holds K [32 kb, 32 kb + 32) of its row per chunk (16 bytes of codes and the
// two block scales, one 16-bit load) and feeds four MFMAs of K = 32 (lane kb's
// 8 K-slots of MFMA j are the chunk's K 32 kb + 8 j .. + 8; the activation
// operand uses the same mapping).  Tiles with more than 16 rows are swept once
// per 16-row block.
#include "gemm.hpp"

namespace moeq {

namespace {

constexpr int kNvDepth = 3;   // 128-K chunks in flight per wave (4 spills)

// 8 E2M1 codes (one dword, low nibble first) times their block scale -> 8 f16, exact
__device__ __forceinline__ h8 fp4x8_to_f16(uint32_t w, h2 s) {
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E4M3 byte SEL of v -> f16 pair {s, s} (exact)
template <int SEL>
__device__ __forceinline__ h2 block_scale_pair(uint32_t v) {
  const _Float16 s = static_cast<_Float16>(__builtin_amdgcn_cvt_f32_fp8(int(v), SEL));
  return h2{s, s};
}

struct NvStage {
  uint4 a0, a1;        // 32 activation bytes of this lane's row
  uint4 b[2];          // 32 codes of each of the two weight-row blocks
  uint32_t s[2];       // their two block scales (low byte: first 16 K, next byte: second)
};

template <int EPI>
__global__ void __launch_bounds__(kThreads, 3)
gemm_nvfp4_kernel(const uint8_t* a_q, const float* a_s, const int32_t* plan, int E, int R,
                  const int32_t* slab_of, int S, const uint8_t* w, const uint8_t* w_bs,
                  const float* w_scale2, int N, int K, void* out, int out_f32) {
  __shared__ v4f red[3 * 2 * kWave];            // quarter sums of waves 1..3
  const int lane = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, kb = lane >> 4;
  const int units_per_tile = N / 32;
  const int tile = blockIdx.x / units_per_tile;
  const int u = blockIdx.x - tile * units_per_tile;
  TileInfo ti;
  if (!tile_info(plan, E, R, tile, ti)) return;   // workgroup-uniform
  // weight slab of the tile's expert; experts stored in another format are skipped
  const int slab = slab_of ? slab_of[ti.e] : ti.e;
  if (slab < 0 || slab >= S) return;                    // workgroup-uniform
  const float scale2 = w_scale2[slab];
  const int G = K >> 7;
  const int g0 = quarter_g0(G, q), gq = quarter_groups(G, q);   // this wave's K quarter

  int col[2];
  unit_columns<EPI, 2>(N, u, col);
  const uint8_t* wrow[2];
  const uint8_t* srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n_glob = int64_t(slab) * N + col[j] + ln;
    wrow[j] = w + n_glob * (K >> 1) + g0 * 64;
    srow[j] = w_bs + n_glob * (K >> 4) + g0 * 8;
  }

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    const bool a_ok = 16 * rb + ln < ti.rows;
    const uint8_t* a_src = a_q + int64_t(ti.row0 + (a_ok ? 16 * rb + ln : 0)) * K + g0 * 128 + kb * 32;
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    NvStage st[kNvDepth];
#pragma unroll
    for (int d = 0; d < kNvDepth; ++d) {
      st[d].a0 = make_uint4(0, 0, 0, 0);
      st[d].a1 = st[d].a0;
    }
    auto issue = [&](int slot, int g) {
      if (a_ok) {
        const uint4* ap = reinterpret_cast<const uint4*>(a_src + g * 128);
        st[slot].a0 = ap[0];
        st[slot].a1 = ap[1];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        st[slot].b[j] = *reinterpret_cast<const uint4*>(wrow[j] + g * 64 + kb * 16);
        st[slot].s[j] = *reinterpret_cast<const uint16_t*>(srow[j] + g * 8 + kb * 2);
      }
    };
    auto consume = [&](int slot, int g, bool refill) {
      // the slot's raw bytes, taken before the refill overwrites it; they are
      // converted step by step between the MFMAs
      const NvStage s = st[slot];
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(slot, g + kNvDepth);
      const uint32_t ad[8] = {s.a0.x, s.a0.y, s.a0.z, s.a0.w, s.a1.x, s.a1.y, s.a1.z, s.a1.w};
      h2 sc[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sc[j][0] = block_scale_pair<0>(s.s[j]);
        sc[j][1] = block_scale_pair<1>(s.s[j]);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const h8 aop = fp8x8_to_f16(ad[2 * m], ad[2 * m + 1]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t bw = m == 0 ? s.b[j].x : m == 1 ? s.b[j].y : m == 2 ? s.b[j].z : s.b[j].w;
          acc[j] = mfma_f16(aop, fp4x8_to_f16(bw, sc[j][m >> 1]), acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) pin(acc[j]);
    };
    pipeline<kNvDepth, 0>(gq, issue, consume);
    quarter_reduce<2>(acc, red, q, lane, rb + 1 < nrb);
    if (q == 0)
      store_block<kNvfp4, EPI>(acc, rb, ti.row0, ti.rows,
                               [a_s, scale2](int p, int) { return a_s[p] * scale2; }, srow, col, ln,
                               kb, N, out, out_f32);
  }
}

}  // namespace

hipError_t launch_grouped_gemm_nvfp4(const uint8_t* a_q, const float* a_s, const void* plan, int E,
                                     int R, const int32_t* slab_of, int S, const uint8_t* w,
                                     const uint8_t* w_block_scale,
                                     const float* w_scale2, int N, int K, int epilogue, void* out,
                                     int out_dtype, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int out_f32 = out_dtype == MOEQ_F32 ? 1 : 0;
  const int64_t units = int64_t(plan_max_tiles(E, R)) * (N / 32);
  const dim3 grid{static_cast<unsigned>(units)};         // one workgroup per unit
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (epilogue == MOEQ_EPI_SILU_MUL)
    hipLaunchKernelGGL(gemm_nvfp4_kernel<MOEQ_EPI_SILU_MUL>, grid, dim3(kThreads), 0, stream, a_q,
                       a_s, p, E, R, slab_of, S, w, w_block_scale, w_scale2, N, K, out, out_f32);
  else
    hipLaunchKernelGGL(gemm_nvfp4_kernel<MOEQ_EPI_NONE>, grid, dim3(kThreads), 0, stream, a_q, a_s,
                       p, E, R, slab_of, S, w, w_block_scale, w_scale2, N, K, out, out_f32);
  return hipGetLastError();
}

}  // namespace moeq
