// Grouped GEMM kernels (wave and tile) over the plan's tiles and their
// launchers; the arithmetic they share with the fused expert MLP (operand
// formats, MFMA, pipelines, group scales) is in gemm.hpp.
#include "gemm.hpp"

#ifndef MOEQ_WAVE_NB
#define MOEQ_WAVE_NB 2
#endif

namespace moeq {

namespace {

// The operand pointers are deliberately not __restrict__: loads through
// restrict-qualified read-only pointers may be hoisted by instruction selection
// past the scheduling barriers of the sweep, which pulls the whole unrolled
// sweep's loads to the top of the kernel and spills them.
template <int WFMT, int EPI, int GS, int NB>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
gemm_wave_kernel(const uint8_t* a_q, const float* a_s, const int32_t* plan, int E, int R,
                 const uint8_t* w, const float* w_scale, int N, int K, void* out, int out_f32) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kb = lane >> 4;
  const int units_per_tile = N / (16 * NB);
  // wave-uniform (readfirstlane): the unit, its tile and the plan entries read
  // from it stay in scalar registers
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  const int tile = unit / units_per_tile;
  const int u = unit - tile * units_per_tile;
  if (tile >= plan[kPlanTiles]) return;                 // wave-uniform
  const TileInfo ti = tile_info(plan, E, R, tile);

  int col[NB];
  unit_columns<EPI, NB>(N, u, col);
  const uint8_t* wrow[NB];
  const float* srow[NB];
  weight_rows<WFMT, NB>(w, w_scale, ti.e, N, K, col, ln, wrow, srow);

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    v4f acc[NB];
    wave_sweep<WFMT, NB, GS, false>(acc, a_q, K, ti.row0, ti.rows, rb, wrow, srow, ln, kb, [] {});
    store_block<WFMT, EPI, NB>(acc, rb, ti.row0, ti.rows, [a_s](int p) { return a_s[p]; }, srow,
                               col, ln, kb, N, out, out_f32);
  }
}

// ------------------------------------------------------------- tile kernel
template <int WFMT>
struct TileStage {
  uint4 a0, a1;          // this thread's 32-byte share of the group's activation slice
  BFrag<WFMT> b[2];
  float s[2];
};

template <int WFMT, int EPI, int GS>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
gemm_tile_kernel(const uint8_t* __restrict__ a_q, const float* __restrict__ a_s,
                 const int32_t* __restrict__ plan, int E, int R, const uint8_t* __restrict__ w,
                 const float* __restrict__ w_scale, int N, int K, void* __restrict__ out,
                 int out_f32) {
  __shared__ uint32_t As[2][MOEQ_TILE_M * kRowDw];

  // Consecutive block ids go to XCDs round-robin; within each run of
  // 8 * n_ntiles ids, XCD x takes the n_ntiles N-tiles of one row tile, so every
  // XCD gets an equal share of the (device-side, unknown here) real tiles.
  const int n_ntiles = N / kBN;
  const int total = n_ntiles * plan_max_tiles(E, R);
  const int run = kXcds * n_ntiles;
  const int bid = blockIdx.x;
  const int logical = (bid / run) * run + (bid % kXcds) * n_ntiles + (bid / kXcds) % n_ntiles;
  if (logical >= total) return;
  const int tile = logical / n_ntiles;
  const int nt = logical - tile * n_ntiles;
  if (tile >= plan[kPlanTiles]) return;                 // workgroup-uniform
  const TileInfo ti = tile_info(plan, E, R, tile);
  const int nrb = (ti.rows + 15) >> 4;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int G = K >> 7;

  int col[2];
  if (EPI == MOEQ_EPI_SILU_MUL) {
    col[0] = nt * 64 + 16 * wave;
    col[1] = (N >> 1) + nt * 64 + 16 * wave;
  } else {
    col[0] = nt * kBN + 16 * wave;
    col[1] = nt * kBN + 16 * (wave + 4);
  }
  const uint8_t* wrow[2];
  const float* srow[2];
  weight_rows<WFMT>(w, w_scale, ti.e, N, K, col, ln, wrow, srow);

  // A staging: thread -> (row tid / 4, 32-byte chunk tid % 4) of the 64 x 128 B slice;
  // rows past the tile read the tile's first row (MFMA rows are independent and
  // those rows are never stored).  The slice of group g is loaded into registers
  // in group g's ring slot, ahead of its weights in issue order, and written to
  // LDS one group before its use: waiting for it never waits for the weight
  // loads of later groups.
  const int st_row = tid >> 2, st_chunk = tid & 3;
  const bool st_valid = st_row < ti.rows;
  const uint8_t* a_src = a_q + int64_t(ti.row0 + (st_valid ? st_row : 0)) * K + st_chunk * 32;
  auto store_a = [&](int buf, const uint4& x0, const uint4& x1) {
    const v8i o = (WFMT == kW4G128) ? shuffle_a(x0, x1) : as_v8i(x0, x1);
    uint4* dst = reinterpret_cast<uint4*>(&As[buf][st_row * kRowDw + st_chunk * 8]);
    dst[0] = make_uint4(uint32_t(o[0]), uint32_t(o[1]), uint32_t(o[2]), uint32_t(o[3]));
    dst[1] = make_uint4(uint32_t(o[4]), uint32_t(o[5]), uint32_t(o[6]), uint32_t(o[7]));
  };

  v4f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[i][0] = v4f{0.f, 0.f, 0.f, 0.f};
    acc[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  constexpr int kDepth = TileDepth<WFMT>::value;
  TileStage<WFMT> st[kDepth];
  GroupScales<WFMT, GS> sc;
  sc.init(srow, kb);
  auto issue = [&](int slot, int g) {
    const uint4* ap = reinterpret_cast<const uint4*>(a_src + g * 128);
    st[slot].a0 = ap[0];
    st[slot].a1 = ap[1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st[slot].b[j].load(wrow[j], g, kb);
      st[slot].s[j] = sc.load(j, g);
    }
  };
  auto consume = [&](int slot, int g, bool refill) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (g == 0) {
      store_a(0, st[slot].a0, st[slot].a1);
      __syncthreads();
    }
    // the next group's slice (its slot is not the one refilled below)
    const int next = (slot + 1 == kDepth) ? 0 : slot + 1;
    const uint4 x0 = st[next].a0, x1 = st[next].a1;
    const v8i b0 = st[slot].b[0].operand();
    const v8i b1 = st[slot].b[1].operand();
    const float s0 = sc.get(0, g, ln, st[slot].s[0]), s1 = sc.get(1, g, ln, st[slot].s[1]);
    __builtin_amdgcn_sched_barrier(0);
    if (refill) issue(slot, g + kDepth);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nrb) {
        const uint4* ap = reinterpret_cast<const uint4*>(&As[buf][(16 * i + ln) * kRowDw + kb * 8]);
        const v8i aop = as_v8i(ap[0], ap[1]);
        accumulate<WFMT>(acc[i][0], aop, b0, s0);
        accumulate<WFMT>(acc[i][1], aop, b1, s1);
      }
    }
    if (more) store_a(buf ^ 1, x0, x1);
    __syncthreads();
  };
  pipeline<kDepth, GS>(G, issue, consume);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < nrb) {
      const v4f blk[2] = {acc[i][0], acc[i][1]};
      store_block<WFMT, EPI>(blk, i, ti.row0, ti.rows, [a_s](int p) { return a_s[p]; }, srow,
                             col, ln, kb, N, out, out_f32);
    }
  }
}

template <int WFMT, int EPI, int GS>
hipError_t launch_kernels(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                          const uint8_t* w, const float* w_scale, int N, int K, void* out,
                          int out_f32, hipStream_t stream) {
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (R <= 64) {
    // few rows per expert: independent waves, one per (tile, 16 NB weight rows)
    constexpr int NB = (EPI == MOEQ_EPI_SILU_MUL) ? 2 : MOEQ_WAVE_NB;
    const int64_t units = int64_t(plan_max_tiles(E, R)) * (N / (16 * NB));
    const int64_t blocks = (units + 3) / 4;
    hipLaunchKernelGGL((gemm_wave_kernel<WFMT, EPI, GS, NB>), dim3(unsigned(blocks)),
                       dim3(kThreads), 0, stream, a_q, a_s, p, E, R, w, w_scale, N, K, out,
                       out_f32);
  } else {
    const int64_t run = int64_t(kXcds) * (N / kBN);
    const int64_t total = int64_t(N / kBN) * plan_max_tiles(E, R);
    const int64_t grid = (total + run - 1) / run * run;
    hipLaunchKernelGGL((gemm_tile_kernel<WFMT, EPI, GS>), dim3(unsigned(grid)), dim3(kThreads), 0,
                       stream, a_q, a_s, p, E, R, w, w_scale, N, K, out, out_f32);
  }
  return hipGetLastError();
}

// K = 4096 and K = 2048 (the hidden size and the expert width of the layer) get
// fully unrolled K sweeps; any other multiple of 128 uses the looped sweep.
template <int WFMT, int EPI>
hipError_t launch_shape(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                        const uint8_t* w, const float* w_scale, int N, int K, void* out,
                        int out_f32, hipStream_t stream) {
  switch (K >> 7) {
    case 32:
      return launch_kernels<WFMT, EPI, 32>(a_q, a_s, plan, E, R, w, w_scale, N, K, out, out_f32,
                                           stream);
    case 16:
      return launch_kernels<WFMT, EPI, 16>(a_q, a_s, plan, E, R, w, w_scale, N, K, out, out_f32,
                                           stream);
    default:
      return launch_kernels<WFMT, EPI, 0>(a_q, a_s, plan, E, R, w, w_scale, N, K, out, out_f32,
                                          stream);
  }
}

template <int WFMT>
hipError_t launch_fmt(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                      const uint8_t* w, const float* w_scale, int N, int K, int epilogue, void* out,
                      int out_f32, hipStream_t stream) {
  if (epilogue == MOEQ_EPI_SILU_MUL)
    return launch_shape<WFMT, MOEQ_EPI_SILU_MUL>(a_q, a_s, plan, E, R, w, w_scale, N, K, out,
                                                 out_f32, stream);
  return launch_shape<WFMT, MOEQ_EPI_NONE>(a_q, a_s, plan, E, R, w, w_scale, N, K, out, out_f32,
                                           stream);
}

}  // namespace

hipError_t launch_grouped_gemm(int wfmt, const uint8_t* a_q, const float* a_s, const void* plan,
                               int E, int R, const uint8_t* w, const float* w_scale, int N, int K,
                               int epilogue, void* out, int out_dtype, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int out_f32 = out_dtype == MOEQ_F32 ? 1 : 0;
  if (wfmt == kW4G128)
    return launch_fmt<kW4G128>(a_q, a_s, plan, E, R, w, w_scale, N, K, epilogue, out, out_f32,
                               stream);
  return launch_fmt<kFp8Row>(a_q, a_s, plan, E, R, w, w_scale, N, K, epilogue, out, out_f32,
                             stream);
}

}  // namespace moeq
