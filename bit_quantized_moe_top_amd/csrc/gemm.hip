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
//
// One workgroup per K-split unit (tile, 16 NB weight rows): wave q sweeps K
// quarter q of the unit for each 16-row block of the tile, the quarters meet
// in LDS, and wave 0 stores the block.  With GS > 0 (G = GS) each quarter's
// sweep is unrolled over its GS / 4 groups; GS == 0 takes any G.
template <int WFMT, int EPI, int GS, int NB>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
gemm_wave_kernel(const uint8_t* a_q, const float* a_s, const int32_t* plan, int E, int R,
                 const uint8_t* w, const ScaleT<WFMT>* w_scale, int N, int K, void* out,
                 int out_f32) {
  static_assert(GS % 4 == 0, "quarters of a compile-time sweep must be whole groups");
  constexpr int GQ = GS / 4;
  // 16-row blocks with at most kStageRows rows (decode) stage a K quarter of
  // up to kStageK bytes of each activation row in LDS: the two 16-byte loads
  // per group of the direct path are mostly masked off for so few rows, and
  // still take a vector memory instruction each
  constexpr int kStageRows = 4, kStageK = 1024, kStageStride = kStageK + 16;
  __shared__ __align__(16) uint8_t a_stage[4][kStageRows][kStageStride];
  __shared__ v4f red[3 * NB * kWave];           // quarter sums of waves 1..3
  const int lane = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, kb = lane >> 4;
  const int units_per_tile = N / (16 * NB);
  const int tile = blockIdx.x / units_per_tile;
  const int u = blockIdx.x - tile * units_per_tile;
  TileInfo ti;
  const bool active = tile_info(plan, E, R, tile, ti);
  // the kernel arguments used after the exit test are loaded ahead of it, with
  // the ones the lookup needs (an asm statement ahead of the plan loads would
  // turn them into vector loads)
  asm volatile("" ::"s"(a_q), "s"(a_s), "s"(w), "s"(w_scale), "s"(out));
  if (!active) return;                          // workgroup-uniform

  int col[NB];
  unit_columns<EPI, NB>(N, u, col);
  const uint8_t* wblk[NB];
  const ScaleT<WFMT>* srow[NB];
  uint32_t wlane;
  weight_rows<WFMT, NB>(w, w_scale, ti.e, N, K, col, ln, kb, wblk, srow, wlane);
  const int G = K >> 7;
  const int g0 = quarter_g0(G, q);
  quarter_rows<WFMT, NB>(g0, wblk, srow);
  const int kq = (GS > 0 ? GQ : quarter_groups(G, q)) * 128;   // K of this wave's quarter

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    v4f acc[NB];
    const int rrows = min(16, ti.rows - 16 * rb);
    // the activation scales of this lane's four rows of the block, loaded ahead
    // of the sweep so that the epilogue does not wait a memory round trip for
    // them (rows past the tile re-read its first row; they are not stored)
    float sa[4] = {0.f, 0.f, 0.f, 0.f};
    if (q == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r_in = 16 * rb + 4 * kb + v;
        sa[v] = a_s[ti.row0 + (r_in < ti.rows ? r_in : 0)];
      }
    }
    if (rrows <= kStageRows && kq <= kStageK) {
      // the block's activation quarter through LDS: one 16-byte load per lane
      // and row, issued ahead of the weight loads
      uint8_t* stage = &a_stage[q][0][0];
      const uint8_t* src = a_q + int64_t(ti.row0 + 16 * rb) * K + g0 * 128 + lane * 16;
      const bool on = lane * 16 < kq;
      // (scalars, not an array: an array captured by the lambda stays in scratch)
      uint4 v0 = {}, v1 = {}, v2 = {}, v3 = {};
      static_assert(kStageRows == 4, "one register per staged row");
      if (on) {
        v0 = *reinterpret_cast<const uint4*>(src);
        if (rrows > 1) v1 = *reinterpret_cast<const uint4*>(src + K);
        if (rrows > 2) v2 = *reinterpret_cast<const uint4*>(src + 2 * int64_t(K));
        if (rrows > 3) v3 = *reinterpret_cast<const uint4*>(src + 3 * int64_t(K));
      }
      wave_sweep<WFMT, NB, GQ, true, kALds>(
          acc, stage, kq, 0, rrows, 0, wblk, srow, wlane, ln, kb,
          [&] {
            if (on) {
              uint8_t* d = stage + lane * 16;
              *reinterpret_cast<uint4*>(d) = v0;
              if (rrows > 1) *reinterpret_cast<uint4*>(d + kStageStride) = v1;
              if (rrows > 2) *reinterpret_cast<uint4*>(d + 2 * kStageStride) = v2;
              if (rrows > 3) *reinterpret_cast<uint4*>(d + 3 * kStageStride) = v3;
            }
          },
          kStageStride);
    } else {
      wave_sweep<WFMT, NB, GQ, false>(acc, a_q + g0 * 128, kq, ti.row0, ti.rows, rb, wblk, srow,
                                      wlane, ln, kb, [] {}, K);
    }
    quarter_reduce<NB>(acc, red, q, lane, rb + 1 < nrb);
    if (q == 0)
      store_block<WFMT, EPI, NB>(acc, rb, ti.row0, ti.rows, [&sa](int, int v) { return sa[v]; },
                                 srow, col, ln, kb, N, out, out_f32);
  }
}

// ------------------------------------------------------------- tile kernel
// CB column blocks (16 weight rows each) per wave: a workgroup covers 64 CB
// weight rows.  CB = 4 halves the activation staging and the LDS reads per
// MFMA against CB = 2, at two waves per SIMD instead of three; the launcher
// takes it for INT4 weights with a fully unrolled K sweep (the looped form does
// not fit the register file) when N is a multiple of 256.
template <int WFMT, int GS, int CB_>
struct TileShape {
  static constexpr int CB = CB_;
  static_assert(CB == 2 || (CB == 4 && kIsW4<WFMT> && GS > 0 && GS % 16 == 0), "tile shape");
  // (the looped sweep, GS == 0, keeps a shallower ring to stay within registers)
  static constexpr int kDepth = (CB == 4 || GS == 0) ? 2 : TileDepth<WFMT>::value;
  static constexpr int kWavesPerSimd = (CB == 4) ? 2 : 3;
  // group scales staged in LDS ([g][wave][ln][j], 4 CB bytes per lane and
  // group) instead of registers
  static constexpr bool kLdsScales = (CB == 4);
};

template <int WFMT, int CB>
struct TileStage {
  uint4 a0, a1;          // this lane's two 16-byte pieces of the group's activation slice
  BFrag<WFMT> b[CB];
  float s[CB];
};

template <int WFMT, int EPI, int GS, int CB_>
__global__ void __launch_bounds__(kThreads, (CB_ == 4) ? 2 : 3)   // TileShape::kWavesPerSimd
gemm_tile_kernel(const uint8_t* __restrict__ a_q, const float* __restrict__ a_s,
                 const int32_t* __restrict__ plan, int E, int R, const uint8_t* __restrict__ w,
                 const ScaleT<WFMT>* __restrict__ w_scale, int N, int K, void* __restrict__ out,
                 int out_f32) {
  using Shape = TileShape<WFMT, GS, CB_>;
  constexpr int CB = Shape::CB;
  constexpr int BN = 64 * CB;                           // weight rows per workgroup
  __shared__ uint32_t As[2][MOEQ_TILE_M * kRowDw];
  // The group scales (staged once, read by every group of the sweep) and, after
  // the sweep's last barrier, the workgroup's bf16 output tile in the same LDS:
  // OC columns (the SiLU-gated product has half as many as the weight rows),
  // rows OS bytes apart (16 bytes of padding spread the rows over the banks).
  constexpr int kSsFloats = Shape::kLdsScales ? GS * 4 * 16 * CB : 1;
  constexpr int OC = (EPI == MOEQ_EPI_SILU_MUL) ? BN / 2 : BN;
  constexpr int OS = OC * 2 + 16;
  constexpr int kOsFloats = MOEQ_TILE_M * OS / 4;
  __shared__ __align__(16) float SsOs[kSsFloats > kOsFloats ? kSsFloats : kOsFloats];
  float* const Ss = SsOs;
  uint8_t* const Os = reinterpret_cast<uint8_t*>(SsOs);

  // Work items are (row tile, N-tile) pairs of the plan's tiles.  Consecutive
  // block ids go to XCDs round-robin (block b to XCD b % 8); XCD x takes a
  // contiguous run of the items, so an expert's row tiles run on one XCD and
  // read its weight slices through one L2 instead of once per tile from HBM.
  // Runs differ by at most one item, and XCD x has at least as many blocks as
  // items (the grid holds n_ntiles blocks per possible tile).
  const int n_ntiles = N / BN;
  const PlanView pv = plan_view(const_cast<int32_t*>(plan), E, R);
  const int n_real = min(max(plan[kPlanTiles], 0), pv.max_tiles);
  const int items = n_real * n_ntiles;
  const int x = int(blockIdx.x) % kXcds, i = int(blockIdx.x) / kXcds;
  const int q = items / kXcds, rem = items - q * kXcds;
  if (i >= q + (x < rem ? 1 : 0)) return;       // workgroup-uniform
  const int idx = x * q + min(x, rem) + i;
  const int tb = idx / n_ntiles;
  int nt;
  TileInfo ti;
  {
    // Inside an expert's items the N-tile is the major index and the row tile
    // the minor one: the row tiles that read one weight slice are neighbours in
    // issue order and stream it together.  The expert's first tile t0 and tile
    // count m follow from its row offsets (its tiles are consecutive in the list,
    // 64 rows each from offsets[e] on).
    const int e = min(max(pv.tile_expert[tb], 0), E - 1);
    const int r_tb = pv.tile_row0[tb];
    const int base = min(max(pv.offsets[e], 0), R);
    const int end = min(max(pv.offsets[e + 1], base), R);
    const int m = max(1, (end - base + MOEQ_TILE_M - 1) / MOEQ_TILE_M);
    const int t0 = tb - min(max((r_tb - base) / MOEQ_TILE_M, 0), tb);
    // (clamps: a plan built for other sizes yields wrong rows, never an access
    // outside the buffers)
    const int local = min(max(idx - t0 * n_ntiles, 0), m * n_ntiles - 1);
    nt = local / m;
    ti.e = e;
    ti.row0 = min(base + MOEQ_TILE_M * (local - nt * m), R);
    ti.rows = max(0, min(MOEQ_TILE_M, end - ti.row0));
    ti.shared_w = m > 1;
    // (no exit for a tile without rows, which only a plan built for other sizes
    // has: it stages and stores nothing, and a late exit test makes the
    // compiler spill the unrolled sweep)
  }
  const int nrb = (ti.rows + 15) >> 4;
  // Weight loads: an expert with one tile is the only reader of its weight
  // slice, which is streamed past L2 (kCpStream); the slices of an expert with
  // several tiles are read once per tile and kept (kCpKeep).  The rest of the
  // kernel comes in two copies, one per policy: a branch per load would split
  // the unrolled sweep into basic blocks.
  const auto body = [&](auto cp) {
    constexpr int CP = decltype(cp)::value;
    // (the wave index as a scalar: the weight block bases derived from it stay in
    // scalar registers)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, kb = lane >> 4;
    const int G = K >> 7;

    // EPI_SILU_MUL: the workgroup takes BN/2 gate rows and the matching up rows;
    // wave w its 8 CB consecutive gate rows (blocks j < CB/2) and their up rows.
    // Otherwise wave w takes blocks w, w + 4, ... of the workgroup's BN rows.
    int col[CB];
  #pragma unroll
    for (int j = 0; j < CB; ++j) {
      if (EPI == MOEQ_EPI_SILU_MUL)
        col[j] = (j < CB / 2 ? 0 : (N >> 1)) + nt * (BN / 2) + wave * (8 * CB) + 16 * (j % (CB / 2));
      else
        col[j] = nt * BN + 16 * (wave + 4 * j);
    }
    const uint8_t* wblk[CB];
    const ScaleT<WFMT>* srow[CB];
    uint32_t wlane;
    weight_rows<WFMT, CB>(w, w_scale, ti.e, N, K, col, ln, kb, wblk, srow, wlane);

    // A staging: wave w stages rows 16 w .. 16 w + 15 of the 64 x 128 B slice;
    // load j of lane l takes segment l % 8 (16 bytes) of row 16 w + 8 j + l / 8,
    // so each load reads 8 whole 128-byte lines.  Waves past the tile's last
    // 16-row block stage nothing; rows past the tile inside it read the tile's
    // first row (MFMA rows are independent and those rows are never stored).
    // The slice of group g is loaded into registers in group g's ring slot,
    // ahead of its weights in issue order, and written to LDS one group before
    // its use: waiting for it never waits for the weight loads of later groups.
    const bool st_on = wave < nrb;                        // wave-uniform
    const int st_seg = lane & 7;
    const int st_r0 = 16 * wave + (lane >> 3), st_r1 = st_r0 + 8;
    const uint8_t* a_src0 = a_q + int64_t(ti.row0 + (st_r0 < ti.rows ? st_r0 : 0)) * K + st_seg * 16;
    const uint8_t* a_src1 = a_q + int64_t(ti.row0 + (st_r1 < ti.rows ? st_r1 : 0)) * K + st_seg * 16;
    auto store_a = [&](int buf, const uint4& x0, const uint4& x1) {
      if (!st_on) return;
      *reinterpret_cast<uint4*>(&As[buf][st_r0 * kRowDw + st_seg * 4]) =
          kIsW4<WFMT> ? shuffle_a16(x0) : x0;
      *reinterpret_cast<uint4*>(&As[buf][st_r1 * kRowDw + st_seg * 4]) =
          kIsW4<WFMT> ? shuffle_a16(x1) : x1;
    };

    v4f acc[4][CB];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    constexpr int kDepth = Shape::kDepth;
    TileStage<WFMT, CB> st[kDepth];
    GroupScales<WFMT, Shape::kLdsScales ? 0 : GS, CB> sc;
    sc.init(srow, kb);
    if constexpr (Shape::kLdsScales) {
      // lane (ln, kb) holds groups [kb G/4, (kb+1) G/4) of its rows; made visible
      // by the barrier before the first group
      constexpr int kPer = GS / 4;
  #pragma unroll
      for (int j = 0; j < CB; ++j)
  #pragma unroll
        for (int i = 0; i < kPer; i += 4) {
          float fv[4];
          load_scales<4>(srow[j] + kb * kPer + i, fv);
  #pragma unroll
          for (int t = 0; t < 4; ++t) Ss[(((kb * kPer + i + t) * 4 + wave) * 16 + ln) * CB + j] = fv[t];
        }
    }
    auto issue = [&](int slot, int g) {
      if (st_on) {
        st[slot].a0 = *reinterpret_cast<const uint4*>(a_src0 + g * 128);
        st[slot].a1 = *reinterpret_cast<const uint4*>(a_src1 + g * 128);
      }
  #pragma unroll
      for (int j = 0; j < CB; ++j) {
        st[slot].b[j].template load<CP>(wblk[j], g * kGroupStride<WFMT>, wlane);
        if constexpr (!Shape::kLdsScales) st[slot].s[j] = sc.load(j, g);
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
      OperandT<WFMT> bop[CB];
      float sg[CB];
  #pragma unroll
      for (int j = 0; j < CB; ++j) bop[j] = st[slot].b[j].operand();
      if constexpr (Shape::kLdsScales) {
        const float4 f = *reinterpret_cast<const float4*>(&Ss[((g * 4 + wave) * 16 + ln) * CB]);
        sg[0] = f.x; sg[1] = f.y; sg[2] = f.z; sg[3] = f.w;
      } else {
  #pragma unroll
        for (int j = 0; j < CB; ++j) sg[j] = sc.get(j, g, ln, st[slot].s[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(slot, g + kDepth);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nrb) {
          const uint4* ap = reinterpret_cast<const uint4*>(&As[buf][(16 * i + ln) * kRowDw + kb * 8]);
          const OperandT<WFMT> aop = a_operand_staged<WFMT>(ap[0], ap[1]);
  #pragma unroll
          for (int j = 0; j < CB; ++j) accumulate<WFMT>(acc[i][j], aop, bop[j], sg[j]);
        }
      }
      if (more) store_a(buf ^ 1, x0, x1);
      __syncthreads();
    };
    pipeline<kDepth, GS>(G, issue, consume);

    if (!out_f32 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      // bf16 output: each value as store_block forms it, parked in LDS (over
      // the group scales, which the sweep's last barrier has retired), then
      // the tile's rows written 16 bytes per lane (a lane holds one column of
      // four rows per block, which stored directly is a 2-byte store each)
      float rs[CB];
      row_scales<WFMT, CB>(srow, rs);
      const int oc0 = EPI == MOEQ_EPI_SILU_MUL ? nt * (BN / 2) : nt * BN;   // first output column
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nrb) {
  #pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r_in = 16 * i + 4 * kb + v;
            if (r_in >= ti.rows) continue;
            const float sa = a_s[ti.row0 + r_in];
            uint16_t* orow = reinterpret_cast<uint16_t*>(Os + r_in * OS);
            if constexpr (EPI == MOEQ_EPI_SILU_MUL) {
  #pragma unroll
              for (int j = 0; j < CB / 2; ++j) {
                const float v0 = sa * acc[i][j][v] * rs[j];
                const float v1 = sa * acc[i][j + CB / 2][v] * rs[j + CB / 2];
                orow[col[j] - oc0 + ln] = f32_to_bf16(silu_f32(v0) * v1);
              }
            } else {
  #pragma unroll
              for (int j = 0; j < CB; ++j)
                orow[col[j] - oc0 + ln] = f32_to_bf16(sa * acc[i][j][v] * rs[j]);
            }
          }
        }
      }
      __syncthreads();
      constexpr int CPR = OC * 2 / 16;               // 16-byte chunks of an output row
      const int ldo = EPI == MOEQ_EPI_SILU_MUL ? N / 2 : N;
      uint16_t* o16 = static_cast<uint16_t*>(out);
      for (int idx = tid; idx < ti.rows * CPR; idx += kThreads) {
        const int r = idx / CPR, c = idx - r * CPR;
        *reinterpret_cast<uint4*>(o16 + int64_t(ti.row0 + r) * ldo + oc0 + 8 * c) =
            *reinterpret_cast<const uint4*>(Os + r * OS + 16 * c);
      }
      return;
    }
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nrb) {
        v4f blk[CB];
  #pragma unroll
        for (int j = 0; j < CB; ++j) blk[j] = acc[i][j];
        store_block<WFMT, EPI, CB>(blk, i, ti.row0, ti.rows, [a_s](int p, int) { return a_s[p]; }, srow,
                                   col, ln, kb, N, out, out_f32);
      }
    }
  };
  if (ti.shared_w) body(std::integral_constant<int, kCpKeep>());
  else body(std::integral_constant<int, kCpStream>());
}

template <int WFMT, int EPI, int GS>
hipError_t launch_kernels(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                          const uint8_t* w, const ScaleT<WFMT>* w_scale, int N, int K, void* out,
                          int out_f32, hipStream_t stream) {
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (R <= kWaveMaxRows) {
    // few rows per expert: one workgroup per K-split unit (tile, 16 NB weight rows)
    constexpr int NB = (EPI == MOEQ_EPI_SILU_MUL) ? 2 : MOEQ_WAVE_NB;
    const int64_t units = int64_t(plan_max_tiles(E, R)) * (N / (16 * NB));
    hipLaunchKernelGGL((gemm_wave_kernel<WFMT, EPI, GS, NB>), dim3(unsigned(units)),
                       dim3(kThreads), 0, stream, a_q, a_s, p, E, R, w, w_scale, N, K, out,
                       out_f32);
  } else {
    auto tile = [&](auto cb) {
      constexpr int CB = decltype(cb)::value;
      // one block per possible work item (the plan's tile count is known on the
      // device only)
      const int64_t grid = int64_t(N / (64 * CB)) * plan_max_tiles(E, R);
      hipLaunchKernelGGL((gemm_tile_kernel<WFMT, EPI, GS, CB>), dim3(unsigned(grid)),
                         dim3(kThreads), 0, stream, a_q, a_s, p, E, R, w, w_scale, N, K, out,
                         out_f32);
    };
    if constexpr (kIsW4<WFMT> && GS > 0) {
      if (N % 256 == 0) tile(std::integral_constant<int, 4>());
      else tile(std::integral_constant<int, 2>());
    } else {
      tile(std::integral_constant<int, 2>());
    }
  }
  return hipGetLastError();
}

// K = 4096 and K = 2048 (the hidden size and the expert width of the layer) get
// fully unrolled K sweeps; any other multiple of 128 uses the looped sweep.
template <int WFMT, int EPI>
hipError_t launch_shape(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                        const uint8_t* w, const ScaleT<WFMT>* w_scale, int N, int K, void* out,
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
                      const uint8_t* w, const ScaleT<WFMT>* w_scale, int N, int K, int epilogue,
                      void* out,
                      int out_f32, hipStream_t stream) {
  if (epilogue == MOEQ_EPI_SILU_MUL)
    return launch_shape<WFMT, MOEQ_EPI_SILU_MUL>(a_q, a_s, plan, E, R, w, w_scale, N, K, out,
                                                 out_f32, stream);
  return launch_shape<WFMT, MOEQ_EPI_NONE>(a_q, a_s, plan, E, R, w, w_scale, N, K, out, out_f32,
                                           stream);
}

}  // namespace

hipError_t launch_grouped_gemm(int wfmt, const uint8_t* a_q, const float* a_s, const void* plan,
                               int E, int R, const uint8_t* w, const void* w_scale, int N, int K,
                               int epilogue, void* out, int out_dtype, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int out_f32 = out_dtype == MOEQ_F32 ? 1 : 0;
  switch (wfmt) {
    case kW4G128:
      return launch_fmt<kW4G128>(a_q, a_s, plan, E, R, w, static_cast<const float*>(w_scale), N, K,
                                 epilogue, out, out_f32, stream);
    case kW4G128Bf16:
      return launch_fmt<kW4G128Bf16>(a_q, a_s, plan, E, R, w,
                                     static_cast<const uint16_t*>(w_scale), N, K, epilogue, out,
                                     out_f32, stream);
    default:
      return launch_fmt<kFp8Row>(a_q, a_s, plan, E, R, w, static_cast<const float*>(w_scale), N, K,
                                 epilogue, out, out_f32, stream);
  }
}

}  // namespace moeq
