// Grouped GEMM over routed experts on the gfx950 FP8 matrix cores.
//
//   out[p, n] = epilogue( a_s[p] * sum_g s_w[e, n, g] * sum_{k in g} a[p, k] * W[e, n, k] )
//
// Weight formats:
//   kW4G128 -- INT4 codes, two per byte (low nibble first), one fp32 scale per
//              (output row, 128-wide K group).  Each code is converted exactly to
//              its OCP E4M3 byte with two v_perm_b32 table lookups and an xor, so
//              the products run on v_mfma_f32_16x16x128_f8f6f4 (FP8 x FP8, fp32
//              accumulate).  One MFMA covers exactly one 128-wide group: its fp32
//              result is the group's partial sum, which is scaled by the group
//              scale and added to the running fp32 accumulator.
//   kFp8Row -- E4M3 weights with one fp32 scale per output row: the MFMA
//              accumulates over all of K and the row scale is applied at the end.
//
// MFMA operand layout (16x16x128, 8 VGPRs per operand): lane (r = l % 16,
// kb = l / 16) supplies 32 K-values of row r; the result lane l holds column
// l % 16 of rows 4 (l / 16) + v, v = 0..3.  The MFMA sums over K, so any K
// permutation applied identically to both operands leaves the result unchanged:
// lane kb takes K-range [32 kb, 32 kb + 32) of the group, and for INT4 weights
// the activation bytes of each 8-byte chunk are reordered to (0,2,4,6,1,3,5,7),
// the order in which the nibble unpack produces the codes (low nibbles, then
// high nibbles).
//
// Each wave owns two 16-column blocks of weight rows: for EPI_NONE 32
// consecutive output columns, for EPI_SILU_MUL 16 gate rows and the matching 16
// up rows (N/2 further), so the SiLU-gated product forms in registers.  A lane
// streams 16 B of packed weights (32 codes) per block per group: lane (n, kb)
// reads bytes [16 kb, 16 kb + 16) of its row's 64-byte group.  Weight loads run
// kDepth groups ahead of their use (a register ring, unrolled so every ring
// index is static) to keep enough bytes in flight to cover HBM latency.
//
// Two kernels share this arithmetic:
//  * wave kernel (few rows per expert, e.g. decode): every wave is independent.
//    Its unit is (plan tile, 32 weight rows); it reads its own activation
//    fragment straight from global memory (tiny, cache-resident), so there is
//    no LDS and no barrier in the K loop.  Tiles with more than 16 rows are swept
//    once per 16-row block.
//  * tile kernel (prefill): a 256-thread workgroup owns one plan tile (<= 64
//    rows) x 128 weight rows.  The 64 x 128 B activation slice of each group is
//    staged once in LDS (double-buffered, one barrier per group) and shared by
//    the four waves, each of which runs all four 16-row blocks against its own
//    32 weight rows.  The linear workgroup id is remapped so that each XCD
//    (workgroups are dispatched to the 8 XCDs round-robin) receives a contiguous
//    run of (tile, N-tile) pairs: the N-tiles of one row tile share that tile's
//    activations in one L2.
// Both grids are sized on the host from R alone; units past the plan's tile
// count exit at once, so nothing is read back from the device.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 128;           // weight rows per tile-kernel workgroup
constexpr int kRowDw = 36;         // LDS row stride in dwords (128 B + 16 B pad)
constexpr int kXcds = 8;
// weight groups in flight per wave (an FP8 group carries twice the bytes of an INT4
// one); the tile kernel's ring also holds each group's activation share, so it
// runs one group shallower to stay at three waves per SIMD
#ifndef MOEQ_W4_DEPTH
#define MOEQ_W4_DEPTH 4
#endif
#ifndef MOEQ_FP8_DEPTH
#define MOEQ_FP8_DEPTH 2
#endif
#ifndef MOEQ_TILE_W4_DEPTH
#define MOEQ_TILE_W4_DEPTH 3
#endif
template <int WFMT>
struct Depth { static constexpr int value = (WFMT == kW4G128) ? MOEQ_W4_DEPTH : MOEQ_FP8_DEPTH; };
template <int WFMT>
struct TileDepth {
  static constexpr int value = (WFMT == kW4G128) ? MOEQ_TILE_W4_DEPTH : MOEQ_FP8_DEPTH;
};

// INT4 nibble (code + 8) -> E4M3 byte of the code, four nibbles (one per byte,
// values 0..15) at a time.  v_perm_b32 looks bytes up in an 8-byte table; a
// selector byte of 8..11 yields the replicated sign bit of table byte 1/3/5/7,
// 12 yields 0x00 and 13..15 yield 0xFF.  With the raw nibble as selector into
// table T and (nibble & 7) into table U, T[n] ^ U[n] is the answer for n < 8 and
// special(n) ^ U[n - 8] for n >= 8; the tables below satisfy both.
constexpr uint32_t kLutT0 = 0x8E8C09D0u, kLutT1 = 0x09737180u;
constexpr uint32_t kLutU0 = 0x4440C700u, kLutU1 = 0xB1B3B548u;

__device__ __forceinline__ uint32_t nib4_to_e4m3(uint32_t n4, uint32_t n4_low3) {
  return __builtin_amdgcn_perm(kLutT1, kLutT0, n4) ^ __builtin_amdgcn_perm(kLutU1, kLutU0, n4_low3);
}

// 16 packed bytes (32 codes) -> the 32 E4M3 bytes of one MFMA operand, in the
// order (codes 0,2,4,6)(1,3,5,7)(8,10,12,14)(9,11,13,15)...
__device__ __forceinline__ v8i unpack_w4(const uint4& p) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sh = w[i] >> 4;
    r[2 * i] = int(nib4_to_e4m3(w[i] & 0x0F0F0F0Fu, w[i] & 0x07070707u));
    r[2 * i + 1] = int(nib4_to_e4m3(sh & 0x0F0F0F0Fu, sh & 0x07070707u));
  }
  return r;
}

// activation bytes of one lane (32 consecutive K) -> operand order matching unpack_w4
__device__ __forceinline__ v8i shuffle_a(const uint4& x0, const uint4& x1) {
  const uint32_t d[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = int(__builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x06040200u));
    r[2 * i + 1] = int(__builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07050301u));
  }
  return r;
}

__device__ __forceinline__ v8i as_v8i(const uint4& x0, const uint4& x1) {
  v8i r;
  r[0] = int(x0.x); r[1] = int(x0.y); r[2] = int(x0.z); r[3] = int(x0.w);
  r[4] = int(x1.x); r[5] = int(x1.y); r[6] = int(x1.z); r[7] = int(x1.w);
  return r;
}

// One group scale.  A relaxed atomic load: the compiler may neither merge the
// scale loads of different groups into wide loads hoisted ahead of the K sweep
// (which costs registers and spills in the unrolled sweep) nor move them.
__device__ __forceinline__ float load_scale(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// weight fragment of one lane for one 16-row block and one group
template <int WFMT>
struct BFrag;

template <>
struct BFrag<kW4G128> {
  uint4 raw;
  __device__ __forceinline__ void load(const uint8_t* row, int g, int kb) {
    raw = *reinterpret_cast<const uint4*>(row + g * 64 + kb * 16);
  }
  __device__ __forceinline__ v8i operand() const { return unpack_w4(raw); }
};

template <>
struct BFrag<kFp8Row> {
  uint4 raw0, raw1;
  __device__ __forceinline__ void load(const uint8_t* row, int g, int kb) {
    const uint4* p = reinterpret_cast<const uint4*>(row + g * 128 + kb * 32);
    raw0 = p[0];
    raw1 = p[1];
  }
  __device__ __forceinline__ v8i operand() const { return as_v8i(raw0, raw1); }
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands FP8 E4M3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

struct TileInfo {
  int e, row0, rows;
};

__device__ __forceinline__ TileInfo tile_info(const int32_t* plan, int E, int R, int tile) {
  const PlanView pv = plan_view(const_cast<int32_t*>(plan), E, R);
  TileInfo t;
  t.e = pv.tile_expert[tile];
  t.row0 = pv.tile_row0[tile];
  t.rows = min(MOEQ_TILE_M, pv.offsets[t.e + 1] - t.row0);
  return t;
}

// weight-row bases (16-row block j of this wave) and their scale rows
template <int WFMT>
__device__ __forceinline__ void weight_rows(const uint8_t* w, const float* w_scale, int e, int N,
                                            int K, const int (&col)[2], int ln,
                                            const uint8_t* (&wrow)[2], const float* (&srow)[2]) {
  const int64_t row_bytes = (WFMT == kW4G128) ? (K >> 1) : K;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n_glob = int64_t(e) * N + col[j] + ln;
    wrow[j] = w + n_glob * row_bytes;
    srow[j] = (WFMT == kW4G128) ? (w_scale + n_glob * (K >> 7)) : (w_scale + n_glob);
  }
}

// epilogue for one 16-row block: lane holds rows 4 kb + v, column col[j] + ln
template <int WFMT, int EPI>
__device__ __forceinline__ void store_block(const v4f (&acc)[2], int rb, int row0, int rows,
                                            const float* a_s, const float* const (&srow)[2],
                                            const int (&col)[2], int ln, int kb, int N, void* out,
                                            int out_f32) {
  float rs[2] = {1.f, 1.f};
  if (WFMT == kFp8Row) {
    rs[0] = srow[0][0];
    rs[1] = srow[1][0];
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r_in = 16 * rb + 4 * kb + v;
    if (r_in >= rows) continue;
    const int p = row0 + r_in;
    const float sa = a_s[p];
    const float v0 = sa * acc[0][v] * rs[0];
    const float v1 = sa * acc[1][v] * rs[1];
    if (EPI == MOEQ_EPI_SILU_MUL) {
      uint16_t* o = static_cast<uint16_t*>(out) + int64_t(p) * (N >> 1);
      o[col[0] + ln] = f32_to_bf16(silu_f32(v0) * v1);
    } else if (out_f32) {
      float* o = static_cast<float*>(out) + int64_t(p) * N;
      o[col[0] + ln] = v0;
      o[col[1] + ln] = v1;
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + int64_t(p) * N;
      o[col[0] + ln] = f32_to_bf16(v0);
      o[col[1] + ln] = f32_to_bf16(v1);
    }
  }
}

// An empty volatile asm that reads and writes the accumulator: it is ordered
// with the surrounding memory operations and scheduling barriers, so the
// arithmetic producing the accumulator cannot drift past it.
__device__ __forceinline__ void pin(v4f& a) {
  asm volatile("" : "+v"(a));
}

template <int WFMT>
__device__ __forceinline__ void accumulate(v4f& acc, const v8i& a, const v8i& b, float s) {
  if (WFMT == kW4G128) {
    const v4f part = mfma_fp8(a, b, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = fmaf(s, part[v], acc[v]);
  } else {
    acc = mfma_fp8(a, b, acc);
  }
}

// Runs consume(slot, g, refill) for g = 0 .. G-1 over a ring of kDepth slots
// that issue(slot, g) fills kDepth groups ahead.  With GS > 0 (G == GS known at
// compile time) the whole sweep is unrolled: no value is carried around a loop
// back-edge, so every load lands directly in its slot's registers and stays in
// flight until its use.  GS == 0 handles any G with a runtime loop.
template <int kDepth, int GS, typename IssueF, typename ConsumeF>
__device__ __forceinline__ void pipeline(int G, IssueF&& issue, ConsumeF&& consume) {
  if constexpr (GS > 0) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < GS) issue(d, d);
#pragma unroll
    for (int g = 0; g < GS; ++g) consume(g % kDepth, g, g + kDepth < GS);
  } else {
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < G) issue(d, d);
    int g0 = 0;
    for (; g0 + 2 * kDepth <= G; g0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) consume(d, g0 + d, true);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (g0 + d < G) consume(d, g0 + d, g0 + d + kDepth < G);
    g0 += kDepth;
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (g0 + d < G) consume(d, g0 + d, false);
  }
}

// Group scales of this lane's two weight rows (col[0] + ln and col[1] + ln).
// With G = GS known at compile time the G scales of a row are spread over its
// four lanes (ln, kb): lane kb holds groups [kb G/4, (kb+1) G/4), fetched with
// 16-byte loads once per sweep, and the scale of group g comes from lane
// (ln, g / (G/4)) by a cross-lane read.  This keeps the per-group scale reads
// (16 rows x 4 bytes, 16 cache lines per instruction) out of the vector memory
// pipeline, which they would otherwise congest as much as the weights do.
// Otherwise (any G) one load per row and group.
template <int WFMT, int GS>
struct GroupScales {
  static constexpr bool kPreload = (WFMT == kW4G128) && GS > 0 && GS % 16 == 0;
  static constexpr int kPerLane = kPreload ? GS / 4 : 1;
  float v[2][kPerLane];
  const float* row[2];

  __device__ __forceinline__ void init(const float* const (&srow)[2], int kb) {
    row[0] = srow[0];
    row[1] = srow[1];
    if constexpr (kPreload) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < kPerLane; i += 4) {
          const float4 f = *reinterpret_cast<const float4*>(srow[j] + kb * kPerLane + i);
          v[j][i] = f.x; v[j][i + 1] = f.y; v[j][i + 2] = f.z; v[j][i + 3] = f.w;
        }
    }
  }
  // scale of group g for block j; `held` is the value a ring stage loaded (non-preload path)
  __device__ __forceinline__ float get(int j, int g, int ln, float held) const {
    if constexpr (kPreload) {
      return __shfl(v[j][g % kPerLane], ln + 16 * (g / kPerLane), 64);
    } else {
      return held;
    }
  }
  __device__ __forceinline__ float load(int j, int g) const {
    if constexpr (kPreload || WFMT != kW4G128) return 1.0f;
    else return load_scale(row[j] + g);
  }
};

// ------------------------------------------------------------- wave kernel
template <int WFMT>
struct WaveStage {
  uint4 a0, a1;          // 32 activation bytes of this lane's row
  BFrag<WFMT> b[2];      // weight fragments of the two 16-row blocks
  float s[2];            // their group scales (INT4 only)
};

// The operand pointers are deliberately not __restrict__: loads through
// restrict-qualified read-only pointers may be hoisted by instruction selection
// past the scheduling barriers below, which pulls the whole unrolled sweep's
// loads to the top of the kernel and spills them.
template <int WFMT, int EPI, int GS>
__global__ void __launch_bounds__(kThreads, 3)   // >= 3 waves per SIMD
gemm_wave_kernel(const uint8_t* a_q, const float* a_s, const int32_t* plan, int E, int R,
                 const uint8_t* w, const float* w_scale, int N, int K, void* out, int out_f32) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kb = lane >> 4;
  const int units_per_tile = N >> 5;
  const int unit = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int tile = unit / units_per_tile;
  const int u = unit - tile * units_per_tile;
  if (tile >= plan[kPlanTiles]) return;                 // wave-uniform
  const TileInfo ti = tile_info(plan, E, R, tile);
  const int G = K >> 7;

  int col[2];
  if (EPI == MOEQ_EPI_SILU_MUL) {
    col[0] = 16 * u;
    col[1] = (N >> 1) + 16 * u;
  } else {
    col[0] = 32 * u;
    col[1] = 32 * u + 16;
  }
  const uint8_t* wrow[2];
  const float* srow[2];
  weight_rows<WFMT>(w, w_scale, ti.e, N, K, col, ln, wrow, srow);

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    // lanes past the tile's rows read its first row: MFMA rows are independent
    // and those rows are never stored
    // Only lanes of real rows load activations (the others keep zeros): MFMA
    // rows are independent and rows past the tile are never stored.
    const bool a_ok = 16 * rb + ln < ti.rows;
    const uint8_t* a_src = a_q + int64_t(ti.row0 + (a_ok ? 16 * rb + ln : 0)) * K + kb * 32;
    constexpr int kDepth = Depth<WFMT>::value;
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    WaveStage<WFMT> st[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      st[d].a0 = make_uint4(0, 0, 0, 0);
      st[d].a1 = st[d].a0;
    }
    GroupScales<WFMT, GS> sc;
    sc.init(srow, kb);

    auto issue = [&](int slot, int g) {
      WaveStage<WFMT>& s = st[slot];
      if (a_ok) {
        const uint4* ap = reinterpret_cast<const uint4*>(a_src + g * 128);
        s.a0 = ap[0];
        s.a1 = ap[1];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        s.b[j].load(wrow[j], g, kb);
        s.s[j] = sc.load(j, g);
      }
    };
    auto consume = [&](int slot, int g, bool refill) {
      const WaveStage<WFMT>& s = st[slot];
      const v8i aop = (WFMT == kW4G128) ? shuffle_a(s.a0, s.a1) : as_v8i(s.a0, s.a1);
      const v8i b0 = s.b[0].operand();
      const v8i b1 = s.b[1].operand();
      const float s0 = sc.get(0, g, ln, s.s[0]), s1 = sc.get(1, g, ln, s.s[1]);
      // refill this ring slot only after the last read of its old contents
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(slot, g + kDepth);
      accumulate<WFMT>(acc[0], aop, b0, s0);
      accumulate<WFMT>(acc[1], aop, b1, s1);
      // Pin this group's arithmetic before the next group's: without it the
      // instruction selector defers the scale FMAs to the end of the unrolled
      // sweep and keeps every group's MFMA result live.
      pin(acc[0]);
      pin(acc[1]);
    };
    pipeline<kDepth, GS>(G, issue, consume);
    store_block<WFMT, EPI>(acc, rb, ti.row0, ti.rows, a_s, srow, col, ln, kb, N, out, out_f32);
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
      store_block<WFMT, EPI>(blk, i, ti.row0, ti.rows, a_s, srow, col, ln, kb, N, out, out_f32);
    }
  }
}

template <int WFMT, int EPI, int GS>
hipError_t launch_kernels(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                          const uint8_t* w, const float* w_scale, int N, int K, void* out,
                          int out_f32, hipStream_t stream) {
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (R <= 64) {
    // few rows per expert: independent waves, one per (tile, 32 weight rows)
    const int64_t units = int64_t(plan_max_tiles(E, R)) * (N >> 5);
    const int64_t blocks = (units + 3) / 4;
    hipLaunchKernelGGL((gemm_wave_kernel<WFMT, EPI, GS>), dim3(unsigned(blocks)), dim3(kThreads),
                       0, stream, a_q, a_s, p, E, R, w, w_scale, N, K, out, out_f32);
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
