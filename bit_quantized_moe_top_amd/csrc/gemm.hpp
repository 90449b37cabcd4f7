// Grouped GEMM over routed experts on the gfx950 FP8 matrix cores: the device
// building blocks shared by the grouped GEMM kernels (gemm.hip) and the fused
// expert MLP (mlp.hip).
//
//   out[p, n] = epilogue( a_s[p] * sum_g s_w[e, n, g] * sum_{k in g} a[p, k] * W[e, n, k] )
//
// Weight formats:
//   kW4G128 -- INT4 codes, two per byte (low nibble first), one fp32 scale per
//              (output row, 128-wide K group); kW4G128Bf16 the same with
//              bfloat16 scales (converted to fp32 as they are read).  Each code is converted exactly to
//              its OCP E4M3 byte with two v_perm_b32 table lookups and an xor, so
//              the products run on v_mfma_f32_16x16x128_f8f6f4 (FP8 x FP8, fp32
//              accumulate).  One MFMA covers exactly one 128-wide group: its fp32
//              result is the group's partial sum, which is scaled by the group
//              scale and added to the running fp32 accumulator.
//   kFp8Row -- E4M3 weights with one fp32 scale per output row: each MFMA's
//              128-wide partial sum is added to the fp32 accumulator and the row
//              scale is applied at the end.
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
// reads bytes [16 kb, 16 kb + 16) of its row's 64-byte group.  INT4 weights are
// read in the library's tiled order (16-row blocks stored group after group), so
// the 16 rows x 64 B that one load instruction of a wave takes are 1024
// contiguous bytes rather than 16 pieces 2 KB apart.  Weight loads run
// kDepth groups ahead of their use (a register ring, unrolled so every ring
// index is static) to keep enough bytes in flight to cover HBM latency.
//
// Two GEMM kernels share this arithmetic (the fused expert MLP runs the wave
// kernel's units):
//  * wave kernel (few rows per expert, e.g. decode): a 256-thread workgroup per
//    unit (plan tile, 32 weight rows); wave q sweeps K quarter q, with the
//    block's activation quarter staged in LDS when it has at most 4 rows (read
//    from global memory otherwise), and the four partial sums meet in LDS at
//    one barrier after the sweep.  Tiles with more than 16 rows are swept once
//    per 16-row block.
//  * tile kernel (prefill): a 256-thread workgroup owns one plan tile (<= 64
//    rows) x 128 or 256 weight rows.  The 64 x 128 B activation slice of each
//    group is staged once in LDS (double-buffered, one barrier per group) and
//    shared by the four waves, each of which runs all four 16-row blocks
//    against its own 32 or 64 weight rows.  The linear workgroup id is remapped so that each XCD
//    (workgroups are dispatched to the 8 XCDs round-robin) receives a contiguous
//    run of (tile, N-tile) pairs: the N-tiles of one row tile share that tile's
//    activations in one L2.
// Both grids are sized on the host from R alone; units past the plan's tile
// count exit at once, so nothing is read back from the device.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
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
// INT4 weights (either scale type)
template <int WFMT>
constexpr bool kIsW4 = (WFMT == kW4G128 || WFMT == kW4G128Bf16);

// element type of the weight scales
template <int WFMT>
struct ScaleOf { using type = float; };
template <>
struct ScaleOf<kW4G128Bf16> { using type = uint16_t; };
template <>
struct ScaleOf<kNvfp4> { using type = uint8_t; };      // E4M3 block scales
template <>
struct ScaleOf<kAqlm> { using type = _Float16; };      // per-row fp16 scales
template <int WFMT>
using ScaleT = typename ScaleOf<WFMT>::type;

__device__ __forceinline__ float scale_value(float s) { return s; }
__device__ __forceinline__ float scale_value(uint16_t s) { return bf16_to_f32(s); }
__device__ __forceinline__ float scale_value(_Float16 s) { return static_cast<float>(s); }

// n consecutive scales (n = 1, 2 or a multiple of 4; p aligned to n scales)
// starting at p, as fp32: one vector load per 4 scales (16 bytes fp32, 8 bf16)
template <int n>
__device__ __forceinline__ void load_scales(const float* p, float* out) {
  if constexpr (n == 1) {
    out[0] = p[0];
  } else if constexpr (n == 2) {
    const float2 f = *reinterpret_cast<const float2*>(p);
    out[0] = f.x; out[1] = f.y;
  } else {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
      const float4 f = *reinterpret_cast<const float4*>(p + i);
      out[i] = f.x; out[i + 1] = f.y; out[i + 2] = f.z; out[i + 3] = f.w;
    }
  }
}
template <int n>
__device__ __forceinline__ void load_scales(const uint16_t* p, float* out) {
  if constexpr (n == 1) {
    out[0] = u2f(uint32_t(p[0]) << 16);
  } else if constexpr (n == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    out[0] = u2f(u << 16); out[1] = u2f(u & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p + i);
      out[i] = u2f(u.x << 16); out[i + 1] = u2f(u.x & 0xFFFF0000u);
      out[i + 2] = u2f(u.y << 16); out[i + 3] = u2f(u.y & 0xFFFF0000u);
    }
  }
}

template <int WFMT>
struct Depth { static constexpr int value = kIsW4<WFMT> ? MOEQ_W4_DEPTH : MOEQ_FP8_DEPTH; };
template <int WFMT>
struct TileDepth {
  static constexpr int value = kIsW4<WFMT> ? MOEQ_TILE_W4_DEPTH : MOEQ_FP8_DEPTH;
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

// the same reorder for one 16-byte piece (two independent 8-byte units)
__device__ __forceinline__ uint4 shuffle_a16(const uint4& x) {
  return make_uint4(__builtin_amdgcn_perm(x.y, x.x, 0x06040200u),
                    __builtin_amdgcn_perm(x.y, x.x, 0x07050301u),
                    __builtin_amdgcn_perm(x.w, x.z, 0x06040200u),
                    __builtin_amdgcn_perm(x.w, x.z, 0x07050301u));
}

__device__ __forceinline__ v8i as_v8i(const uint4& x0, const uint4& x1) {
  v8i r;
  r[0] = int(x0.x); r[1] = int(x0.y); r[2] = int(x0.z); r[3] = int(x0.w);
  r[4] = int(x1.x); r[5] = int(x1.y); r[6] = int(x1.z); r[7] = int(x1.w);
  return r;
}

__device__ __forceinline__ v4f mfma_f16(const h8& a, const h8& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E4M3 bytes (two dwords) -> 8 f16, exact (every E4M3 value is an f16 value)
__device__ __forceinline__ h8 fp8x8_to_f16(uint32_t d0, uint32_t d1) {
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 K-values of one row as four f16 operands of v_mfma_f32_16x16x32_f16:
// m[j] holds the lane's bytes 8 j .. 8 j + 7, so MFMA j of a 128-K group sums
// K 32 kb + 8 j + (0..7) over the lanes kb -- each K once, the same mapping for
// both operands.
struct F16x32 {
  h8 m[4];
};
__device__ __forceinline__ F16x32 fp8x32_to_f16(const uint4& x0, const uint4& x1) {
  F16x32 r;
  r.m[0] = fp8x8_to_f16(x0.x, x0.y);
  r.m[1] = fp8x8_to_f16(x0.z, x0.w);
  r.m[2] = fp8x8_to_f16(x1.x, x1.y);
  r.m[3] = fp8x8_to_f16(x1.z, x1.w);
  return r;
}

// One group scale.  A relaxed atomic load: the compiler may neither merge the
// scale loads of different groups into wide loads hoisted ahead of the K sweep
// (which costs registers and spills in the unrolled sweep) nor move them.
__device__ __forceinline__ float load_scale(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_scale(const uint16_t* p) {
  return bf16_to_f32(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// weight fragment of one lane for one 16-row block and one group
template <int WFMT>
struct BFrag;

// Bytes between consecutive 128-K groups of a weight block: INT4 in the tiled
// order (a group of a 16-row block is 16 x 64 contiguous bytes), FP8-row in
// rows (the next 128 bytes of each row).
template <int WFMT>
constexpr int kGroupStride = kIsW4<WFMT> ? 16 * 64 : 128;

// 16 bytes at base + off + lane by a buffer load: base (the weight block's first
// byte) goes into a buffer resource and off (the group's group_offset) into the
// scalar offset, both wave-uniform; only the lane's 32-bit offset lane is a
// vector register, shared by every load of a sweep.  (A flat global load would
// need a 64-bit vector address per load once off is not a compile-time
// constant, and the unrolled sweep would run out of registers.)  Word 3 of the
// resource: 32-bit data format, the setting for untyped buffer access on gfx9;
// the record count is the largest the 32-bit offsets can reach.
// CP is the load's cache policy: kCpStream (the non-temporal bit) for weights
// that no other workgroup reads again -- a 1 GiB streaming read runs 7% faster
// with it (5.75 against 5.41 TB/s, measured) -- kCpKeep for weights that other
// row tiles of the same expert read again and should find in L2.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kCpKeep = 0, kCpStream = 2;
template <int CP>
__device__ __forceinline__ uint4 load_weight16(const uint8_t* base, int off, uint32_t lane) {
  const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(base), static_cast<short>(0), 0x7FFFFFFF, 0x00020000);
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(res, int(lane), off, CP);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// BFrag::load<CP>(base, off, lane): base the weight block's first byte, off the
// group's offset g kGroupStride (both wave-uniform), lane this lane's offset
// (weight_rows), CP the cache policy.
template <>
struct BFrag<kW4G128> {
  uint4 raw;
  template <int CP>
  __device__ __forceinline__ void load(const uint8_t* base, int off, uint32_t lane) {
    raw = load_weight16<CP>(base, off, lane);
  }
  __device__ __forceinline__ v8i operand() const { return unpack_w4(raw); }
};

template <>
struct BFrag<kW4G128Bf16> : BFrag<kW4G128> {};

// (FP8 rows keep the default policy whatever CP asks for: a row's 128-byte line
// is split over the fragment's two loads, and with the non-temporal bit the
// line fetched for the first half is not kept for the second -- the row-FP8
// prefill gate/up GEMM ran 20% slower with it)
template <>
struct BFrag<kFp8Row> {
  uint4 raw0, raw1;
  template <int CP>
  __device__ __forceinline__ void load(const uint8_t* base, int off, uint32_t lane) {
    raw0 = load_weight16<kCpKeep>(base, off, lane);
    raw1 = load_weight16<kCpKeep>(base, off, lane + 16);
  }
  __device__ __forceinline__ F16x32 operand() const { return fp8x32_to_f16(raw0, raw1); }
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands FP8 E4M3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// MFMA operand of each weight format: INT4 codes become E4M3 bytes for the FP8
// MFMA.  Row-scaled FP8 weights and their activations become f16 for the f16
// MFMA: the FP8 MFMAs sum their products in a narrower internal format (for
// products of two full-range E4M3 values the result was measured up to 2e-5 of
// the sum of the products' magnitudes away from the exact sum, against 3e-8 --
// fp32 rounding -- for the same products through v_mfma_f32_16x16x32_f16), which
// would leave the row-FP8 layer's h about 4x further from the exact values than
// the INT4 layer's (whose integer-valued weights keep the products' exponents
// close).  The f16 MFMA has half the FP8 rate; the row-FP8 layer streams 64
// weight bytes per 128 flops of each row and stays HBM-bound.
template <int WFMT>
struct OperandOf { using type = v8i; };
template <>
struct OperandOf<kFp8Row> { using type = F16x32; };
template <int WFMT>
using OperandT = typename OperandOf<WFMT>::type;

// a lane's 32 activation bytes as the format's operand (INT4: reordered to the
// order the nibble unpack produces; FP8-row: as f16)
template <int WFMT>
__device__ __forceinline__ OperandT<WFMT> a_operand(const uint4& x0, const uint4& x1) {
  if constexpr (WFMT == kFp8Row) return fp8x32_to_f16(x0, x1);
  else return shuffle_a(x0, x1);
}
// the same from bytes staged in LDS, where INT4 activations are kept reordered
template <int WFMT>
__device__ __forceinline__ OperandT<WFMT> a_operand_staged(const uint4& x0, const uint4& x1) {
  if constexpr (WFMT == kFp8Row) return fp8x32_to_f16(x0, x1);
  else return as_v8i(x0, x1);
}

struct TileInfo {
  int e, row0, rows;
  bool shared_w;         // a neighbouring tile in the list has the same expert
};

// The tile's expert, first row and row count, from one round of independent
// plan loads (nothing waits on the expert id): tiles list the active experts'
// rows in order, 64 at a time, so a tile's rows end where the next tile's
// begin, and the last tile's at offsets[E].  Returns whether tile is one of the
// plan's tiles (ti is meaningful only then); the loads stay inside the tile
// list for any tile >= 0.
__device__ __forceinline__ bool tile_info(const int32_t* plan, int E, int R, int tile,
                                          TileInfo& ti) {
  const PlanView pv = plan_view(const_cast<int32_t*>(plan), E, R);
  const int tl = min(tile, pv.max_tiles - 1);
  const int n = plan[kPlanTiles];
  const int e = pv.tile_expert[tl];
  const int e_prev = pv.tile_expert[max(tl - 1, 0)];
  const int e_next = pv.tile_expert[min(tl + 1, pv.max_tiles - 1)];
  const int row0 = pv.tile_row0[tl];
  const int next = pv.tile_row0[min(tl + 1, pv.max_tiles - 1)];
  const int end_all = pv.offsets[E];
  // Every value is consumed here, ahead of the caller's exit test: otherwise
  // the compiler sinks the loads the exit path does not need (and the kernel
  // arguments they address with) below the test, and the lookup takes several
  // scalar memory round trips in a row instead of one.  The values are uniform
  // over the caller's wave.
  asm volatile("" ::"s"(n), "s"(e), "s"(e_prev), "s"(e_next), "s"(row0), "s"(next), "s"(end_all));
  // clamped to the caller's E and R: a plan built for other sizes then yields
  // wrong rows, never an access outside the weight or activation buffers
  ti.e = min(max(e, 0), E - 1);
  ti.row0 = min(max(row0, 0), R);
  ti.rows = max(0, min(min(MOEQ_TILE_M, (tile + 1 < n ? next : end_all) - ti.row0), R - ti.row0));
  // (tiles of one expert are consecutive in the list; entries past the list's
  // end may hold anything, which only affects a cache policy)
  ti.shared_w = (tl > 0 && e_prev == e) || (tl + 1 < n && e_next == e);
  return tile < n;
}

// Weights of the 16-row blocks j of this wave (rows col[j] .. col[j] + 15 of
// expert e, col[j] a multiple of 16 and wave-uniform): wblk[j] the block's first
// byte (16 rows x K/2 bytes per INT4 block, K bytes per FP8 row), srow[j] the
// scales of this lane's row col[j] + ln, and lane the lane's byte offset inside
// a block's group (INT4 tiled order: row ln at 64 ln, bytes 16 kb; FP8 rows:
// row ln at ln K, bytes 32 kb).
template <int WFMT, int NB = 2>
__device__ __forceinline__ void weight_rows(const uint8_t* w, const ScaleT<WFMT>* w_scale, int e,
                                            int N, int K, const int (&col)[NB], int ln, int kb,
                                            const uint8_t* (&wblk)[NB],
                                            const ScaleT<WFMT>* (&srow)[NB], uint32_t& lane) {
  lane = kIsW4<WFMT> ? uint32_t(ln * 64 + kb * 16) : uint32_t(ln * K + kb * 32);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t n_glob = int64_t(e) * N + col[j] + ln;
    wblk[j] = w + (int64_t(e) * N + col[j]) * (kIsW4<WFMT> ? (K >> 1) : K);
    srow[j] = kIsW4<WFMT> ? (w_scale + n_glob * (K >> 7)) : (w_scale + n_glob);
  }
}

// epilogue for one 16-row block: lane holds rows 4 kb + v, column col[j] + ln;
// row_scale(p, v) is the activation scale of sorted row p (v: its slot 0..3
// among this lane's four rows of the block, for scales held in registers)
// the weight-row scales applied at the end (row-scaled FP8 only)
template <int WFMT, int NB = 2>
__device__ __forceinline__ void row_scales(const ScaleT<WFMT>* const (&srow)[NB], float (&rs)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if constexpr (WFMT == kFp8Row || WFMT == kAqlm) rs[j] = scale_value(srow[j][0]);
    else rs[j] = 1.0f;
  }
}

// SiLU-gated product of result row v (gate block 0, up block 1) as bf16
__device__ __forceinline__ uint16_t silu_mul_bf16(const v4f (&acc)[2], int v, float sa,
                                                  const float (&rs)[2]) {
  const float v0 = sa * acc[0][v] * rs[0];
  const float v1 = sa * acc[1][v] * rs[1];
  return f32_to_bf16(silu_f32(v0) * v1);
}

// (EPI_SILU_MUL: blocks j < NB/2 gate rows, block j + NB/2 the matching up rows)
template <int WFMT, int EPI, int NB = 2, typename RowScaleF>
__device__ __forceinline__ void store_block(const v4f (&acc)[NB], int rb, int row0, int rows,
                                            RowScaleF&& row_scale,
                                            const ScaleT<WFMT>* const (&srow)[NB],
                                            const int (&col)[NB], int ln, int kb, int N, void* out,
                                            int out_f32) {
  float rs[NB];
  row_scales<WFMT, NB>(srow, rs);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r_in = 16 * rb + 4 * kb + v;
    if (r_in >= rows) continue;
    const int p = row0 + r_in;
    const float sa = row_scale(p, v);
    if constexpr (EPI == MOEQ_EPI_SILU_MUL && NB == 2) {
      uint16_t* o = static_cast<uint16_t*>(out) + int64_t(p) * (N >> 1);
      o[col[0] + ln] = silu_mul_bf16(acc, v, sa, rs);
    } else if constexpr (EPI == MOEQ_EPI_SILU_MUL) {
      // blocks j < NB/2 hold gate rows, block j + NB/2 the matching up rows
      uint16_t* o = static_cast<uint16_t*>(out) + int64_t(p) * (N >> 1);
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        const float v0 = sa * acc[j][v] * rs[j];
        const float v1 = sa * acc[j + NB / 2][v] * rs[j + NB / 2];
        o[col[j] + ln] = f32_to_bf16(silu_f32(v0) * v1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float vj = sa * acc[j][v] * rs[j];
        if (out_f32)
          static_cast<float*>(out)[int64_t(p) * N + col[j] + ln] = vj;
        else
          static_cast<uint16_t*>(out)[int64_t(p) * N + col[j] + ln] = f32_to_bf16(vj);
      }
    }
  }
}

// An empty volatile asm that reads and writes the accumulator: it is ordered
// with the surrounding memory operations and scheduling barriers, so the
// arithmetic producing the accumulator cannot drift past it.
__device__ __forceinline__ void pin(v4f& a) {
  asm volatile("" : "+v"(a));
}

// INT4: one FP8 MFMA per 128-K group from zero, its partial sum scaled by the
// group scale into the fp32 accumulator.  FP8-row: four f16 MFMAs accumulating
// into it directly (the row scale is applied at the end).
__device__ __forceinline__ void accumulate_op(v4f& acc, const v8i& a, const v8i& b, float s) {
  const v4f part = mfma_fp8(a, b, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = fmaf(s, part[v], acc[v]);
}
__device__ __forceinline__ void accumulate_op(v4f& acc, const F16x32& a, const F16x32& b, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = mfma_f16(a.m[j], b.m[j], acc);
}
template <int WFMT>
__device__ __forceinline__ void accumulate(v4f& acc, const OperandT<WFMT>& a,
                                           const OperandT<WFMT>& b, float s) {
  accumulate_op(acc, a, b, s);
}

// Runs consume(slot, g, refill) for g = 0 .. G-1 over a ring of kDepth slots
// that issue(slot, g) fills kDepth groups ahead (the first kDepth issues are
// left to the caller when kPrologue is false).  With GS > 0 (G == GS known at
// compile time) the whole sweep is unrolled: no value is carried around a loop
// back-edge, so every load lands directly in its slot's registers and stays in
// flight until its use.  GS == 0 handles any G with a runtime loop.
template <int kDepth, int GS, bool kPrologue = true, typename IssueF, typename ConsumeF>
__device__ __forceinline__ void pipeline(int G, IssueF&& issue, ConsumeF&& consume) {
  if constexpr (GS > 0) {
    if constexpr (kPrologue) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d)
        if (d < GS) issue(d, d);
    }
#pragma unroll
    for (int g = 0; g < GS; ++g) consume(g % kDepth, g, g + kDepth < GS);
  } else {
    if constexpr (kPrologue) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d)
        if (d < G) issue(d, d);
    }
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
// one vector load per four scales once per sweep, and the scale of group g comes from lane
// (ln, g / (G/4)) by a cross-lane read.  This keeps the per-group scale reads
// (16 rows x 4 bytes, 16 cache lines per instruction) out of the vector memory
// pipeline, which they would otherwise congest as much as the weights do.
// Otherwise (any G) one load per row and group.
template <int WFMT, int GS, int NB = 2>
struct GroupScales {
  static constexpr bool kPreload = kIsW4<WFMT> && GS > 0 && GS % 4 == 0;
  static constexpr int kPerLane = kPreload ? GS / 4 : 1;
  float v[NB][kPerLane];
  const ScaleT<WFMT>* row[NB];

  __device__ __forceinline__ void init(const ScaleT<WFMT>* const (&srow)[NB], int kb) {
#pragma unroll
    for (int j = 0; j < NB; ++j) row[j] = srow[j];
    if constexpr (kPreload) {
#pragma unroll
      for (int j = 0; j < NB; ++j) load_scales<kPerLane>(srow[j] + kb * kPerLane, v[j]);
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
    if constexpr (kPreload || !kIsW4<WFMT>) return 1.0f;
    else return load_scale(row[j] + g);
  }
};

// ------------------------------------------------------------- wave kernel
template <int WFMT, int NB>
struct WaveStage {
  uint4 a0, a1;          // 32 activation bytes of this lane's row
  BFrag<WFMT> b[NB];     // weight fragments of the NB 16-row blocks
  float s[NB];           // their group scales (INT4 only)
};

// Output columns of a wave unit u: EPI_SILU_MUL takes gate rows 16u.. and the
// matching up rows N/2 + 16u..; otherwise 16 NB consecutive rows 16 NB u..
template <int EPI, int NB = 2>
__device__ __forceinline__ void unit_columns(int N, int u, int (&col)[NB]) {
  if constexpr (EPI == MOEQ_EPI_SILU_MUL && NB == 2) {
    col[0] = 16 * u;
    col[1] = (N >> 1) + 16 * u;
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) col[j] = 16 * (NB * u + j);
  }
}

// Where a wave sweep reads its activation rows: global memory (row r of the
// tile at a_q + (row0 + r) a_stride, a_stride = K when 0) or LDS (row r at
// a_q + r * a_stride, a_q an LDS address).
enum ASource { kAGlobal = 0, kALds = 1 };

// One K sweep of a wave unit over the 16-row block rb of a tile (rows row0 ..
// row0 + rows - 1): acc[j] receives the fp32 sums (group scales applied,
// activation scale not) of the lane's rows 16 rb + 4 kb + v against weight
// column block j.  Only lanes of real rows load activations (the others keep
// zeros): MFMA rows are independent and rows past the tile are never stored.
// With kSplit the first kDepth groups' weights are issued, then before_a()
// runs (e.g. producing the activations), then their activations; otherwise
// each group's activations and weights are issued together.
// The weights: block bases wblk and scales srow (as quarter_rows leaves them),
// lane offset wlane (weight_rows).
template <int WFMT, int NB, int GS, bool kSplit, int ASRC = kAGlobal, typename HookF>
__device__ __forceinline__ void wave_sweep(v4f (&acc)[NB], const uint8_t* a_q, int K, int row0,
                                           int rows, int rb, const uint8_t* const (&wblk)[NB],
                                           const ScaleT<WFMT>* const (&srow)[NB], uint32_t wlane,
                                           int ln, int kb, HookF&& before_a, int a_stride = 0) {
  const int G = K >> 7;
  const bool a_ok = 16 * rb + ln < rows;
  const int a_row = a_ok ? 16 * rb + ln : 0;
  const uint8_t* a_src = (ASRC == kALds) ? a_q + a_row * a_stride + kb * 32
                                         : a_q + int64_t(row0 + a_row) * (a_stride ? a_stride : K) + kb * 32;
  constexpr int kDepth = Depth<WFMT>::value;
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  WaveStage<WFMT, NB> st[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    st[d].a0 = make_uint4(0, 0, 0, 0);
    st[d].a1 = st[d].a0;
  }
  GroupScales<WFMT, GS, NB> sc;
  sc.init(srow, kb);

  auto issue_a = [&](int slot, int g) {
    if (a_ok) {
      const uint4* ap = reinterpret_cast<const uint4*>(a_src + g * 128);
      st[slot].a0 = ap[0];
      st[slot].a1 = ap[1];
    }
  };
  auto issue_b = [&](int slot, int g) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // a K-split unit is the only reader of its weights
      st[slot].b[j].template load<kCpStream>(wblk[j], g * kGroupStride<WFMT>, wlane);
      st[slot].s[j] = sc.load(j, g);
    }
  };
  auto issue = [&](int slot, int g) {
    issue_a(slot, g);
    issue_b(slot, g);
  };
  auto consume = [&](int slot, int g, bool refill) {
    const WaveStage<WFMT, NB>& s = st[slot];
    const OperandT<WFMT> aop = a_operand<WFMT>(s.a0, s.a1);
    OperandT<WFMT> b[NB];
    float sg[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      b[j] = s.b[j].operand();
      sg[j] = sc.get(j, g, ln, s.s[j]);
    }
    // refill this ring slot only after the last read of its old contents
    __builtin_amdgcn_sched_barrier(0);
    if (refill) issue(slot, g + kDepth);
#pragma unroll
    for (int j = 0; j < NB; ++j) accumulate<WFMT>(acc[j], aop, b[j], sg[j]);
    // Pin this group's arithmetic before the next group's: without it the
    // instruction selector defers the scale FMAs to the end of the unrolled
    // sweep and keeps every group's MFMA result live.
#pragma unroll
    for (int j = 0; j < NB; ++j) pin(acc[j]);
  };
  if constexpr (kSplit) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < G) issue_b(d, d);
    before_a();
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < G) issue_a(d, d);
    pipeline<kDepth, GS, false>(G, issue, consume);
  } else {
    pipeline<kDepth, GS, true>(G, issue, consume);
  }
}

// ------------------------------------------------------ K-split wave units
// A K-split unit is one workgroup whose wave q sweeps the groups
// [q G / 4, (q + 1) G / 4) of the unit's K (the K quarters); the partial sums
// meet in LDS.  A unit then streams its weight rows on all four SIMDs of a CU
// at once and ends about four times sooner than as one wave, so the
// dispatcher balances the CUs at that finer granularity (the end of a launch
// is no longer set by the slowest of thousands of long waves).

// groups of quarter q of G: [g0, g0 + n)
__device__ __forceinline__ int quarter_g0(int G, int q) { return (q * G) >> 2; }
__device__ __forceinline__ int quarter_groups(int G, int q) { return (((q + 1) * G) >> 2) - ((q * G) >> 2); }

// Moves this wave's weight blocks and scale pointers to the first group g0 of
// its quarter.
template <int WFMT, int NB>
__device__ __forceinline__ void quarter_rows(int g0, const uint8_t* (&wblk)[NB],
                                             const ScaleT<WFMT>* (&srow)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    wblk[j] += g0 * kGroupStride<WFMT>;
    if constexpr (kIsW4<WFMT>) srow[j] += g0;             // per-group scales; FP8-row: per row
  }
}

// Sums the four waves' partial accumulators into wave 0 in the fixed order
// acc0 + (acc1 + (acc2 + acc3)): waves 1..3 write theirs to red (3 x NB x 64
// v4f of LDS), one barrier, wave 0 adds.  Every wave of the workgroup calls it;
// red is free again after the next barrier of the caller (or this function's
// next call, whose writes come after wave 0's reads only if the caller
// separates them -- callers looping over blocks pass again_after = true).
template <int NB>
__device__ __forceinline__ void quarter_reduce(v4f (&acc)[NB], v4f* red, int q, int lane,
                                               bool again_after) {
  if (q > 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) red[((q - 1) * NB + j) * kWave + lane] = acc[j];
  }
  __syncthreads();
  if (q == 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = acc[j] + (red[j * kWave + lane] +
                         (red[(NB + j) * kWave + lane] + red[(2 * NB + j) * kWave + lane]));
  }
  if (again_after) __syncthreads();
}

}  // namespace

}  // namespace moeq
