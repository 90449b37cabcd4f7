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
// Work decomposition.  A workgroup (256 threads, 4 waves) computes one plan tile
// (<= 64 rows of one expert, sorted order) by 128 weight rows.  Wave w owns two
// 16-column blocks: for EPI_NONE columns nt*128 + 16*(w + 4j); for EPI_SILU_MUL
// the gate block nt*64 + 16w and the matching up block N/2 + nt*64 + 16w, so the
// SiLU-gated product is formed in registers.  Each lane streams 16 B of packed
// weights (32 codes) per block per group: lane (n = l % 16, kb = l / 16) reads
// bytes [16 kb, 16 kb + 16) of its row's 64-byte group.  The activation tile
// (up to 64 rows x 128 B per group) is staged in LDS, double-buffered, with its
// bytes permuted inside every 8-byte chunk to (0,2,4,6,1,3,5,7) -- the order in
// which the nibble unpack produces the codes (low nibbles, then high nibbles).
// The MFMA sums over K, so any K permutation applied identically to both
// operands leaves the result unchanged.
//
// Grid: (N/128) * max_tiles workgroups, rounded up to a multiple of 8.  The
// linear workgroup id is remapped so that each of the 8 XCDs (workgroups are
// dispatched to XCDs round-robin) receives a contiguous run of logical tiles:
// the N-tiles of one row tile share that tile's activations in one L2.
// Workgroups past the plan's tile count exit at once, so the grid can be sized
// on the host from R alone, without reading the plan back.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 128;           // weight rows per workgroup
constexpr int kRowDw = 36;         // LDS row stride in dwords (128 B + 16 B pad)
constexpr int kXcds = 8;

// INT4 nibble (code + 8) -> E4M3 byte of the code, four nibbles (one per byte,
// values 0..15) at a time.  v_perm_b32 looks bytes up in an 8-byte table; a
// selector byte of 8..11 yields the replicated sign bit of table byte 1/3/5/7,
// 12 yields 0x00 and 13..15 yield 0xFF.  With the raw nibble as selector into
// table T and (nibble & 7) into table U, T[n] ^ U[n] is the answer for n < 8 and
// special(n) ^ U[n - 8] for n >= 8; the tables below satisfy both.
constexpr uint32_t kLutT0 = 0x8E8C09D0u, kLutT1 = 0x09737180u;
constexpr uint32_t kLutU0 = 0x4440C700u, kLutU1 = 0xB1B3B548u;

__device__ __forceinline__ uint32_t nib4_to_e4m3(uint32_t n4) {
  const uint32_t a = __builtin_amdgcn_perm(kLutT1, kLutT0, n4);
  const uint32_t b = __builtin_amdgcn_perm(kLutU1, kLutU0, n4 & 0x07070707u);
  return a ^ b;
}

// 16 packed bytes (32 codes) -> the 32 E4M3 bytes of one MFMA operand, in the
// order (codes 0,2,4,6)(1,3,5,7)(8,10,12,14)(9,11,13,15)...
__device__ __forceinline__ v8i unpack_w4(const uint4& p) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x0F0F0F0Fu;
    const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;
    r[2 * i] = int(nib4_to_e4m3(lo));
    r[2 * i + 1] = int(nib4_to_e4m3(hi));
  }
  return r;
}

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
  __device__ __forceinline__ v8i operand() const {
    v8i r;
    r[0] = int(raw0.x); r[1] = int(raw0.y); r[2] = int(raw0.z); r[3] = int(raw0.w);
    r[4] = int(raw1.x); r[5] = int(raw1.y); r[6] = int(raw1.z); r[7] = int(raw1.w);
    return r;
  }
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands FP8 E4M3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// MB = 16-row blocks computed per K sweep (4: the whole 64-row tile at once;
// 1: one block per sweep, for decode-sized tiles where blocks beyond the first
// are rare).
template <int WFMT, int EPI, int MB>
__global__ void __launch_bounds__(kThreads)
grouped_gemm_kernel(const uint8_t* __restrict__ a_q, const float* __restrict__ a_s,
                    const int32_t* __restrict__ plan, int E, int R,
                    const uint8_t* __restrict__ w, const float* __restrict__ w_scale, int N,
                    int K, void* __restrict__ out, int out_f32) {
  constexpr int kRowsLds = 16 * MB;
  __shared__ uint32_t As[2][kRowsLds * kRowDw];

  // ---- which tile / N-tile: XCD-contiguous remap of the linear block id
  const int n_ntiles = N / kBN;
  const int total = n_ntiles * plan_max_tiles(E, R);
  const int per_xcd = gridDim.x / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total) return;
  const int tile = logical / n_ntiles;
  const int nt = logical - tile * n_ntiles;
  if (tile >= plan[kPlanTiles]) return;
  const PlanView pv = plan_view(const_cast<int32_t*>(plan), E, R);
  const int e = pv.tile_expert[tile];
  const int row0 = pv.tile_row0[tile];
  const int end = pv.offsets[e + 1];
  const int tile_rows = min(MOEQ_TILE_M, end - row0);
  const int nrb = (tile_rows + 15) >> 4;

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
  const int64_t w_row_bytes = (WFMT == kW4G128) ? (K >> 1) : K;
  const uint8_t* wrow[2];
  const float* srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n_glob = int64_t(e) * N + col[j] + ln;
    wrow[j] = w + n_glob * w_row_bytes;
    srow[j] = (WFMT == kW4G128) ? (w_scale + n_glob * G) : (w_scale + n_glob);
  }

  // A staging: thread -> (row, 32-byte chunk) of the tile slice
  const int st_row = tid >> 2, st_chunk = tid & 3;
  const bool stager = st_row < kRowsLds;

  for (int rb0 = 0; rb0 < nrb; rb0 += MB) {
    const int p_st = row0 + 16 * rb0 + st_row;
    const bool st_valid = stager && (16 * rb0 + st_row) < tile_rows;
    const uint8_t* a_src = a_q + int64_t(st_valid ? p_st : 0) * K + st_chunk * 32;

    // rows past the tile read row 0 of a_q (always valid) and are zeroed
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    auto load_a = [=](int g, uint4 (&x)[2]) {
      const uint4* p = reinterpret_cast<const uint4*>(a_src + g * 128);
      x[0] = p[0];
      x[1] = p[1];
      if (!st_valid) { x[0] = zero4; x[1] = zero4; }
    };
    auto store_a = [&](int buf, const uint4 (&x)[2]) {
      const uint32_t d[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (WFMT == kW4G128) {     // (0,2,4,6)(1,3,5,7) inside each 8-byte chunk
          o[2 * i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x06040200u);
          o[2 * i + 1] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07050301u);
        } else {
          o[2 * i] = d[2 * i];
          o[2 * i + 1] = d[2 * i + 1];
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(&As[buf][st_row * kRowDw + st_chunk * 8]);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    };

    v4f acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    BFrag<WFMT> b_cur[2], b_nxt[2];
    float s_cur[2] = {1.f, 1.f}, s_nxt[2] = {1.f, 1.f};
    {
      uint4 x[2];
      if (stager) load_a(0, x);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        b_cur[j].load(wrow[j], 0, kb);
        if (WFMT == kW4G128) s_cur[j] = srow[j][0];
      }
      if (stager) store_a(0, x);
    }
    __syncthreads();

    for (int g = 0; g < G; ++g) {
      const int buf = g & 1;
      const bool more = g + 1 < G;
      uint4 x[2];
      if (more) {
        if (stager) load_a(g + 1, x);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          b_nxt[j].load(wrow[j], g + 1, kb);
          if (WFMT == kW4G128) s_nxt[j] = srow[j][g + 1];
        }
      }
      v8i bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bop[j] = b_cur[j].operand();
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (rb0 + i < nrb) {
          const uint4* ap = reinterpret_cast<const uint4*>(&As[buf][(16 * i + ln) * kRowDw + kb * 8]);
          const uint4 a0 = ap[0], a1 = ap[1];
          v8i aop;
          aop[0] = int(a0.x); aop[1] = int(a0.y); aop[2] = int(a0.z); aop[3] = int(a0.w);
          aop[4] = int(a1.x); aop[5] = int(a1.y); aop[6] = int(a1.z); aop[7] = int(a1.w);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (WFMT == kW4G128) {
              const v4f part = mfma_fp8(aop, bop[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(s_cur[j], part[v], acc[i][j][v]);
            } else {
              acc[i][j] = mfma_fp8(aop, bop[j], acc[i][j]);
            }
          }
        }
      }
      if (more && stager) store_a(buf ^ 1, x);
      __syncthreads();
      if (more) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          b_cur[j] = b_nxt[j];
          s_cur[j] = s_nxt[j];
        }
      }
    }

    // ---- epilogue: lane holds rows 16 i + 4 kb + v, column col[j] + ln
    float rs[2] = {1.f, 1.f};
    if (WFMT == kFp8Row) {
      rs[0] = srow[0][0];
      rs[1] = srow[1][0];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (rb0 + i >= nrb) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r_in = 16 * (rb0 + i) + 4 * kb + v;
        if (r_in >= tile_rows) continue;
        const int p = row0 + r_in;
        const float sa = a_s[p];
        const float v0 = sa * acc[i][0][v] * rs[0];
        const float v1 = sa * acc[i][1][v] * rs[1];
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
    if (rb0 + MB < nrb) __syncthreads();   // LDS reuse by the next row-block sweep
  }
}

template <int WFMT, int EPI, int MB>
hipError_t launch_one(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                      const uint8_t* w, const float* w_scale, int N, int K, void* out, int out_f32,
                      hipStream_t stream) {
  const int64_t total = int64_t(N / kBN) * plan_max_tiles(E, R);
  const int64_t grid = (total + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((grouped_gemm_kernel<WFMT, EPI, MB>), dim3(unsigned(grid)), dim3(kThreads), 0,
                     stream, a_q, a_s, static_cast<const int32_t*>(plan), E, R, w, w_scale, N, K,
                     out, out_f32);
  return hipGetLastError();
}

template <int WFMT>
hipError_t launch_fmt(const uint8_t* a_q, const float* a_s, const void* plan, int E, int R,
                      const uint8_t* w, const float* w_scale, int N, int K, int epilogue, void* out,
                      int out_f32, hipStream_t stream) {
  // R <= 64 routed rows (decode): tiles hold at most a few rows -> one 16-row
  // block per K sweep keeps the register footprint small.
  const bool small = R <= 64;
  if (epilogue == MOEQ_EPI_SILU_MUL) {
    return small ? launch_one<WFMT, MOEQ_EPI_SILU_MUL, 1>(a_q, a_s, plan, E, R, w, w_scale, N, K,
                                                          out, out_f32, stream)
                 : launch_one<WFMT, MOEQ_EPI_SILU_MUL, 4>(a_q, a_s, plan, E, R, w, w_scale, N, K,
                                                          out, out_f32, stream);
  }
  return small ? launch_one<WFMT, MOEQ_EPI_NONE, 1>(a_q, a_s, plan, E, R, w, w_scale, N, K, out,
                                                    out_f32, stream)
               : launch_one<WFMT, MOEQ_EPI_NONE, 4>(a_q, a_s, plan, E, R, w, w_scale, N, K, out,
                                                    out_f32, stream);
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
