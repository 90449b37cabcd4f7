// Dense bf16 GEMM for the shared experts: out = epilogue(a @ w^T), fp32 accumulate,
// on v_mfma_f32_16x16x32_bf16.  Three tilings: 256-row tiles (shared_gemm_wide.hip)
// when they give every CU a workgroup, the 128-row large-tile kernel below for
// other prefill-sized M, the small-tile one for small M or shapes neither covers.
//
// Workgroup tile: 128 rows of a x 128 rows of w (the weight rows: for EPI_NONE
// the 128 output columns nt*128.., for EPI_SILU_MUL the 64 gate rows nt*64..
// and the matching 64 up rows N/2 + nt*64..).  K advances 32 at a time through
// double-buffered LDS tiles (row stride 80 B: conflict-free 16-byte reads).
// Four waves in a 2 x 2 arrangement, each computing 64 rows x 4 column blocks
// of 16 (16 MFMAs per K step).  The MFMA lane layout: operand lane (r = l % 16,
// kq = l / 16) holds k = 8 kq .. 8 kq + 7 of row r; result lane l holds column
// l % 16 of rows 4 (l / 16) .. 4 (l / 16) + 3.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kT = 256;
constexpr int kBM = 128, kBNw = 128, kBK = 32;
constexpr int kStrideH = 40;  // bf16 elements per LDS row (32 + 8 pad) = 80 B

template <int EPI>
__global__ void __launch_bounds__(kT)
shared_gemm_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w, int M, int N,
                   int K, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kStrideH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBNw * kStrideH];
  const int n_ntiles = N / kBNw;
  const int mt = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - mt * n_ntiles;
  const int m0 = mt * kBM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ln = lane & 15, kq = lane >> 4;

  // staging: thread -> (tile row tid/2, 16-element half tid%2) for both A and B
  const int sr = tid >> 1, sh = tid & 1;
  // rows past M re-read row M - 1: their results are never stored
  const uint16_t* a_src = a + int64_t(min(m0 + sr, M - 1)) * K + sh * 16;
  int w_row;
  if (EPI == MOEQ_EPI_SILU_MUL) w_row = sr < 64 ? nt * 64 + sr : (N >> 1) + nt * 64 + (sr - 64);
  else w_row = nt * kBNw + sr;
  const uint16_t* w_src = w + int64_t(w_row) * K + sh * 16;

  // the four 16-column blocks of this wave, as B-tile row offsets
  int cb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (EPI == MOEQ_EPI_SILU_MUL) cb[q] = (q < 2) ? 32 * wn + 16 * q : 64 + 32 * wn + 16 * (q - 2);
    else cb[q] = 64 * wn + 16 * q;
  }

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  // staging registers as plain scalars (arrays passed to lambdas by reference
  // were left in scratch memory)
  uint4 ra0, ra1, rb0, rb1;
  const uint4* pa = reinterpret_cast<const uint4*>(a_src);
  const uint4* pb = reinterpret_cast<const uint4*>(w_src);
  ra0 = pa[0]; ra1 = pa[1]; rb0 = pb[0]; rb1 = pb[1];
  uint4* da = reinterpret_cast<uint4*>(&As[0][sr * kStrideH + sh * 16]);
  uint4* db = reinterpret_cast<uint4*>(&Bs[0][sr * kStrideH + sh * 16]);
  constexpr int kBufA = kBM * kStrideH / 8, kBufB = kBNw * kStrideH / 8;  // in uint4
  da[0] = ra0; da[1] = ra1; db[0] = rb0; db[1] = rb1;
  __syncthreads();
  const int steps = K / kBK;
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < steps;
    if (more) {
      const int o = (s + 1) * kBK / 8;
      ra0 = pa[o]; ra1 = pa[o + 1]; rb0 = pb[o]; rb1 = pb[o + 1];
    }
    v8bf bop[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bop[q] = *reinterpret_cast<const v8bf*>(&Bs[buf][(cb[q] + ln) * kStrideH + kq * 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8bf aop = *reinterpret_cast<const v8bf*>(&As[buf][(64 * wm + 16 * i + ln) * kStrideH + kq * 8]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[q], acc[i][q], 0, 0, 0);
    }
    if (more) {
      const int nb = buf ^ 1;
      da[nb * kBufA] = ra0; da[nb * kBufA + 1] = ra1;
      db[nb * kBufB] = rb0; db[nb * kBufB + 1] = rb1;
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 64 * wm + 16 * i + 4 * kq + v;
      if (m >= M) continue;
      if (EPI == MOEQ_EPI_SILU_MUL) {
        uint16_t* o = out + int64_t(m) * (N >> 1);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          o[nt * 64 + cb[q] + ln] = f32_to_bf16(silu_f32(acc[i][q][v]) * acc[i][q + 2][v]);
      } else {
        uint16_t* o = out + int64_t(m) * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[nt * kBNw + cb[q] + ln] = f32_to_bf16(acc[i][q][v]);
      }
    }
  }
}

// ---------------------------------------------------------------- large tiles
// For the shared experts' prefill shapes (M in the thousands, K % 32 == 0):
// workgroup tile 128 rows of a x BN weight rows (BN = 256, or 128 when 256
// would leave fewer than two workgroups per CU), K advancing 32 per barrier
// through double-buffered LDS (61 KB at BN = 256: two workgroups per CU).
// Four waves in a 2 x 2 arrangement, each owning 64 rows x BN/2 columns
// (NQ = BN/32 column blocks of 16; 4 NQ MFMAs of 16x16x32 per K step, 16 NQ
// fp32 accumulators per lane).  Per step a wave reads 4 A and NQ B operands
// (16 B per lane each) from LDS, and the next step's global loads are in
// flight during the current step's MFMAs.  With EPI_SILU_MUL the BN weight
// rows are BN/2 gate rows and their BN/2 up rows; column block q of a wave
// (q < NQ/2) is gate, q + NQ/2 the matching up block.
constexpr int kBM2 = 128, kBK2 = 32;
constexpr int kStride2 = kBK2 + 8;         // bf16 per LDS row: 80 B, conflict-free 16 B reads

template <int BN>
__host__ __device__ constexpr size_t big_lds_bytes() {
  return size_t(2) * (kBM2 + BN) * kStride2 * sizeof(uint16_t);
}

template <int EPI, int BN>
__global__ void __launch_bounds__(kT, 2)
shared_gemm_big_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w, int M,
                       int N, int K, uint16_t* __restrict__ out) {
  static_assert(BN == 256 || BN == 128, "tile width");
  constexpr int NQ = BN / 32;              // column blocks per wave
  constexpr int BP = BN / 64;              // B staging passes of 64 rows
  extern __shared__ __attribute__((aligned(16))) uint16_t smem2[];
  uint16_t* As = smem2;                                  // [2][kBM2 * kStride2]
  uint16_t* Bs = smem2 + 2 * kBM2 * kStride2;            // [2][BN * kStride2]
  const int n_ntiles = N / BN;
  const int mt = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - mt * n_ntiles;
  const int m0 = mt * kBM2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ln = lane & 15, kq = lane >> 4;

  // staging: thread -> (row tid / 4, 16-byte piece tid % 4) of each 64-row
  // pass; A takes two passes, B takes BP (for EPI_SILU_MUL the first BP/2 are
  // gate rows, the rest the matching up rows)
  const int srow = tid >> 2, spiece = (tid & 3) * 8;
  const int64_t pass_step = int64_t(64) * K;
  // rows past M re-read row M - 1: their results are never stored, and rows
  // of a product do not mix
  const uint16_t* a_r0 = a + int64_t(min(m0 + srow, M - 1)) * K + spiece;
  const uint16_t* a_r1 = a + int64_t(min(m0 + srow + 64, M - 1)) * K + spiece;
  const uint16_t* w_lo;          // passes 0 .. BP/2 - 1
  const uint16_t* w_hi;          // passes BP/2 .. BP - 1
  if (EPI == MOEQ_EPI_SILU_MUL) {
    w_lo = w + int64_t(nt * (BN / 2) + srow) * K + spiece;
    w_hi = w + int64_t((N >> 1) + nt * (BN / 2) + srow) * K + spiece;
  } else {
    w_lo = w + int64_t(nt * BN + srow) * K + spiece;
    w_hi = w_lo + (BP / 2) * pass_step;
  }
  // B-tile row of column block q of this wave
  int cb[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (EPI == MOEQ_EPI_SILU_MUL) cb[q] = (q < NQ / 2 ? 0 : BN / 2) + (BN / 4) * wn + 16 * (q % (NQ / 2));
    else cb[q] = (BN / 2) * wn + 16 * q;
  }

  v4f acc[4][NQ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  // staging registers as scalars (arrays captured by lambdas stay in scratch);
  // rb2, rb3 are used only when BN = 256
  uint4 ra0, ra1, rb0, rb1, rb2 = {}, rb3 = {};
#define SG_LD(p) (*reinterpret_cast<const uint4*>(p))
#define SG_GLOAD(k0)                                                             \
  do {                                                                           \
    ra0 = SG_LD(a_r0 + (k0));                                                    \
    ra1 = SG_LD(a_r1 + (k0));                                                    \
    if (BP == 4) {                                                               \
      rb0 = SG_LD(w_lo + (k0));                                                  \
      rb1 = SG_LD(w_lo + pass_step + (k0));                                      \
      rb2 = SG_LD(w_hi + (k0));                                                  \
      rb3 = SG_LD(w_hi + pass_step + (k0));                                      \
    } else {                                                                     \
      rb0 = SG_LD(w_lo + (k0));                                                  \
      rb1 = SG_LD(w_hi + (k0));                                                  \
    }                                                                            \
  } while (0)
#define SG_ST(base, pass, v) (*reinterpret_cast<uint4*>((base) + (pass) * 64 * kStride2) = (v))
#define SG_SSTORE(buf)                                                           \
  do {                                                                           \
    uint16_t* as_ = As + (buf) * kBM2 * kStride2 + srow * kStride2 + spiece;     \
    uint16_t* bs_ = Bs + (buf) * BN * kStride2 + srow * kStride2 + spiece;       \
    SG_ST(as_, 0, ra0); SG_ST(as_, 1, ra1);                                      \
    SG_ST(bs_, 0, rb0); SG_ST(bs_, 1, rb1);                                      \
    if (BP == 4) { SG_ST(bs_, 2, rb2); SG_ST(bs_, 3, rb3); }                     \
  } while (0)

  SG_GLOAD(0);
  SG_SSTORE(0);
  __syncthreads();
  const int steps = K / kBK2;
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < steps;
    if (more) SG_GLOAD((s + 1) * kBK2);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* A = As + buf * kBM2 * kStride2;
    const uint16_t* B = Bs + buf * BN * kStride2;
    const int kk = kq * 8;
    v8bf aop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      aop[i] = *reinterpret_cast<const v8bf*>(&A[(64 * wm + 16 * i + ln) * kStride2 + kk]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const v8bf bop = *reinterpret_cast<const v8bf*>(&B[(cb[q] + ln) * kStride2 + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], bop, acc[i][q], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      __syncthreads();                 // every wave is done reading buf ^ 1 (step s - 1)
      SG_SSTORE(buf ^ 1);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 64 * wm + 16 * i + 4 * kq + v;
      if (m >= M) continue;
      if (EPI == MOEQ_EPI_SILU_MUL) {
        uint16_t* o = out + int64_t(m) * (N >> 1);
#pragma unroll
        for (int q = 0; q < NQ / 2; ++q)
          o[nt * (BN / 2) + cb[q] + ln] = f32_to_bf16(silu_f32(acc[i][q][v]) * acc[i][q + NQ / 2][v]);
      } else {
        uint16_t* o = out + int64_t(m) * N;
#pragma unroll
        for (int q = 0; q < NQ; ++q) o[nt * BN + cb[q] + ln] = f32_to_bf16(acc[i][q][v]);
      }
    }
  }
}
#undef SG_LD
#undef SG_GLOAD
#undef SG_ST
#undef SG_SSTORE

template <int BN>
hipError_t launch_big(const uint16_t* a, const uint16_t* w, int M, int N, int K, int epilogue,
                      uint16_t* out, hipStream_t stream) {
  const int64_t blocks = int64_t((M + kBM2 - 1) / kBM2) * (N / BN);
  const size_t lds = big_lds_bytes<BN>();
  auto fn = (epilogue == MOEQ_EPI_SILU_MUL) ? shared_gemm_big_kernel<MOEQ_EPI_SILU_MUL, BN>
                                            : shared_gemm_big_kernel<MOEQ_EPI_NONE, BN>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fn, dim3(unsigned(blocks)), dim3(kT), lds, stream, a, w, M, N, K, out);
  return hipGetLastError();
}

}  // namespace

// 256-row tiles (shared_gemm_wide.hip): the tile width for this shape, 0 when
// they are not taken
int shared_wide_bn(int M, int N, int K);
hipError_t launch_shared_gemm_wide(int bn, const uint16_t* a, const uint16_t* w, int M, int N,
                                   int K, int epilogue, uint16_t* out, hipStream_t stream);

hipError_t launch_shared_gemm_bf16(const uint16_t* a, const uint16_t* w, int M, int N, int K,
                                   int epilogue, uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int wide_bn = shared_wide_bn(M, N, K);
  if (wide_bn) return launch_shared_gemm_wide(wide_bn, a, w, M, N, K, epilogue, out, stream);
  if (M >= 256 && K % kBK2 == 0) {
    // 128 x 256 tiles when they give at least two workgroups per CU (512),
    // else 128 x 128
    const int64_t mtiles = (M + kBM2 - 1) / kBM2;
    if (N % 256 == 0 && mtiles * (N / 256) >= 512)
      return launch_big<256>(a, w, M, N, K, epilogue, out, stream);
    if (N % 128 == 0) return launch_big<128>(a, w, M, N, K, epilogue, out, stream);
  }
  const int64_t blocks = int64_t((M + kBM - 1) / kBM) * (N / kBNw);
  if (epilogue == MOEQ_EPI_SILU_MUL)
    hipLaunchKernelGGL(shared_gemm_kernel<MOEQ_EPI_SILU_MUL>, dim3(unsigned(blocks)), dim3(kT), 0,
                       stream, a, w, M, N, K, out);
  else
    hipLaunchKernelGGL(shared_gemm_kernel<MOEQ_EPI_NONE>, dim3(unsigned(blocks)), dim3(kT), 0,
                       stream, a, w, M, N, K, out);
  return hipGetLastError();
}

}  // namespace moeq
