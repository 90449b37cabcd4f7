// Dense bf16 GEMM for the shared experts: out = epilogue(a @ w^T), fp32 accumulate,
// on v_mfma_f32_16x16x32_bf16.
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
  const int a_row = m0 + sr;
  const bool a_ok = a_row < M;
  const uint16_t* a_src = a + int64_t(a_ok ? a_row : 0) * K + sh * 16;
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

  auto gload = [&](int k0, uint4 (&ra)[2], uint4 (&rb)[2]) {
    const uint4* pa = reinterpret_cast<const uint4*>(a_src + k0);
    const uint4* pb = reinterpret_cast<const uint4*>(w_src + k0);
    if (a_ok) { ra[0] = pa[0]; ra[1] = pa[1]; }
    else { ra[0] = make_uint4(0, 0, 0, 0); ra[1] = ra[0]; }
    rb[0] = pb[0];
    rb[1] = pb[1];
  };
  auto sstore = [&](int buf, const uint4 (&ra)[2], const uint4 (&rb)[2]) {
    uint4* da = reinterpret_cast<uint4*>(&As[buf][sr * kStrideH + sh * 16]);
    uint4* db = reinterpret_cast<uint4*>(&Bs[buf][sr * kStrideH + sh * 16]);
    da[0] = ra[0]; da[1] = ra[1];
    db[0] = rb[0]; db[1] = rb[1];
  };

  uint4 ra[2], rb[2];
  gload(0, ra, rb);
  sstore(0, ra, rb);
  __syncthreads();
  const int steps = K / kBK;
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < steps;
    if (more) gload((s + 1) * kBK, ra, rb);
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
    if (more) sstore(buf ^ 1, ra, rb);
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

}  // namespace

hipError_t launch_shared_gemm_bf16(const uint16_t* a, const uint16_t* w, int M, int N, int K,
                                   int epilogue, uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
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
