// Grouped GEMM over AQLM expert weights (the cold experts of the NVFP4 + AQLM
// hybrid checkpoint) with per-token FP8 activations.  For output row r and
// group g of 8 input channels the weights are
//   W[r, 8g .. 8g+7] = (sum over books b of codebook_b[codes_b[r, g]]) * row_scale[r]
// (codebook rows: 8 fp16 values; one or two books; int16 codes index a
// 65536-entry book through idx & 0xFFFF).
//
// The per-row scale factors out of every dot product, so it is applied in the
// epilogue; what enters the MFMA is the codebook row itself.  In the MFMA
// layout of v_mfma_f32_16x16x32_f16 a lane supplies 8 consecutive K of one
// weight row -- exactly one AQLM group -- so the B operand of a lane is one
// gathered 16-byte codebook row, used as it is (f16); each book gets its own
// MFMA, accumulating into the same fp32 sums, so no two fp16 codebook values
// are ever added in f16.  Activations are widened to f16 exactly.  Products
// are exact and accumulate in fp32.
//
// Memory: a lane reads its 4 codes of a 128-K chunk with one 8-byte (int16) or
// 4-byte (uint8) load from HBM, then gathers 4 codebook rows (16 bytes each,
// one per MFMA step) per book.  A 65536-entry book is 1 MB: it stays in the L2
// (and MALL), not in LDS; the gathers, not the 2-bit code stream, bound the
// kernel.  Codes run kAqDepth chunks ahead through a register ring; each
// chunk's gathers are issued before the ring refill, so waiting for them never
// waits for the refill.
//
// slab_of and the wave-unit structure are those of the NVFP4 kernel.
#include "gemm.hpp"

namespace moeq {

namespace {

// chunks of codes in flight per wave (two books hold twice the gathered rows)
template <int NBOOK>
constexpr int kAqDepth = (NBOOK > 1) ? 2 : 3;

// the 4 codes of a lane for one chunk: 16-bit (int16, entry = code & 0xFFFF) or 8-bit
template <bool W16>
struct Codes4 {
  uint2 raw;
  __device__ __forceinline__ void load(const uint8_t* row, int g, int kb) {
    if constexpr (W16) {
      raw = *reinterpret_cast<const uint2*>(row + g * 32 + kb * 8);
    } else {
      raw.x = *reinterpret_cast<const uint32_t*>(row + g * 16 + kb * 4);
      raw.y = 0;
    }
  }
  __device__ __forceinline__ uint32_t entry(int m) const {
    if constexpr (W16) {
      const uint32_t w = (m < 2) ? raw.x : raw.y;
      return (m & 1) ? (w >> 16) : (w & 0xFFFFu);
    } else {
      return (raw.x >> (8 * m)) & 0xFFu;
    }
  }
};

template <bool W16_0, bool W16_1, int NBOOK>
struct AqStage {
  uint4 a0, a1;                      // 32 activation bytes of this lane's row
  Codes4<W16_0> c0[2];               // book 0 codes of the two weight-row blocks
  Codes4<W16_1> c1[NBOOK > 1 ? 2 : 1];
};

template <int EPI, int NBOOK, bool W16_0, bool W16_1>
__global__ void __launch_bounds__(kThreads, 3)
gemm_aqlm_kernel(const uint8_t* a_q, const float* a_s, const int32_t* plan, int E, int R,
                 const int32_t* slab_of, int S, const uint8_t* codes0, const uint8_t* codes1,
                 const uint16_t* book0, const uint16_t* book1, int last0, int last1,
                 const _Float16* row_scale, int N, int K, void* out, int out_f32) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kb = lane >> 4;
  const int units_per_tile = N / 32;
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  const int tile = unit / units_per_tile;
  const int u = unit - tile * units_per_tile;
  TileInfo ti;
  if (!tile_info(plan, E, R, tile, ti)) return;   // wave-uniform
  const int slab = slab_of ? slab_of[ti.e] : ti.e;
  if (slab < 0 || slab >= S) return;                    // wave-uniform
  const int G = K >> 7;
  const int64_t code_row0 = int64_t(K >> 3) * (W16_0 ? 2 : 1);   // bytes per row of codes
  const int64_t code_row1 = int64_t(K >> 3) * (W16_1 ? 2 : 1);

  int col[2];
  unit_columns<EPI, 2>(N, u, col);
  const uint8_t* crow0[2];
  const uint8_t* crow1[2];
  const _Float16* srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n_glob = int64_t(slab) * N + col[j] + ln;
    crow0[j] = codes0 + n_glob * code_row0;
    crow1[j] = (NBOOK > 1) ? codes1 + n_glob * code_row1 : nullptr;
    srow[j] = row_scale + n_glob;
  }

  const int nrb = (ti.rows + 15) >> 4;
  for (int rb = 0; rb < nrb; ++rb) {
    const bool a_ok = 16 * rb + ln < ti.rows;
    const uint8_t* a_src = a_q + int64_t(ti.row0 + (a_ok ? 16 * rb + ln : 0)) * K + kb * 32;
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    AqStage<W16_0, W16_1, NBOOK> st[kAqDepth<NBOOK>];
#pragma unroll
    for (int d = 0; d < kAqDepth<NBOOK>; ++d) {
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
        st[slot].c0[j].load(crow0[j], g, kb);
        if constexpr (NBOOK > 1) st[slot].c1[j].load(crow1[j], g, kb);
      }
    };
    auto consume = [&](int slot, int g, bool refill) {
      const AqStage<W16_0, W16_1, NBOOK> s = st[slot];
      // gathers of this chunk's codebook rows, issued before the refill
      uint4 r0[2][4], r1[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // codes past a book's last entry (invalid input) read its last row
          const uint32_t e0 = min(s.c0[j].entry(m), uint32_t(last0));
          r0[j][m] = *reinterpret_cast<const uint4*>(book0 + e0 * 8);
          if constexpr (NBOOK > 1) {
            const uint32_t e1 = min(s.c1[j].entry(m), uint32_t(last1));
            r1[j][m] = *reinterpret_cast<const uint4*>(book1 + e1 * 8);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(slot, g + kAqDepth<NBOOK>);
      const uint32_t ad[8] = {s.a0.x, s.a0.y, s.a0.z, s.a0.w, s.a1.x, s.a1.y, s.a1.z, s.a1.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const h8 aop = fp8x8_to_f16(ad[2 * m], ad[2 * m + 1]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j] = mfma_f16(aop, __builtin_bit_cast(h8, r0[j][m]), acc[j]);
          if constexpr (NBOOK > 1) acc[j] = mfma_f16(aop, __builtin_bit_cast(h8, r1[j][m]), acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) pin(acc[j]);
    };
    pipeline<kAqDepth<NBOOK>, 0>(G, issue, consume);
    store_block<kAqlm, EPI>(acc, rb, ti.row0, ti.rows, [a_s](int p, int) { return a_s[p]; }, srow, col,
                            ln, kb, N, out, out_f32);
  }
}

template <int EPI, int NBOOK, bool W16_0, bool W16_1>
void launch_aqlm_kernel(dim3 grid, hipStream_t stream, const uint8_t* a_q, const float* a_s,
                        const int32_t* plan, int E, int R, const int32_t* slab_of, int S,
                        const void* const* codes, const int* entries,
                        const uint16_t* const* books, const uint16_t* row_scale, int N, int K,
                        void* out, int out_f32) {
  hipLaunchKernelGGL((gemm_aqlm_kernel<EPI, NBOOK, W16_0, W16_1>), grid, dim3(kThreads), 0, stream,
                     a_q, a_s, plan, E, R, slab_of, S, static_cast<const uint8_t*>(codes[0]),
                     NBOOK > 1 ? static_cast<const uint8_t*>(codes[1]) : nullptr, books[0],
                     NBOOK > 1 ? books[1] : nullptr, entries[0] - 1,
                     NBOOK > 1 ? entries[1] - 1 : 0, reinterpret_cast<const _Float16*>(row_scale), N,
                     K, out, out_f32);
}

template <int EPI>
void launch_aqlm_epi(dim3 grid, hipStream_t stream, const uint8_t* a_q, const float* a_s,
                     const int32_t* plan, int E, int R, const int32_t* slab_of, int S,
                     int n_books,
                     const void* const* codes, const int* entries, const uint16_t* const* books,
                     const uint16_t* row_scale, int N, int K, void* out, int out_f32) {
  const bool w0 = entries[0] > 256;
  if (n_books == 1) {
    if (w0)
      launch_aqlm_kernel<EPI, 1, true, false>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                              entries, books, row_scale, N, K, out, out_f32);
    else
      launch_aqlm_kernel<EPI, 1, false, false>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                               entries, books, row_scale, N, K, out, out_f32);
    return;
  }
  const bool w1 = entries[1] > 256;
  if (w0 && w1)
    launch_aqlm_kernel<EPI, 2, true, true>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                           entries, books, row_scale, N, K, out, out_f32);
  else if (w0)
    launch_aqlm_kernel<EPI, 2, true, false>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                            entries, books, row_scale, N, K, out, out_f32);
  else if (w1)
    launch_aqlm_kernel<EPI, 2, false, true>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                            entries, books, row_scale, N, K, out, out_f32);
  else
    launch_aqlm_kernel<EPI, 2, false, false>(grid, stream, a_q, a_s, plan, E, R, slab_of, S, codes,
                                             entries, books, row_scale, N, K, out, out_f32);
}

}  // namespace

hipError_t launch_grouped_gemm_aqlm(const uint8_t* a_q, const float* a_s, const void* plan, int E,
                                    int R, const int32_t* slab_of, int S, int n_books,
                                    const void* const* codes, const int* book_entries,
                                    const uint16_t* const* codebooks, const uint16_t* row_scale,
                                    int N, int K, int epilogue, void* out, int out_dtype,
                                    hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int out_f32 = out_dtype == MOEQ_F32 ? 1 : 0;
  const int64_t units = int64_t(plan_max_tiles(E, R)) * (N / 32);
  const dim3 grid(unsigned((units + 3) / 4));
  const int32_t* p = static_cast<const int32_t*>(plan);
  if (epilogue == MOEQ_EPI_SILU_MUL)
    launch_aqlm_epi<MOEQ_EPI_SILU_MUL>(grid, stream, a_q, a_s, p, E, R, slab_of, S, n_books, codes,
                                       book_entries, codebooks, row_scale, N, K, out, out_f32);
  else
    launch_aqlm_epi<MOEQ_EPI_NONE>(grid, stream, a_q, a_s, p, E, R, slab_of, S, n_books, codes,
                                   book_entries, codebooks, row_scale, N, K, out, out_f32);
  return hipGetLastError();
}

}  // namespace moeq
