// Dense bf16 GEMM for the shared experts, 256-row tiles: out = epilogue(a @ w^T)
// with fp32 accumulation on v_mfma_f32_16x16x32_bf16, for shapes large enough
// to give every CU a 256-row tile (the shared experts at prefill).  The MFMA
// lane layout is that of the kernels in shared_gemm.hip: operand lane
// (r = l % 16, kq = l / 16) holds k = 8 kq .. 8 kq + 7 of row r; result lane l
// holds column l % 16 of rows 4 (l / 16) .. 4 (l / 16) + 3.
//
// Workgroup tile 256 rows of a x BN weight rows (BN = 256, or 128 when 256
// would leave CUs idle), eight waves: two per SIMD, since one wave alone issues
// an MFMA only about every 27 cycles where the unit takes 16.  The waves form
// a WM x WN grid, each owning 256/WM rows x BN/WN columns: 128 x 64 at BN = 256
// (8 A blocks x 4 column blocks, 128 fp32 accumulators per lane), 64 x 64 at
// BN = 128.  With EPI_SILU_MUL the BN weight rows are BN/2 gate rows and the
// matching BN/2 up rows; a wave's first NQ/2 column blocks are gate columns,
// the other NQ/2 the up columns of the same outputs.
//
// Operands reach LDS by buffer loads that write LDS directly (no staging
// registers, no LDS store instructions): one load of a wave moves 8 rows x 128 B
// (16 bytes per lane; whole 128-byte lines, so each lane group's request to L2
// is a full line) into 1 KB of LDS.  The LDS holds a ring of slots of 64 K
// (2 x 64 KB at BN = 256, 3 x 48 KB at BN = 128).  Chunk c (8 K values) of
// row r sits at position c ^ swz(r): the 16 rows x 16 bytes an MFMA operand
// read takes then fall in distinct LDS banks.  A slot is consumed in two
// halves of 32 K; a wave reads the operands of the next half into a second
// register set before the MFMAs of the current one, which do not wait for
// them, and the barrier that opens slot s + 1 (once its loads have landed)
// also frees slot s's buffer for the loads of slot s + kSlots.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8, kTw = 64 * kWaves;
constexpr int kBMw = 256, kBKs = 64;
constexpr int kRowB = kBKs * 2;            // bytes of a slot row: one 128-byte line

template <int BN>
__host__ __device__ constexpr int slot_bytes() { return (kBMw + BN) * kRowB; }

// slots in the ring: 2 x 64 KB at BN = 256, 3 x 48 KB at BN = 128
template <int BN>
__host__ __device__ constexpr int ring_slots() { return BN == 256 ? 2 : 3; }

template <int BN>
__host__ __device__ constexpr size_t wide_lds_bytes() { return size_t(ring_slots<BN>()) * slot_bytes<BN>(); }

// Position of 16-byte chunk c of row r: c ^ swz(r), swz(r) = (r mod 16) / 2.
// An operand read takes chunk kq (the lane's K quarter, kq = lane / 16) of rows
// ln = lane % 16.  The LDS serves a 16-byte read 32 lanes at a time over
// 128 banks (512 bytes): lanes 0..31 (kq 0, 1) and 32..63 (kq 2, 3) must then
// address distinct 16-byte slots modulo 512 bytes, i.e. rows ln, ln + 4,
// ln + 8, ln + 12 (same slot group) must differ in swz(r) / 2 -- which r / 2
// does.  (Measured: swz(r) = (r ^ (r / 8)) mod 8, distinct only over 16
// consecutive lanes, cost 4 bank-conflict cycles per read, doubling each
// read's LDS time; the 64-byte rows of a 32-K slot with
// swz = ((r / 2) ^ (r / 4)) mod 4 had none.)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base) {
  // word 3: 32-bit data format (untyped access); offsets stay below 2^31
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0),
                                           0x7FFFFFFF, 0x00020000);
}

// s_waitcnt vmcnt(n), the other counters unconstrained
template <int n>
__device__ __forceinline__ void wait_vmem() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int EPI, int BN, int WM>
__global__ void __launch_bounds__(kTw, 1)
shared_gemm_wide_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w, int M,
                        int N, int K, uint16_t* __restrict__ out) {
  static_assert(BN == 256 || BN == 128, "tile width");
  constexpr int WN = kWaves / WM;
  constexpr int RM = kBMw / WM;            // rows per wave
  constexpr int MB = RM / 16;              // A blocks per wave
  constexpr int CN = BN / WN;              // columns per wave
  constexpr int NQ = CN / 16;              // column blocks per wave
  static_assert(NQ % 2 == 0 && MB >= 1, "wave tile");
  constexpr int AJ = kBMw / (8 * kWaves);  // A loads per wave and slot (8 rows each)
  constexpr int BJ = BN / (8 * kWaves);    // B loads per wave and slot
  constexpr int L = AJ + BJ;               // loads per lane and slot
  constexpr int SB = slot_bytes<BN>();
  constexpr int kSlots = ring_slots<BN>();
  static_assert(wide_lds_bytes<BN>() <= 160 * 1024, "LDS");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_w[];
  const int n_ntiles = N / BN;
  const int mt = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - mt * n_ntiles;
  const int m0 = mt * kBMw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int ln = lane & 15, kq = lane >> 4;

  // loads: lane -> row lr = lane / 8 of an 8-row load (row group g), LDS chunk
  // lane % 8, which holds K chunk (lane % 8) ^ swz(8 g + lr), i.e. swz(lr) for
  // even g and swz(8 + lr) for odd g.  Wave v loads A row groups AJ v + j
  // (rows past M re-read the last row: their results are never stored) and
  // B-tile row groups BJ v + j.
  // The first BN/2 B-tile rows are weight rows lo_row.., the rest hi_row..
  // (with EPI_SILU_MUL the gate rows and the matching up rows): waves 0..3
  // load lo rows, waves 4..7 hi rows.
  const int lr = lane >> 3;
  const uint32_t chunk0 = uint32_t(((lane & 7) ^ swz(lr)) * 16);       // even row groups
  const uint32_t chunk1 = uint32_t(((lane & 7) ^ swz(8 + lr)) * 16);   // odd row groups
  const uint32_t row_bytes = uint32_t(K) * 2u;
  const int a_rows = min(kBMw, M - m0);
  const __amdgpu_buffer_rsrc_t ares = rows_rsrc(a + int64_t(m0) * K);
  uint32_t aoff[AJ];
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int g = AJ * wave + j;
    aoff[j] = uint32_t(min(8 * g + lr, a_rows - 1)) * row_bytes + ((g & 1) ? chunk1 : chunk0);
  }
  const int64_t lo_row = EPI == MOEQ_EPI_SILU_MUL ? int64_t(nt) * (BN / 2) : int64_t(nt) * BN;
  const int64_t hi_row = EPI == MOEQ_EPI_SILU_MUL ? (N >> 1) + lo_row : lo_row + BN / 2;
  const __amdgpu_buffer_rsrc_t bres = rows_rsrc(w + (wave < kWaves / 2 ? lo_row : hi_row) * K);
  // B row group BJ v + j sits 8 (BJ (v % 4) + j) rows into this wave's run
  const uint32_t brow = uint32_t(lr) * row_bytes;
  const int bgroup0 = BJ * (wave % (kWaves / 2));

  const int slots = K / kBKs;              // >= 1
  // slot st into buffer st % kSlots; past the last slot the last one is read
  // again (into a buffer no later slot reads)
  auto issue = [&](int st) {
    uint8_t* buf = smem_w + (st % kSlots) * SB;
    const int kb = min(st, slots - 1) * kRowB;
#pragma unroll
    for (int j = 0; j < AJ; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, buf + 8 * (AJ * wave + j) * kRowB, 16,
                                               aoff[j], kb, 0, 0);
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int g = bgroup0 + j;           // group within the lo or hi run
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          bres, buf + (kBMw + 8 * (BJ * wave + j)) * kRowB, 16,
          brow + ((g & 1) ? chunk1 : chunk0), int(8 * g * row_bytes) + kb, 0, 0);
    }
  };

  // B-tile row of column block q of this wave
  int cb[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (EPI == MOEQ_EPI_SILU_MUL)
      cb[q] = (q < NQ / 2 ? 0 : BN / 2) + (CN / 2) * wn + 16 * (q % (NQ / 2));
    else
      cb[q] = CN * wn + 16 * q;
  }
  // operand reads of half h (K chunks 4 h .. 4 h + 3) of a slot: row ln of a
  // 16-row block, K chunk 4 h + kq at position (4 h + kq) ^ swz(ln)
  const int rd0 = ln * kRowB + ((kq ^ swz(ln)) * 16);
  const int rd1 = ln * kRowB + (((4 + kq) ^ swz(ln)) * 16);
  struct Ops { v8bf a[MB], b[NQ]; };
  auto read_ops = [&](int st, int h, Ops& o) {
    const uint8_t* buf = smem_w + (st % kSlots) * SB + (h ? rd1 : rd0);
    const uint8_t* A = buf + (RM * wm) * kRowB;
    const uint8_t* B = buf + kBMw * kRowB;
#pragma unroll
    for (int i = 0; i < MB; ++i) o.a[i] = *reinterpret_cast<const v8bf*>(A + 16 * i * kRowB);
#pragma unroll
    for (int q = 0; q < NQ; ++q) o.b[q] = *reinterpret_cast<const v8bf*>(B + cb[q] * kRowB);
  };

  v4f acc[MB][NQ];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](const Ops& o) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < MB; ++i)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[q], acc[i][q], 0, 0, 0);
  };
  // The first kSlots slots are issued up front.  Opening slot st: this lane's
  // loads of st have landed once at most those of the kSlots - 2 slots issued
  // after it are outstanding (kSlots - 1 of them before the first opening);
  // after the barrier every wave's loads of st are in LDS and every wave has
  // read all of slot st - 1 (lgkmcnt(0) ahead of the barrier; the operands of
  // its second half are in registers), whose buffer the loads of
  // st + kSlots - 1 then take.  The barrier is a bare s_barrier: the workgroup
  // fence of __syncthreads would also wait for the loads still in flight.
#pragma unroll
  for (int st = 0; st < kSlots; ++st) issue(st);
  wait_vmem<(kSlots - 1) * L>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  Ops cur, nxt;
  read_ops(0, 0, cur);
  __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the operands of slot 0 in registers
  // slot s: its second half's operands read, its first half's MFMAs; slot
  // s + 1 opened and its first half's operands read, the second half's MFMAs
  for (int s = 0; s < slots; ++s) {
    read_ops(s, 1, nxt);
    mfmas(cur);
    cur = nxt;
    if (s + 1 < slots) {
      wait_vmem<(kSlots - 2) * L>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue(s + kSlots);
      read_ops(s + 1, 0, nxt);
    }
    mfmas(cur);
    cur = nxt;
  }
  wait_vmem<0>();                          // the loads past the last slot

#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + RM * wm + 16 * i + 4 * kq + v;
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

// wave grid: 2 x 4 (128 x 64 per wave) at BN = 256, 4 x 2 (64 x 64) at BN = 128
template <int BN>
constexpr int wide_wm() { return BN == 256 ? 2 : 4; }

template <int BN>
hipError_t launch_wide(const uint16_t* a, const uint16_t* w, int M, int N, int K, int epilogue,
                       uint16_t* out, hipStream_t stream) {
  const int64_t blocks = int64_t((M + kBMw - 1) / kBMw) * (N / BN);
  const size_t lds = wide_lds_bytes<BN>();
  constexpr int WM = wide_wm<BN>();
  auto fn = (epilogue == MOEQ_EPI_SILU_MUL) ? shared_gemm_wide_kernel<MOEQ_EPI_SILU_MUL, BN, WM>
                                            : shared_gemm_wide_kernel<MOEQ_EPI_NONE, BN, WM>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fn, dim3(unsigned(blocks)), dim3(kTw), lds, stream, a, w, M, N, K, out);
  return hipGetLastError();
}

}  // namespace

int shared_wide_bn(int M, int N, int K) {
  // (the buffer loads address a tile's rows with 32-bit offsets: at most 256
  // rows of 2 K bytes, so K stays below 2^21)
  if (M <= 0 || K % kBKs != 0 || K >= (1 << 21)) return 0;
  // 256 x 256 tiles when they give every CU a workgroup, else 256 x 128
  const int64_t mtiles = (M + kBMw - 1) / kBMw;
  if (N % 256 == 0 && mtiles * (N / 256) >= 256) return 256;
  if (N % 128 == 0 && mtiles * (N / 128) >= 256) return 128;
  return 0;
}

hipError_t launch_shared_gemm_wide(int bn, const uint16_t* a, const uint16_t* w, int M, int N,
                                   int K, int epilogue, uint16_t* out, hipStream_t stream) {
  return bn == 256 ? launch_wide<256>(a, w, M, N, K, epilogue, out, stream)
                   : launch_wide<128>(a, w, M, N, K, epilogue, out, stream);
}

}  // namespace moeq
