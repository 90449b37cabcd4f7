// Launchers of the libmoeq kernels.  Arguments are validated by the C-ABI layer
// (api.hip) before any of these is called; each returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moeq.h"

namespace moeq {

// Largest R for which the grouped GEMMs and the expert MLP take the K-split
// wave units (decode-sized batches, about one row per active expert) instead
// of the 64-row tile kernel; measured crossover between 192 and 250 at the
// Inkling-Small shapes with top-6 of 256 experts.
constexpr int kWaveMaxRows = 192;

// plan word offsets (see moe_plan_size in moeq.h)
constexpr int kPlanHeader = 16;
enum PlanWord { kPlanR = 0, kPlanE = 1, kPlanActive = 2, kPlanTiles = 3, kPlanT = 4, kPlanK = 5,
                kPlanDropped = 6 };

struct PlanView {
  int32_t* base;
  int32_t* row_pos;      // [R]   (first: located from R alone)
  int32_t* sorted_rows;  // [R]
  int32_t* offsets;      // [E+1]
  int32_t* active;       // [E]
  int32_t* tile_expert;  // [max_tiles]
  int32_t* tile_row0;    // [max_tiles]
  int32_t* scratch;      // [plan_chunks(R) * E] used while the plan is built
  int max_tiles;
};

__host__ __device__ inline int plan_max_tiles(int E, int R) {
  return (R + MOEQ_TILE_M - 1) / MOEQ_TILE_M + (E < R ? E : R);
}

// chunks of 1024 routed rows ranked by separate workgroups
__host__ __device__ inline int plan_chunks(int R) { return (R + 1023) / 1024 > 0 ? (R + 1023) / 1024 : 1; }

__host__ __device__ inline PlanView plan_view(void* plan, int E, int R) {
  PlanView v;
  v.base = static_cast<int32_t*>(plan);
  v.row_pos = v.base + kPlanHeader;
  v.sorted_rows = v.row_pos + R;
  v.offsets = v.sorted_rows + R;
  v.active = v.offsets + (E + 1);
  v.tile_expert = v.active + E;
  v.max_tiles = plan_max_tiles(E, R);
  v.tile_row0 = v.tile_expert + v.max_tiles;
  v.scratch = v.tile_row0 + v.max_tiles;
  return v;
}

__host__ __device__ inline size_t plan_words(int E, int R) {
  return size_t(kPlanHeader) + size_t(E + 1) + 2 * size_t(R) + size_t(E) +
         2 * size_t(plan_max_tiles(E, R)) + size_t(plan_chunks(R)) * size_t(E);
}

// logits [T, E] = x [T, H] (fp32 or bf16) . Wr [E, H]^T, fp32 accumulation
hipError_t launch_router_logits(const void* x, int x_dtype, int T, int H, const float* wr, int E,
                                float* logits, hipStream_t stream);
hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int renormalize, int32_t* ids, float* w, hipStream_t stream);

hipError_t launch_quant_fp8(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x,
                            uint8_t* q, float* scale, hipStream_t stream);

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, const uint8_t* x_q,
                          const float* x_s, int H, uint8_t* xp_q, float* xp_s, void* plan,
                          hipStream_t stream);

// plan + quantization of x + scatter of the codes (x rows of <= 4096 elements)
hipError_t launch_permute_quant(const int32_t* ids, int T, int k, int E, const void* x,
                                int x_dtype, int H, uint8_t* x_q, float* x_s, uint8_t* xp_q,
                                float* xp_s, void* plan, hipStream_t stream);
hipError_t launch_requant_fnuz(const uint8_t* w_fnuz, const float* s_fnuz, int64_t rows, int K,
                               uint8_t* w_ocp, float* s_ocp, hipStream_t stream);
// streaming read of bytes (a multiple of 16) from buf; one XOR word per wave
// into sink [MOEQ_READ_PROBE_BLOCKS * 4]
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

// packed INT4 rows [rows][K/2] -> the tiled order [rows/16][K/128][16][64]
// (rows % 16 == 0, K % 128 == 0, 16-byte aligned, no overlap)
hipError_t launch_tile_int4(const uint8_t* packed, int64_t rows, int K, uint8_t* tiled,
                            hipStream_t stream);

// INT4 g128 packing; bf16_scales: scales stored as bfloat16 (uint16), else fp32
hipError_t launch_pack_int4(const float* w, int64_t rows, int K, uint8_t* packed, void* scales,
                            int bf16_scales, hipStream_t stream);

// weight formats of the grouped GEMM: INT4 g128 with fp32 or bf16 group scales,
// row-scaled E4M3 (fp32 row scales); w_scale points to scales of that type
enum WeightFormat { kW4G128 = 0, kFp8Row = 1, kW4G128Bf16 = 2, kNvfp4 = 3, kAqlm = 4 };

hipError_t launch_grouped_gemm(int wfmt, const uint8_t* a_q, const float* a_s, const void* plan,
                               int E, int R, const uint8_t* w, const void* w_scale, int N, int K,
                               int epilogue, void* out, int out_dtype, hipStream_t stream);

// NVFP4 weights: E2M1 codes [S, N, K/2], E4M3 block-16 scales [S, N, K/16], fp32
// per-slab scale2 [S]; slab_of [E] maps experts to slabs (values outside
// [0, S): not NVFP4), NULL for the identity
hipError_t launch_grouped_gemm_nvfp4(const uint8_t* a_q, const float* a_s, const void* plan, int E,
                                     int R, const int32_t* slab_of, int S, const uint8_t* w,
                                     const uint8_t* w_block_scale,
                                     const float* w_scale2, int N, int K, int epilogue, void* out,
                                     int out_dtype, hipStream_t stream);

// AQLM weights (1 or 2 codebooks of 8-wide fp16 rows): codes[b] [S, N, K/8]
// (uint8 when book b has <= 256 entries, else int16), codebooks[b] [entries, 8]
// fp16, row_scale [S, N] fp16; slab_of as for NVFP4
constexpr int kAqlmMaxBooks = 2;
hipError_t launch_grouped_gemm_aqlm(const uint8_t* a_q, const float* a_s, const void* plan, int E,
                                    int R, const int32_t* slab_of, int S, int n_books,
                                    const void* const* codes, const int* book_entries,
                                    const uint16_t* const* codebooks, const uint16_t* row_scale,
                                    int N, int K, int epilogue, void* out, int out_dtype,
                                    hipStream_t stream);

// E is read from the plan header on the device.
hipError_t launch_combine(const uint16_t* o, const void* plan, const float* w,
                          const uint16_t* shared, int T, int k, int H, uint16_t* y,
                          hipStream_t stream);

// moe_route_topk + quant_fp8_per_token + moe_permute (with the gather) in one
// launch for T <= kFrontSmallT tokens; separate launches otherwise.
constexpr int kFrontSmallT = 16;
hipError_t launch_front(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, const void* x, int x_dtype, int H, int32_t* ids, float* w,
                        uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, void* plan,
                        hipStream_t stream);

// gate/up GEMM + SiLU, FP8 quantization of h and down GEMM: two launches for
// R <= kWaveMaxRows and I <= 2048 (the down GEMM quantizes h), three otherwise.
hipError_t launch_expert_mlp(int wfmt, const uint8_t* xp_q, const float* xp_s, const void* plan,
                             int E,
                             int R, const uint8_t* w13, const void* s13, const uint8_t* w2,
                             const void* s2, int H, int I, uint16_t* h, uint8_t* h_q, float* h_s,
                             uint16_t* o, hipStream_t stream);

// bytes of the scratch array the allocation-free expert MLP needs for R rows of
// width I (h, h_q, h_s, each 256-byte aligned), and that MLP itself
size_t noalloc_mlp_bytes(int R, int I);
hipError_t launch_expert_mlp_noalloc(int wfmt, const uint8_t* xp_q, const float* xp_s,
                                     const void* plan, int E, int R, const uint8_t* w13,
                                     const void* s13, const uint8_t* w2, const void* s2, int H,
                                     int I, uint16_t* o, hipStream_t stream);

hipError_t launch_shared_gemm_bf16(const uint16_t* a, const uint16_t* w, int M, int N, int K,
                                   int epilogue, uint16_t* out, hipStream_t stream);

}  // namespace moeq
