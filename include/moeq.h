/*
 * moeq.h -- C ABI of libmoeq, the quantized mixture-of-experts expert layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (one sparse MoE layer of an Inkling-Small-shaped model):
 *   route     moe_route_topk        logits -> top-k expert ids and weights
 *   quantize  quant_fp8_per_token   x -> OCP E4M3 codes + one fp32 scale per row
 *   permute   moe_permute           group the (token, slot) rows by expert
 *   gate/up   moe_grouped_gemm_w4a8 (epilogue SILU_MUL)   -> h (bf16)
 *   quantize  quant_fp8_per_token   h -> E4M3 codes + scales
 *   down      moe_grouped_gemm_w4a8 (epilogue NONE)      -> o (bf16)
 *   combine   moe_combine           y_t = sum_j w_tj * o_tj (+ shared_t)
 * with the row-scaled FP8 expert variant (moe_grouped_gemm_fp8row), the offline
 * weight preparation (pack_int4_g128; moe_requant_fp8_fnuz for E4M3FNUZ
 * checkpoints) and the dense bf16 shared-expert GEMM (moe_shared_gemm_bf16).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless stated otherwise.  The library never
 *    allocates, frees or retains them; every buffer is owned by the caller.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream).  No call synchronizes the stream.
 *    Inputs must stay valid until the enqueued work has completed.
 *  - Matrices are row-major and contiguous unless a leading dimension is given.
 *  - Every call returns MOEQ_OK (0) or an error code.  Arguments are validated
 *    before any HIP call is made, so argument errors are reported even on a
 *    machine without a GPU.  MOEQ_ERR_DEVICE means the current device is not
 *    gfx950; MOEQ_ERR_LAUNCH means a kernel launch failed.
 *  - Every call is deterministic: repeated calls on the same inputs produce
 *    bit-identical outputs (no floating-point atomics).
 *  - Values named "bf16" are raw bfloat16 bit patterns (uint16); "E4M3" values
 *    are raw OCP FP8 E4M3 bytes (uint8; max 448; 0x7F/0xFF are NaN).
 *
 * Sources (page title, section) for what each call computes are cited per
 * function.  Where the pages are silent the call documents the reading used.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ_ABI_VERSION 3

/* status codes */
#define MOEQ_OK               0
#define MOEQ_ERR_INVALID_ARG  1  /* null pointer, non-positive size, misalignment, inconsistent sizes */
#define MOEQ_ERR_UNSUPPORTED  2  /* a size outside what the kernels implement (see each call) */
#define MOEQ_ERR_WORKSPACE    3  /* plan buffer smaller than moe_plan_size(E, R) */
#define MOEQ_ERR_DEVICE       4  /* no device, or the current device is not gfx950 */
#define MOEQ_ERR_LAUNCH       5  /* a kernel launch failed (hipGetLastError) */
#define MOEQ_ERR_SCRATCH      6  /* sizes beyond the library's scratch array (no-allocation call) */

/* element types */
#define MOEQ_F32   0
#define MOEQ_BF16  1

/* GEMM epilogues */
#define MOEQ_EPI_NONE      0  /* out[p, n] = acc[p, n]                                   */
#define MOEQ_EPI_SILU_MUL  1  /* out[p, i] = silu(acc[p, i]) * acc[p, N/2 + i], i < N/2  */

/* Rows of one GEMM tile.  The permutation plan lists the tiles of this height. */
#define MOEQ_TILE_M 64

/* Library limits. */
#define MOEQ_MAX_EXPERTS 1024
#define MOEQ_MAX_TOPK    8

int         moe_abi_version(void);
const char* moe_status_string(int status);

/*
 * Bytes of the permutation plan for E experts and R = T*k routed rows.
 *
 * Plan layout (int32 words), written by moe_permute and read by the GEMMs and
 * the combine; callers may read it but must not modify it:
 *   [0] R   [1] E   [2] n_active   [3] n_tiles   [4] T   [5] k
 *   [6] number of ids outside [0, E) that were dropped   [7..15] reserved (0)
 *   row_pos     [R]        routed row r = t*k + j -> sorted position p (-1 if dropped)
 *   sorted_rows [R]        sorted position p -> routed row r
 *   offsets     [E+1]      offsets[e] = first sorted position of expert e
 *   active      [E]        experts with at least one row, increasing (n_active used)
 *   tile_expert [max_tiles] expert of each MOEQ_TILE_M-row tile (n_tiles used)
 *   tile_row0   [max_tiles] first sorted position of each tile
 *   scratch     [chunks * E] per-chunk counts used while the plan is built
 * with max_tiles = ceil(R / MOEQ_TILE_M) + min(E, R) and chunks = max(1, ceil(R / 1024)).
 * Returns 0 for E <= 0 or R < 0.
 *
 * Every call that reads a plan takes its byte count (plan_bytes) and the E and
 * R it was built for, and returns MOEQ_ERR_WORKSPACE when plan_bytes <
 * moe_plan_size(E, R): every device read of the plan then stays inside the
 * buffer.  A plan built by moe_permute for other E or R (the header words 0
 * and 1 record them) is a caller error the library cannot see without reading
 * device memory; the kernels clamp every expert id and row index they take
 * from a plan to [0, E) and [0, R], so such a plan gives wrong values, never an
 * access outside the caller's buffers.
 */
size_t moe_plan_size(int E, int R);

/*
 * moe_router_logits -- the router's linear layer, the step in front of the
 * top-k selection: logits[t, e] = sum_h x[t, h] * w_router[e, h].
 *
 * Each token is routed by its scores over the experts ("Inkling-512k-NVFP4-
 * AQLM-hybrid", intro: 6 of 256 routed experts per token); the pages do not
 * give the router's precision, the reading implemented is fp32 weights and
 * fp32 accumulation (fused multiply-adds; bf16 x is widened exactly).  A bias,
 * if any, is added by moe_route_topk.
 *
 *   x [T, H] fp32 or bf16 (x_dtype)   w_router [E, H] fp32   logits [T, E] fp32 (out)
 * Limits: T >= 0, H % 16 == 0, T*E and E*H < 2^31; x and w_router 16-byte aligned.
 */
int moe_router_logits(const void* x, int x_dtype, int T, int H, const float* w_router, int E,
                      float* logits, void* stream);

/*
 * moe_route_topk -- top-k routing.
 *
 * Inkling routes each token to 6 of its 256 routed experts
 * ("Inkling-512k-NVFP4-AQLM-hybrid", intro).  The routing function itself is
 * not on the pages; the reading implemented: s = logits + bias (one fp32
 * addition; bias may be NULL); the k largest s per token, ties to the lower
 * expert index, written best first; weights w_j = exp(s_j - s_max) divided by
 * the sum over the k selected experts (renormalize != 0) or over all E experts
 * (renormalize == 0).
 *
 *   logits    [T, E] fp32, finite       bias  [E] fp32 or NULL
 *   topk_ids  [T, k] int32 (out)        topk_w [T, k] fp32 (out)
 * Limits: 1 <= E <= MOEQ_MAX_EXPERTS, 1 <= k <= min(E, MOEQ_MAX_TOPK), T >= 0.
 */
int moe_route_topk(const float* logits, const float* bias, int T, int E, int k,
                   int renormalize, int32_t* topk_ids, float* topk_w, void* stream);

/*
 * quant_fp8_per_token -- dynamic per-row FP8 quantization.
 *
 * One scale per token row ("wstewart3/Inkling-Small-W4A8-G128", section 1
 * settings table: dynamic FP8 input activations, token strategy; "Inkling 2
 * Small FP8 for AMD MI300X", "Precision and files": per-token dynamic
 * activations and scale = max(abs(row)) / fmax).  gfx950's FP8 is OCP E4M3,
 * so fmax = 448:
 *   amax = max_k |x[m, k]|;  scale[m] = fp32(amax / 448);
 *   q[m, k] = E4M3_RNE_saturating(fp32(x[m, k] / scale[m]))   (IEEE divisions)
 * A row of zeros gets scale 0 and codes 0x00.  Also used for the row-scaled
 * FP8 expert weights (rows = output channels), which is the same arithmetic.
 *
 *   x      [M, K] fp32 or bf16 (x_dtype), row stride ld_x elements, finite
 *   q      [M, K] E4M3 (out, row stride K)      scale [M] fp32 (out)
 * Limits: M >= 0, K >= 8, K % 8 == 0, ld_x >= K, ld_x % 8 == 0, x 16-byte aligned.
 */
int quant_fp8_per_token(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x,
                        uint8_t* q, float* scale, void* stream);

/*
 * moe_permute -- stable counting sort of the routed rows by expert, and the
 * optional gather of the quantized activations into that order.
 *
 * Needed so that each expert's rows form one contiguous block for the grouped
 * GEMM (the pages name fused grouped-GEMM kernels: "Inkling-512k-NVFP4-AQLM-
 * hybrid", intro and "Serving").  Row r = t*k + j carries expert topk_ids[t, j];
 * rows are ordered by expert and, within one expert, by increasing r.
 *
 *   topk_ids [T, k] int32
 *   x_q [T, H] E4M3 and x_s [T] fp32, or both NULL (plan only)
 *   xp_q [R, H] E4M3 (out): xp_q[p] = x_q[sorted_rows[p] / k]; xp_s [R] likewise
 *   plan (out), plan_bytes >= moe_plan_size(E, T*k)
 * Ids outside [0, E) are dropped (counted in plan word 6, row_pos = -1).
 * Limits: T >= 0, 1 <= k <= MOEQ_MAX_TOPK, 1 <= E <= MOEQ_MAX_EXPERTS,
 * H % 16 == 0 when gathering, x_q / xp_q 16-byte aligned.
 */
int moe_permute(const int32_t* topk_ids, int T, int k, int E,
                const uint8_t* x_q, const float* x_s, int H,
                uint8_t* xp_q, float* xp_s, void* plan, size_t plan_bytes, void* stream);

/*
 * moe_route_quant_permute -- moe_route_topk, quant_fp8_per_token on x and
 * moe_permute (with the gather), in that order, as one call.
 *
 * Every output equals the one the three separate calls produce (same routines,
 * bit-identical).  For T <= 16 tokens (decode-sized batches) all of it runs in a
 * single 1024-thread workgroup launch, which removes three launch latencies
 * from the layer; larger T uses the separate kernels.
 *
 *   logits [T, E] fp32, bias [E] or NULL, x [T, H] fp32 or bf16 (x_dtype)
 *   topk_ids [T, k], topk_w [T, k], x_q [T, H], x_s [T], xp_q [T*k, H], xp_s [T*k],
 *   plan (out; plan_bytes >= moe_plan_size(E, T*k))
 * Limits: those of the three calls; H % 16 == 0; x, x_q, xp_q 16-byte aligned.
 */
int moe_route_quant_permute(const float* logits, const float* bias, int T, int E, int k,
                            int renormalize, const void* x, int x_dtype, int H, int32_t* topk_ids,
                            float* topk_w, uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s,
                            void* plan, size_t plan_bytes, void* stream);

/*
 * pack_int4_g128 -- symmetric INT4 quantization in groups of 128 along K and
 * the physical packing (offline weight preparation).
 *
 * Groups of 128 along the input dimension ("wstewart3/Inkling-Small-W4A8-G128",
 * section 1 settings table; section 6: a [2048, 4096] projection has scales
 * [2048, 32]).  Codes in [-8, 7], stored as nibble = code + 8, eight codes per
 * little-endian int32 word with the first code in the least significant nibble
 * (same page, section 7 "Recover and physically pack INT4").  The scale rule is
 * not on the pages; the reading implemented:
 *   s = fp32(max|group| / 7);  c = clamp(rne(fp32(w / s)), -8, 7);  s = 0 -> c = 0
 *
 *   w        [rows, K] fp32 (rows = experts * output channels), finite
 *   packed   [rows, K/2] bytes (out) -- the byte view of [rows, K/8] int32 words
 *   scales   [rows, K/128] fp32 (out)
 * Limits: rows >= 0, K % 128 == 0, w 16-byte aligned.
 */
int pack_int4_g128(const float* w, int64_t rows, int K, uint8_t* packed, float* scales,
                   void* stream);

/*
 * pack_int4_g128_bf16s -- pack_int4_g128 with bfloat16 group scales.
 *
 * The W4A8 card's payload accounting ("wstewart3/Inkling-Small-W4A8-G128",
 * section 5: the I8 / BF16 / F32 byte totals) implies 16-bit scales in the
 * exported checkpoint.  Reading implemented: the stored scale is the bfloat16
 * rounding (RNE) of fp32(max|group| / 7), and the codes are taken against the
 * stored value:  s = bf16(fp32(a / 7));  c = clamp(rne(fp32(w / s)), -8, 7).
 *
 *   w [rows, K] fp32, packed [rows, K/2] bytes (out), scales [rows, K/128] bf16 (out)
 * Limits: as pack_int4_g128.
 */
int pack_int4_g128_bf16s(const float* w, int64_t rows, int K, uint8_t* packed, uint16_t* scales,
                         void* stream);

/*
 * moe_read_bandwidth_probe -- a measurement helper, not a step of the layer:
 * streams `bytes` from device memory the way a well-fed read stream does (16
 * bytes per lane, consecutive lanes on consecutive addresses, many independent
 * loads in flight per thread, MOEQ_READ_PROBE_BLOCKS workgroups striding over
 * the buffer) and stores the XOR of all 32-bit words read, one partial word per
 * wave, into sink.  Its bytes per second on a buffer much larger than the
 * device's caches is the practical HBM read ceiling that the weight-streaming
 * GEMMs are compared against (the 8 TB/s peak is the interface's, not a rate a
 * kernel reads at).
 *
 *   buf  [bytes] device memory, 16-byte aligned, bytes % 16 == 0 (bytes = 0: nothing)
 *   sink [MOEQ_READ_PROBE_BLOCKS * 4] uint32 (out): the XOR of every sink word
 *        equals the XOR of every 32-bit word of buf
 * Errors: MOEQ_ERR_INVALID_ARG for null, misaligned or ragged buffers, or more
 * than 2^40 bytes.
 */
#define MOEQ_READ_PROBE_BLOCKS 8192
int moe_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * moe_tile_int4_weights -- packed INT4 weights (pack_int4_g128's layout, which is
 * the checkpoint's) into the tiled order every INT4 GEMM and expert-MLP call
 * reads (offline weight preparation, once per weight tensor).
 *
 * The checkpoint stores each output row's packed codes contiguously
 * ("wstewart3/Inkling-Small-W4A8-G128", section 7: I32 [N, K/8] per projection).
 * The kernels read a 128-wide K group of 16 consecutive rows per wave load
 * instruction, which in that order is 16 pieces of 64 bytes 2 KB apart; the
 * tiled order makes them 1024 contiguous bytes.  Tiled order (a permutation of
 * whole bytes; no code changes):
 *   w_tiled[((b * G + g) * 16 + r) * 64 + c] = w_packed[(16 b + r) * K/2 + 64 g + c]
 * for block b < rows/16, group g < G = K/128, row r < 16, byte c < 64.  With
 * N % 16 == 0 the blocks of an expert stack [E, N, K/2] never straddle two
 * experts, so rows = E * N tiles the stack in one call, and tiling it a few
 * experts at a time gives the same bytes.
 *
 *   w_packed [rows, K/2] bytes (the byte view of [rows, K/8] int32 words)
 *   w_tiled  [rows, K/2] bytes (out), not overlapping w_packed
 * Limits: rows % 16 == 0, K % 128 == 0, both buffers 16-byte aligned.
 * Errors: MOEQ_ERR_UNSUPPORTED for rows % 16 != 0 or K % 128 != 0;
 * MOEQ_ERR_INVALID_ARG for overlapping, null or misaligned buffers.
 */
int moe_tile_int4_weights(const uint8_t* w_packed, int64_t rows, int K, uint8_t* w_tiled,
                          void* stream);

/*
 * moe_requant_fp8_fnuz -- row-scaled E4M3FNUZ expert weights to row-scaled OCP
 * E4M3 (offline weight preparation).
 *
 * The row-FP8 MI300X card ("Inkling 2 Small FP8 for AMD MI300X", "Precision and
 * files") stores expert weights as E4M3FNUZ bytes (exponent bias 8, max 240,
 * 0x80 the only NaN) with one fp32 scale per output channel, scale =
 * max|row| / 240, tensors [n_experts, out_channels].  gfx950's FP8 is OCP E4M3,
 * so each row is converted once:
 *   w[r, k]  = fp32(s_fnuz[r] * fnuz(w_fnuz[r, k]))          (one rounding)
 *   s_ocp[r] = fp32(max_k |w[r, k]| / 448)
 *   w_ocp[r, k] = E4M3_RNE_saturating(fp32(w[r, k] / s_ocp[r]))   (IEEE division)
 * i.e. quant_fp8_per_token applied to the dequantized rows.  Reading: the
 * FNUZ NaN code 0x80 is read as 0 (checkpoints hold no NaN weights).
 *
 *   w_fnuz [rows, K] E4M3FNUZ bytes    s_fnuz [rows] fp32 (>= 0)
 *   w_ocp  [rows, K] E4M3 (out)        s_ocp  [rows] fp32 (out)
 * rows = experts * output channels.  Limits: rows >= 0, K % 8 == 0, w_fnuz and
 * w_ocp 8-byte aligned.
 */
int moe_requant_fp8_fnuz(const uint8_t* w_fnuz, const float* s_fnuz, int64_t rows, int K,
                         uint8_t* w_ocp, float* s_ocp, void* stream);

/*
 * moe_grouped_gemm_w4a8 -- grouped GEMM over the routed experts with INT4 g128
 * weights and FP8 activations.
 *
 * INT4 weights with FP8 activations keep the FP8 matrix cores in use
 * ("wstewart3/Inkling-Small-W4A8-G128", intro; section 1 settings table).  For
 * sorted row p of expert e (per the plan) and output column n:
 *   acc[p, n] = sum_g s_w[e, n, g] * sum_{k in group g} E4M3(a_q[p, k]) * c[e, n, k]
 *   v[p, n]   = a_s[p] * acc[p, n]
 * The INT4 codes are converted exactly to E4M3 and multiplied on the FP8 MFMA
 * units; each 128-wide group's fp32 partial sum is scaled by its group scale.
 * Epilogue NONE: out[p, n] = v[p, n]  ([R, N], out_dtype bf16 or fp32).
 * Epilogue SILU_MUL (w13 = gate rows then up rows, "Inkling-512k-NVFP4-AQLM-
 * hybrid", "On-disk tensor format"): out[p, i] = bf16(silu(v[p, i]) * v[p, N/2+i])
 * ([R, N/2], out_dtype must be bf16).
 *
 *   a_q [R, K] E4M3, a_s [R] fp32 -- rows in plan order
 *   plan, plan_bytes -- from moe_permute with the same E and R (read only)
 *   w_packed [E, N, K/2] bytes in the tiled order of moe_tile_int4_weights
 *     (from pack_int4_g128's output, or from the checkpoint's int32
 *     [E, N, K/8] .weight_packed words viewed as bytes), w_scales [E, N, K/128]
 *     fp32 (row order, as written by pack_int4_g128)
 * Limits: K % 128 == 0, N % 128 == 0, R >= 0, 1 <= E <= MOEQ_MAX_EXPERTS;
 * a_q, w_packed and w_scales 16-byte aligned.
 */
int moe_grouped_gemm_w4a8(const uint8_t* a_q, const float* a_s, const void* plan,
                          size_t plan_bytes, int E, int R, const uint8_t* w_packed,
                          const float* w_scales, int N, int K, int epilogue, void* out,
                          int out_dtype, void* stream);

/*
 * moe_grouped_gemm_w4a8_bf16s -- moe_grouped_gemm_w4a8 with bfloat16 group
 * scales w_scales [E, N, K/128] (as written by pack_int4_g128_bf16s; the
 * 16-bit scales the W4A8 card's payload accounting implies, section 5).  Each
 * scale is widened exactly to fp32 and applied as in moe_grouped_gemm_w4a8.
 * Limits and errors: as moe_grouped_gemm_w4a8.
 */
int moe_grouped_gemm_w4a8_bf16s(const uint8_t* a_q, const float* a_s, const void* plan,
                                size_t plan_bytes, int E, int R, const uint8_t* w_packed,
                                const uint16_t* w_scales, int N, int K, int epilogue, void* out,
                                int out_dtype, void* stream);

/*
 * moe_grouped_gemm_nvfp4 -- grouped GEMM over NVFP4 expert weights (the hot
 * experts of the NVFP4 + AQLM hybrid checkpoint) with per-token FP8 activations.
 *
 * Weight format ("Inkling-512k-NVFP4-AQLM-hybrid", "On-disk tensor format" and
 * "Dequant math", hot): E2M1 codes two per byte, the low nibble the first
 * weight; one E4M3 scale per 16 consecutive input channels; one fp32 scale2
 * per expert:  W[e, n, k] = e2m1(code) * e4m3(w_block_scale[e, n, k/16]) * w_scale2[e].
 * For sorted row p of expert e (per the plan):
 *   v[p, n] = a_s[p] * w_scale2[e] * sum_k E4M3(a_q[p, k]) * e2m1(c[e, n, k]) * s_b[e, n, k/16]
 * with exact products and fp32 accumulation; epilogue and out as in
 * moe_grouped_gemm_w4a8.  The activation format is this library's per-token
 * FP8 (the card quantizes only the weights; the reading used here keeps the
 * layer's activation path).
 *
 *   slab_of [E] int32 or NULL: weight slab of each routed expert; a value
 *     outside [0, S) (-1 by convention) marks an expert stored in another
 *     format, whose rows this call leaves untouched (the hybrid card's hot_ids
 *     list the routed expert of each NVFP4 slab; slab_of is its inverse).
 *     NULL: slab e is expert e (then E <= S).
 *   S -- number of slabs in the weight tensors
 *   w_fp4 [S, N, K/2] bytes, w_block_scale [S, N, K/16] E4M3 bytes, w_scale2 [S] fp32
 * Limits: K % 128 == 0, N % 128 == 0, 1 <= E <= MOEQ_MAX_EXPERTS; a_q, w_fp4 and
 * w_block_scale 16-byte aligned.
 */
int moe_grouped_gemm_nvfp4(const uint8_t* a_q, const float* a_s, const void* plan,
                           size_t plan_bytes, int E, int R, const int32_t* slab_of, int S,
                           const uint8_t* w_fp4,
                           const uint8_t* w_block_scale,
                           const float* w_scale2, int N, int K, int epilogue, void* out,
                           int out_dtype, void* stream);

/*
 * moe_grouped_gemm_aqlm -- grouped GEMM over AQLM expert weights (the cold
 * experts of the NVFP4 + AQLM hybrid checkpoint) with per-token FP8 activations.
 *
 * Weight format ("Inkling-512k-NVFP4-AQLM-hybrid", "On-disk tensor format" and
 * "Dequant math", cold): groups of 8 input channels; per book b a code per
 * (row, group) -- uint8 for books of <= 256 entries, else int16 read as
 * idx & 0xFFFF -- selecting an 8-wide fp16 codebook row; one fp16 scale per
 * output row:
 *   W[e, n, 8g:8g+8] = (sum_b codebook_b[codes_b[e, n, g]]) * row_scale[e, n]
 *   v[p, n] = a_s[p] * sum_k E4M3(a_q[p, k]) * W[e, n, k]
 * with exact products and fp32 accumulation (each book's rows enter the sum
 * separately, never added to each other in fp16); epilogue and out as in
 * moe_grouped_gemm_w4a8.
 *
 *   slab_of [E] int32 or NULL, S -- as in moe_grouped_gemm_nvfp4 (cold_ids inverse)
 *   n_books 1 or 2; codes, book_entries, codebooks: HOST arrays of n_books
 *     entries: device pointers to codes_b [S, N, K/8], the entry counts
 *     (1 .. 65536), device pointers to codebook_b [entries_b, 8] fp16
 *   row_scale [S, N] fp16
 * Codes at or past a book's entry count are invalid input; they read the
 * book's last row.
 * Limits: K % 128 == 0, N % 128 == 0, 1 <= E <= MOEQ_MAX_EXPERTS; a_q and the
 * codebooks 16-byte aligned, int16 codes 8-byte and uint8 codes 4-byte aligned.
 */
int moe_grouped_gemm_aqlm(const uint8_t* a_q, const float* a_s, const void* plan,
                          size_t plan_bytes, int E, int R, const int32_t* slab_of, int S,
                          int n_books, const void* const* codes,
                          const int* book_entries, const uint16_t* const* codebooks,
                          const uint16_t* row_scale, int N, int K, int epilogue, void* out,
                          int out_dtype, void* stream);

/*
 * moe_grouped_gemm_fp8row -- grouped GEMM with row-scaled FP8 expert weights.
 *
 * Expert weights E4M3 with one fp32 scale per output channel, scale tensor
 * [n_experts, out_channels] ("Inkling 2 Small FP8 for AMD MI300X", "Precision
 * and files"):
 *   v[p, n] = a_s[p] * s_row[e, n] * sum_k E4M3(a_q[p, k]) * E4M3(w[e, n, k])
 * Epilogues as for moe_grouped_gemm_w4a8.
 *
 *   w_fp8 [E, N, K] E4M3, w_row_scale [E, N] fp32
 * Limits: K % 128 == 0, N % 128 == 0; a_q, w_fp8 and w_row_scale 16-byte aligned.
 */
int moe_grouped_gemm_fp8row(const uint8_t* a_q, const float* a_s, const void* plan,
                            size_t plan_bytes, int E, int R, const uint8_t* w_fp8,
                            const float* w_row_scale, int N, int K, int epilogue, void* out,
                            int out_dtype, void* stream);

/*
 * moe_expert_mlp_w4a8 -- the routed experts' MLP: gate/up GEMM with the
 * SiLU-gated product, FP8 quantization of h, down GEMM.
 *
 * Exactly the three calls
 *   moe_grouped_gemm_w4a8(xp_q, xp_s, w13, N = 2I, K = H, SILU_MUL) -> h
 *   quant_fp8_per_token(h)                                          -> h_q, h_s
 *   moe_grouped_gemm_w4a8(h_q, h_s, w2, N = H, K = I, NONE)          -> o (bf16)
 * with bit-identical results.  For R <= 192 (decode-sized batches) and
 * I <= 2048 the down GEMM quantizes h itself -- each of its waves quantizes its
 * K quarter of the rows of h into LDS while its weight loads are in flight --
 * so the call makes two launches instead of three; otherwise the three.
 *
 *   xp_q [R, H] E4M3, xp_s [R] fp32 -- rows in plan order (moe_permute)
 *   plan, plan_bytes -- from moe_permute / moe_route_quant_permute with E, R (read only)
 *   w13 [E, 2I, H/2] packed INT4 (gate rows then up rows), w13_scales [E, 2I, H/128]
 *   w2  [E, H, I/2] packed INT4, w2_scales [E, H, I/128]
 *   (both weight tensors in the tiled order of moe_tile_int4_weights)
 *   h [R, I] bf16, h_q [R, I] E4M3, h_s [R] fp32, o [R, H] bf16 (outputs)
 * Limits: H % 128 == 0, I % 128 == 0, 1 <= E <= MOEQ_MAX_EXPERTS; xp_q, h_q,
 * the weights and their scales 16-byte aligned.
 */
int moe_expert_mlp_w4a8(const uint8_t* xp_q, const float* xp_s, const void* plan, size_t plan_bytes,
                        int E, int R, const uint8_t* w13, const float* w13_scales,
                        const uint8_t* w2, const float* w2_scales, int H, int I, uint16_t* h,
                        uint8_t* h_q, float* h_s, uint16_t* o, void* stream);

/*
 * moe_expert_mlp_w4a8_bf16s -- moe_expert_mlp_w4a8 with bfloat16 group scales
 * (w13_scales [E, 2I, H/128], w2_scales [E, H, I/128]): exactly the three calls
 * with moe_grouped_gemm_w4a8_bf16s, bit-identical.  Limits: as
 * moe_expert_mlp_w4a8.
 */
int moe_expert_mlp_w4a8_bf16s(const uint8_t* xp_q, const float* xp_s, const void* plan,
                              size_t plan_bytes, int E, int R, const uint8_t* w13,
                              const uint16_t* w13_scales, const uint8_t* w2,
                              const uint16_t* w2_scales, int H, int I, uint16_t* h, uint8_t* h_q,
                              float* h_s, uint16_t* o, void* stream);

/*
 * moe_expert_mlp_w4a8_noalloc -- moe_expert_mlp_w4a8 for callers that cannot
 * allocate device memory (code under graph capture, serving loops, harnesses
 * that forbid allocation): the caller passes only the inputs and o; the
 * intermediates h, h_q and h_s live in a device array inside the library of
 * MOEQ_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  o equals moe_expert_mlp_w4a8's o bit for bit.
 *
 * Size limit: 256-byte-aligned h (R*I*2), h_q (R*I) and h_s (R*4) together
 * within MOEQ_NOALLOC_SCRATCH_BYTES (R <= 5457 at I = 2048), else
 * MOEQ_ERR_SCRATCH.  Every call on one GPU uses the same array: calls that
 * overlap on a GPU (other streams, other host threads) race and must be
 * serialized by the caller; calls on one stream are ordered.  The call
 * allocates nothing, on the host or the device.
 * Arguments, other limits and errors: as moe_expert_mlp_w4a8.
 */
#define MOEQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moe_expert_mlp_w4a8_noalloc(const uint8_t* xp_q, const float* xp_s, const void* plan,
                                size_t plan_bytes, int E, int R, const uint8_t* w13,
                                const float* w13_scales, const uint8_t* w2,
                                const float* w2_scales, int H, int I, uint16_t* o, void* stream);

/*
 * moe_expert_mlp_fp8row -- moe_expert_mlp_w4a8 with row-scaled FP8 expert
 * weights (the moe_grouped_gemm_fp8row arithmetic):
 *   w13 [E, 2I, H] E4M3, w13_scales [E, 2I] fp32; w2 [E, H, I] E4M3, w2_scales [E, H] fp32.
 */
int moe_expert_mlp_fp8row(const uint8_t* xp_q, const float* xp_s, const void* plan,
                          size_t plan_bytes,
                          int E, int R, const uint8_t* w13, const float* w13_scales,
                          const uint8_t* w2, const float* w2_scales, int H, int I, uint16_t* h,
                          uint8_t* h_q, float* h_s, uint16_t* o, void* stream);

/*
 * moe_combine -- weighted sum of each token's expert outputs.
 *
 * Not on the pages; the reading implemented (fp32 accumulation in slot order):
 *   y[t, c] = bf16( sum_{j=0}^{k-1} w[t, j] * o[row_pos[t*k + j], c] + shared[t, c] )
 * Rows dropped by moe_permute contribute nothing.
 *
 *   o [R, H] bf16 in plan order (R = T*k)
 *   plan, plan_bytes -- from moe_permute with E and R = T*k (read only)
 *   topk_w [T, k] fp32;  shared [T, H] bf16 or NULL;  y [T, H] bf16 (out)
 * Limits: H % 8 == 0, 1 <= k <= MOEQ_MAX_TOPK, 1 <= E <= MOEQ_MAX_EXPERTS;
 * o, shared and y 16-byte aligned.
 */
int moe_combine(const uint16_t* o, const void* plan, size_t plan_bytes, int E,
                const float* topk_w, const uint16_t* shared, int T, int k, int H, uint16_t* y,
                void* stream);

/*
 * moe_shared_gemm_bf16 -- dense bf16 GEMM for the shared experts.
 *
 * Inkling-Small keeps its 2 shared experts per sparse layer in BF16: the W4A8
 * conversion quantizes only the routed experts' weights
 * ("wstewart3/Inkling-Small-W4A8-G128", section 1 table; section 7 dry-run
 * table lists the shared gate/up pairs among the unquantized tensors).  out = epilogue(a @ w^T) with fp32 accumulation:
 *   NONE:     out[m, n] = bf16(acc[m, n])                       [M, N]
 *   SILU_MUL: out[m, i] = bf16(silu(acc[m, i]) * acc[m, N/2+i])  [M, N/2]
 *
 *   a [M, K] bf16, w [N, K] bf16 (out, in orientation)
 * Limits: M >= 0, K % 32 == 0, N % 128 == 0; a and w 16-byte aligned.
 */
int moe_shared_gemm_bf16(const uint16_t* a, const uint16_t* w, int M, int N, int K, int epilogue,
                         uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
