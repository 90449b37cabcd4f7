// C ABI of libmoeq (declared in include/moeq.h): argument validation, the
// gfx950 device check, and the kernel launches on the caller's stream.
//
// Validation happens before any HIP call, so argument errors are reported on a
// machine without a GPU.  No entry point allocates, frees or synchronizes.
#include <string.h>

#include "kernels.hpp"

namespace {

constexpr int kMaxDevices = 64;
// per-device result of the architecture check: 0 unknown, 1 gfx950, -1 other
int g_device_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOEQ_ERR_DEVICE;
  if (dev < kMaxDevices && g_device_ok[dev] != 0) return g_device_ok[dev] > 0 ? MOEQ_OK : MOEQ_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOEQ_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_ok[dev] = ok ? 1 : -1;
  return ok ? MOEQ_OK : MOEQ_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(hipError_t err) { return err == hipSuccess ? MOEQ_OK : MOEQ_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// a plan read by a kernel: 4-byte aligned and at least moe_plan_size(E, R) bytes
int check_plan(const void* plan, size_t plan_bytes, int E, int R) {
  if (reinterpret_cast<uintptr_t>(plan) & 3u) return MOEQ_ERR_INVALID_ARG;
  if (plan_bytes < moeq::plan_words(E, R) * sizeof(int32_t)) return MOEQ_ERR_WORKSPACE;
  return MOEQ_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOEQ_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOEQ_OK: return "ok";
    case MOEQ_ERR_INVALID_ARG: return "invalid argument";
    case MOEQ_ERR_UNSUPPORTED: return "unsupported size";
    case MOEQ_ERR_WORKSPACE: return "plan buffer too small";
    case MOEQ_ERR_DEVICE: return "no gfx950 device";
    case MOEQ_ERR_LAUNCH: return "kernel launch failed";
    case MOEQ_ERR_SCRATCH: return "sizes exceed the library's scratch array";
    default: return "unknown status";
  }
}

size_t moe_plan_size(int E, int R) {
  if (E <= 0 || R < 0) return 0;
  return moeq::plan_words(E, R) * sizeof(int32_t);
}

int moe_route_topk(const float* logits, const float* bias, int T, int E, int k, int renormalize,
                   int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E <= 0 || k <= 0) return MOEQ_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w)) return MOEQ_ERR_INVALID_ARG;
  if (k > E) return MOEQ_ERR_INVALID_ARG;
  if (E > MOEQ_MAX_EXPERTS || k > MOEQ_MAX_TOPK) return MOEQ_ERR_UNSUPPORTED;
  if (T == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_route_topk(logits, bias, T, E, k, renormalize, topk_ids,
                                               topk_w, as_stream(stream)));
}

int moe_router_logits(const void* x, int x_dtype, int T, int H, const float* w_router, int E,
                      float* logits, void* stream) {
  if (T < 0 || H <= 0 || E <= 0) return MOEQ_ERR_INVALID_ARG;
  if (x_dtype != MOEQ_F32 && x_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (T > 0 && (!x || !w_router || !logits)) return MOEQ_ERR_INVALID_ARG;
  if (H % 16 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(T) * E > 0x7FFFFFFF || int64_t(E) * H > 0x7FFFFFFF) return MOEQ_ERR_UNSUPPORTED;
  if (T > 0 && (!aligned16(x) || !aligned16(w_router) || (reinterpret_cast<uintptr_t>(logits) & 3u)))
    return MOEQ_ERR_INVALID_ARG;
  if (T == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(
      moeq::launch_router_logits(x, x_dtype, T, H, w_router, E, logits, as_stream(stream)));
}

int quant_fp8_per_token(const void* x, int x_dtype, int64_t M, int K, int64_t ld_x, uint8_t* q,
                        float* scale, void* stream) {
  if (M < 0 || K <= 0 || ld_x < K) return MOEQ_ERR_INVALID_ARG;
  if (x_dtype != MOEQ_F32 && x_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (M > 0 && (!x || !q || !scale)) return MOEQ_ERR_INVALID_ARG;
  if (K % 8 != 0 || ld_x % 8 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (M > 0 && (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u))) return MOEQ_ERR_INVALID_ARG;
  if (M == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_quant_fp8(x, x_dtype, M, K, ld_x, q, scale, as_stream(stream)));
}

int moe_requant_fp8_fnuz(const uint8_t* w_fnuz, const float* s_fnuz, int64_t rows, int K,
                         uint8_t* w_ocp, float* s_ocp, void* stream) {
  if (rows < 0 || K <= 0) return MOEQ_ERR_INVALID_ARG;
  if (rows > 0 && (!w_fnuz || !s_fnuz || !w_ocp || !s_ocp)) return MOEQ_ERR_INVALID_ARG;
  if (K % 8 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (rows > 0 && ((reinterpret_cast<uintptr_t>(w_fnuz) & 7u) ||
                   (reinterpret_cast<uintptr_t>(w_ocp) & 7u)))
    return MOEQ_ERR_INVALID_ARG;
  if (rows == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(
      moeq::launch_requant_fnuz(w_fnuz, s_fnuz, rows, K, w_ocp, s_ocp, as_stream(stream)));
}

int moe_permute(const int32_t* topk_ids, int T, int k, int E, const uint8_t* x_q, const float* x_s,
                int H, uint8_t* xp_q, float* xp_s, void* plan, size_t plan_bytes, void* stream) {
  if (T < 0 || k <= 0 || E <= 0 || !plan) return MOEQ_ERR_INVALID_ARG;
  if (E > MOEQ_MAX_EXPERTS || k > MOEQ_MAX_TOPK) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(T) * k > 0x3FFFFFFF) return MOEQ_ERR_UNSUPPORTED;
  if (T > 0 && !topk_ids) return MOEQ_ERR_INVALID_ARG;
  const int R = T * k;
  const bool gather = x_q != nullptr || x_s != nullptr;
  if (gather) {
    if (!x_q || !x_s || !xp_q || !xp_s || H <= 0) return MOEQ_ERR_INVALID_ARG;
    if (H % 16 != 0) return MOEQ_ERR_UNSUPPORTED;
    if (!aligned16(x_q) || !aligned16(xp_q)) return MOEQ_ERR_INVALID_ARG;
  }
  if (plan_bytes < moe_plan_size(E, R)) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(plan) & 3u) return MOEQ_ERR_INVALID_ARG;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_permute(topk_ids, T, k, E, gather ? x_q : nullptr, x_s, H, xp_q,
                                            xp_s, plan, as_stream(stream)));
}

int moe_route_quant_permute(const float* logits, const float* bias, int T, int E, int k,
                            int renormalize, const void* x, int x_dtype, int H, int32_t* topk_ids,
                            float* topk_w, uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s,
                            void* plan, size_t plan_bytes, void* stream) {
  if (T < 0 || E <= 0 || k <= 0 || H <= 0 || !plan) return MOEQ_ERR_INVALID_ARG;
  if (x_dtype != MOEQ_F32 && x_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (k > E) return MOEQ_ERR_INVALID_ARG;
  if (E > MOEQ_MAX_EXPERTS || k > MOEQ_MAX_TOPK) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(T) * k > 0x3FFFFFFF || H % 16 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (T > 0 && (!logits || !x || !topk_ids || !topk_w || !x_q || !x_s || !xp_q || !xp_s))
    return MOEQ_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x) || !aligned16(x_q) || !aligned16(xp_q))) return MOEQ_ERR_INVALID_ARG;
  if (plan_bytes < moe_plan_size(E, T * k)) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(plan) & 3u) return MOEQ_ERR_INVALID_ARG;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_front(logits, bias, T, E, k, renormalize, x, x_dtype, H,
                                          topk_ids, topk_w, x_q, x_s, xp_q, xp_s, plan,
                                          as_stream(stream)));
}

static int pack_common(const float* w, int64_t rows, int K, uint8_t* packed, void* scales,
                       int bf16_scales, void* stream) {
  if (rows < 0 || K <= 0) return MOEQ_ERR_INVALID_ARG;
  if (K % 128 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (rows > 0 && (!w || !packed || !scales)) return MOEQ_ERR_INVALID_ARG;
  if (rows > 0 && (!aligned16(w) || (reinterpret_cast<uintptr_t>(packed) & 3u)))
    return MOEQ_ERR_INVALID_ARG;
  if (rows == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(
      moeq::launch_pack_int4(w, rows, K, packed, scales, bf16_scales, as_stream(stream)));
}

int pack_int4_g128(const float* w, int64_t rows, int K, uint8_t* packed, float* scales,
                   void* stream) {
  return pack_common(w, rows, K, packed, scales, 0, stream);
}

int pack_int4_g128_bf16s(const float* w, int64_t rows, int K, uint8_t* packed, uint16_t* scales,
                         void* stream) {
  return pack_common(w, rows, K, packed, scales, 1, stream);
}

int moe_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return MOEQ_OK;
  if (!buf || !sink || !aligned16(buf) || bytes % 16 != 0 || bytes > (size_t(1) << 40))
    return MOEQ_ERR_INVALID_ARG;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_read_probe(buf, int64_t(bytes), sink, as_stream(stream)));
}

int moe_tile_int4_weights(const uint8_t* w_packed, int64_t rows, int K, uint8_t* w_tiled,
                          void* stream) {
  if (rows < 0 || K <= 0) return MOEQ_ERR_INVALID_ARG;
  if (K % 128 != 0 || rows % 16 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (rows == 0) return MOEQ_OK;
  if (!w_packed || !w_tiled || !aligned16(w_packed) || !aligned16(w_tiled))
    return MOEQ_ERR_INVALID_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w_packed);
  const uintptr_t b = reinterpret_cast<uintptr_t>(w_tiled);
  const uintptr_t n = uintptr_t(rows) * uintptr_t(K / 2);
  if (a < b + n && b < a + n) return MOEQ_ERR_INVALID_ARG;      // the ranges overlap
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_tile_int4(w_packed, rows, K, w_tiled, as_stream(stream)));
}

static int gemm_common(int wfmt, const uint8_t* a_q, const float* a_s, const void* plan,
                       size_t plan_bytes, int E, int R, const uint8_t* w, const void* w_scale, int N,
                       int K, int epilogue, void* out, int out_dtype, void* stream) {
  if (R < 0 || E <= 0 || N <= 0 || K <= 0) return MOEQ_ERR_INVALID_ARG;
  if (epilogue != MOEQ_EPI_NONE && epilogue != MOEQ_EPI_SILU_MUL) return MOEQ_ERR_INVALID_ARG;
  if (out_dtype != MOEQ_F32 && out_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (epilogue == MOEQ_EPI_SILU_MUL && out_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (E > MOEQ_MAX_EXPERTS) return MOEQ_ERR_UNSUPPORTED;
  if (K % 128 != 0 || N % 128 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(N / 128) * moeq::plan_max_tiles(E, R) > 0x7FFFFFF0) return MOEQ_ERR_UNSUPPORTED;
  if (R > 0 && (!a_q || !a_s || !plan || !w || !w_scale || !out)) return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && (!aligned16(a_q) || !aligned16(w) || !aligned16(w_scale))) return MOEQ_ERR_INVALID_ARG;
  if (R == 0) return MOEQ_OK;
  if (int rc = check_plan(plan, plan_bytes, E, R)) return rc;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_grouped_gemm(wfmt, a_q, a_s, plan, E, R, w, w_scale, N, K,
                                                 epilogue, out, out_dtype, as_stream(stream)));
}

int moe_grouped_gemm_w4a8(const uint8_t* a_q, const float* a_s, const void* plan,
                          size_t plan_bytes, int E, int R, const uint8_t* w_packed,
                          const float* w_scales, int N, int K, int epilogue, void* out,
                          int out_dtype, void* stream) {
  return gemm_common(moeq::kW4G128, a_q, a_s, plan, plan_bytes, E, R, w_packed, w_scales, N, K,
                     epilogue, out, out_dtype, stream);
}

int moe_grouped_gemm_w4a8_bf16s(const uint8_t* a_q, const float* a_s, const void* plan,
                                size_t plan_bytes, int E, int R, const uint8_t* w_packed,
                                const uint16_t* w_scales, int N, int K, int epilogue, void* out,
                                int out_dtype, void* stream) {
  return gemm_common(moeq::kW4G128Bf16, a_q, a_s, plan, plan_bytes, E, R, w_packed, w_scales, N,
                     K, epilogue, out, out_dtype, stream);
}

// checks shared by the NVFP4 and AQLM grouped GEMMs
static int hybrid_common(const uint8_t* a_q, const float* a_s, const void* plan,
                         size_t plan_bytes, int E, int R, const int32_t* slab_of, int S, int N,
                         int K, int epilogue, void* out, int out_dtype) {
  if (R < 0 || E <= 0 || N <= 0 || K <= 0 || S < 0) return MOEQ_ERR_INVALID_ARG;
  if (epilogue != MOEQ_EPI_NONE && epilogue != MOEQ_EPI_SILU_MUL) return MOEQ_ERR_INVALID_ARG;
  if (out_dtype != MOEQ_F32 && out_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (epilogue == MOEQ_EPI_SILU_MUL && out_dtype != MOEQ_BF16) return MOEQ_ERR_INVALID_ARG;
  if (!slab_of && E > S) return MOEQ_ERR_INVALID_ARG;     // identity map needs a slab per expert
  if (E > MOEQ_MAX_EXPERTS) return MOEQ_ERR_UNSUPPORTED;
  if (K % 128 != 0 || N % 128 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(N / 32) * moeq::plan_max_tiles(E, R) > 0x7FFFFFF0) return MOEQ_ERR_UNSUPPORTED;
  if (R > 0 && (!a_q || !a_s || !plan || !out)) return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && !aligned16(a_q)) return MOEQ_ERR_INVALID_ARG;
  if (R > 0) return check_plan(plan, plan_bytes, E, R);
  return MOEQ_OK;
}

int moe_grouped_gemm_nvfp4(const uint8_t* a_q, const float* a_s, const void* plan,
                           size_t plan_bytes, int E, int R, const int32_t* slab_of, int S,
                           const uint8_t* w_fp4, const uint8_t* w_block_scale,
                           const float* w_scale2, int N, int K, int epilogue, void* out,
                           int out_dtype, void* stream) {
  if (int rc = hybrid_common(a_q, a_s, plan, plan_bytes, E, R, slab_of, S, N, K, epilogue, out,
                             out_dtype))
    return rc;
  if (R > 0 && S > 0 && (!w_fp4 || !w_block_scale || !w_scale2)) return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && S > 0 && (!aligned16(w_fp4) || !aligned16(w_block_scale)))
    return MOEQ_ERR_INVALID_ARG;
  if (R == 0 || S == 0) return MOEQ_OK;               // no expert is stored in this format
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_grouped_gemm_nvfp4(a_q, a_s, plan, E, R, slab_of, S, w_fp4,
                                                       w_block_scale, w_scale2, N, K, epilogue,
                                                       out, out_dtype, as_stream(stream)));
}

int moe_grouped_gemm_aqlm(const uint8_t* a_q, const float* a_s, const void* plan,
                          size_t plan_bytes, int E, int R, const int32_t* slab_of, int S,
                          int n_books, const void* const* codes, const int* book_entries,
                          const uint16_t* const* codebooks, const uint16_t* row_scale, int N, int K,
                          int epilogue, void* out, int out_dtype, void* stream) {
  if (int rc = hybrid_common(a_q, a_s, plan, plan_bytes, E, R, slab_of, S, N, K, epilogue, out,
                             out_dtype))
    return rc;
  if (n_books < 1 || n_books > moeq::kAqlmMaxBooks) return MOEQ_ERR_UNSUPPORTED;
  if (!codes || !book_entries || !codebooks) return MOEQ_ERR_INVALID_ARG;
  for (int b = 0; b < n_books; ++b)
    if (book_entries[b] < 1 || book_entries[b] > 65536) return MOEQ_ERR_UNSUPPORTED;
  if (R > 0 && S > 0 && !row_scale) return MOEQ_ERR_INVALID_ARG;
  for (int b = 0; R > 0 && S > 0 && b < n_books; ++b) {
    if (!codes[b] || !codebooks[b]) return MOEQ_ERR_INVALID_ARG;
    const uintptr_t align = book_entries[b] > 256 ? 7u : 3u;      // 8- or 4-byte code loads
    if ((reinterpret_cast<uintptr_t>(codes[b]) & align) || !aligned16(codebooks[b]))
      return MOEQ_ERR_INVALID_ARG;
  }
  if (R > 0 && S > 0 && (reinterpret_cast<uintptr_t>(row_scale) & 1u)) return MOEQ_ERR_INVALID_ARG;
  if (R == 0 || S == 0) return MOEQ_OK;               // no expert is stored in this format
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_grouped_gemm_aqlm(a_q, a_s, plan, E, R, slab_of, S, n_books,
                                                      codes, book_entries, codebooks, row_scale,
                                                      N, K, epilogue, out, out_dtype,
                                                      as_stream(stream)));
}

int moe_grouped_gemm_fp8row(const uint8_t* a_q, const float* a_s, const void* plan,
                            size_t plan_bytes, int E, int R, const uint8_t* w_fp8,
                            const float* w_row_scale, int N, int K, int epilogue, void* out,
                            int out_dtype, void* stream) {
  return gemm_common(moeq::kFp8Row, a_q, a_s, plan, plan_bytes, E, R, w_fp8, w_row_scale, N, K,
                     epilogue, out, out_dtype, stream);
}

// the checks of the expert MLP calls; with_intermediates: h, h_q, h_s are
// caller buffers (else the library's scratch array holds them)
static int mlp_checks(const uint8_t* xp_q, const float* xp_s, const void* plan, size_t plan_bytes,
                      int E, int R, const uint8_t* w13, const void* s13, const uint8_t* w2,
                      const void* s2, int H, int I, bool with_intermediates, const uint16_t* h,
                      const uint8_t* h_q, const float* h_s, const uint16_t* o) {
  if (R < 0 || E <= 0 || H <= 0 || I <= 0) return MOEQ_ERR_INVALID_ARG;
  if (E > MOEQ_MAX_EXPERTS) return MOEQ_ERR_UNSUPPORTED;
  if (H % 128 != 0 || I % 128 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(2 * int64_t(I) / 128) * moeq::plan_max_tiles(E, R) > 0x7FFFFFF0 ||
      int64_t(H / 128) * moeq::plan_max_tiles(E, R) > 0x7FFFFFF0)
    return MOEQ_ERR_UNSUPPORTED;
  if (R > 0 && (!xp_q || !xp_s || !plan || !w13 || !s13 || !w2 || !s2 || !o))
    return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && with_intermediates && (!h || !h_q || !h_s)) return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && (!aligned16(xp_q) || !aligned16(w13) || !aligned16(s13) || !aligned16(w2) ||
                !aligned16(s2)))
    return MOEQ_ERR_INVALID_ARG;
  if (R > 0 && with_intermediates && (!aligned16(h_q) || !aligned16(h))) return MOEQ_ERR_INVALID_ARG;
  if (R == 0) return MOEQ_OK;
  return check_plan(plan, plan_bytes, E, R);
}

static int mlp_common(int wfmt, const uint8_t* xp_q, const float* xp_s, const void* plan,
                      size_t plan_bytes, int E, int R, const uint8_t* w13, const void* s13,
                      const uint8_t* w2, const void* s2, int H, int I, uint16_t* h, uint8_t* h_q,
                      float* h_s, uint16_t* o, void* stream) {
  if (int rc = mlp_checks(xp_q, xp_s, plan, plan_bytes, E, R, w13, s13, w2, s2, H, I, true, h,
                          h_q, h_s, o))
    return rc;
  if (R == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_expert_mlp(wfmt, xp_q, xp_s, plan, E, R, w13, s13, w2, s2, H,
                                               I, h, h_q, h_s, o, as_stream(stream)));
}

int moe_expert_mlp_w4a8(const uint8_t* xp_q, const float* xp_s, const void* plan, size_t plan_bytes,
                        int E, int R, const uint8_t* w13, const float* w13_scales,
                        const uint8_t* w2, const float* w2_scales, int H, int I, uint16_t* h,
                        uint8_t* h_q, float* h_s, uint16_t* o, void* stream) {
  return mlp_common(moeq::kW4G128, xp_q, xp_s, plan, plan_bytes, E, R, w13, w13_scales, w2,
                    w2_scales, H, I, h, h_q, h_s, o, stream);
}

int moe_expert_mlp_w4a8_bf16s(const uint8_t* xp_q, const float* xp_s, const void* plan,
                              size_t plan_bytes, int E, int R, const uint8_t* w13,
                              const uint16_t* w13_scales, const uint8_t* w2,
                              const uint16_t* w2_scales, int H, int I, uint16_t* h, uint8_t* h_q,
                              float* h_s, uint16_t* o, void* stream) {
  return mlp_common(moeq::kW4G128Bf16, xp_q, xp_s, plan, plan_bytes, E, R, w13, w13_scales, w2,
                    w2_scales, H, I, h, h_q, h_s, o, stream);
}

int moe_expert_mlp_fp8row(const uint8_t* xp_q, const float* xp_s, const void* plan,
                          size_t plan_bytes,
                          int E, int R, const uint8_t* w13, const float* w13_scales,
                          const uint8_t* w2, const float* w2_scales, int H, int I, uint16_t* h,
                          uint8_t* h_q, float* h_s, uint16_t* o, void* stream) {
  return mlp_common(moeq::kFp8Row, xp_q, xp_s, plan, plan_bytes, E, R, w13, w13_scales, w2,
                    w2_scales, H, I, h, h_q, h_s, o, stream);
}

int moe_expert_mlp_w4a8_noalloc(const uint8_t* xp_q, const float* xp_s, const void* plan,
                                size_t plan_bytes, int E, int R, const uint8_t* w13,
                                const float* w13_scales, const uint8_t* w2,
                                const float* w2_scales, int H, int I, uint16_t* o, void* stream) {
  if (int rc = mlp_checks(xp_q, xp_s, plan, plan_bytes, E, R, w13, w13_scales, w2, w2_scales, H,
                          I, false, nullptr, nullptr, nullptr, o))
    return rc;
  if (R == 0) return MOEQ_OK;
  if (moeq::noalloc_mlp_bytes(R, I) > MOEQ_NOALLOC_SCRATCH_BYTES) return MOEQ_ERR_SCRATCH;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_expert_mlp_noalloc(moeq::kW4G128, xp_q, xp_s, plan, E, R, w13,
                                                       w13_scales, w2, w2_scales, H, I, o,
                                                       as_stream(stream)));
}

int moe_combine(const uint16_t* o, const void* plan, size_t plan_bytes, int E,
                const float* topk_w, const uint16_t* shared, int T, int k, int H, uint16_t* y,
                void* stream) {
  if (T < 0 || k <= 0 || H <= 0 || E <= 0) return MOEQ_ERR_INVALID_ARG;
  if (k > MOEQ_MAX_TOPK || E > MOEQ_MAX_EXPERTS) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t(T) * k > 0x3FFFFFFF) return MOEQ_ERR_UNSUPPORTED;
  if (H % 8 != 0) return MOEQ_ERR_UNSUPPORTED;
  if ((H / 8 + 255) / 256 > 65535) return MOEQ_ERR_UNSUPPORTED;   // grid (T, 2048-column blocks)
  if (T > 0 && (!o || !plan || !topk_w || !y)) return MOEQ_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(o) || !aligned16(y) || (shared && !aligned16(shared))))
    return MOEQ_ERR_INVALID_ARG;
  if (T == 0) return MOEQ_OK;
  if (int rc = check_plan(plan, plan_bytes, E, T * k)) return rc;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_combine(o, plan, topk_w, shared, T, k, H, y, as_stream(stream)));
}

int moe_shared_gemm_bf16(const uint16_t* a, const uint16_t* w, int M, int N, int K, int epilogue,
                         uint16_t* out, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return MOEQ_ERR_INVALID_ARG;
  if (epilogue != MOEQ_EPI_NONE && epilogue != MOEQ_EPI_SILU_MUL) return MOEQ_ERR_INVALID_ARG;
  if (K % 32 != 0 || N % 128 != 0) return MOEQ_ERR_UNSUPPORTED;
  if (int64_t((M + 127) / 128) * (N / 128) > 0x7FFFFFFF) return MOEQ_ERR_UNSUPPORTED;
  if (M > 0 && (!a || !w || !out)) return MOEQ_ERR_INVALID_ARG;
  if (M > 0 && (!aligned16(a) || !aligned16(w))) return MOEQ_ERR_INVALID_ARG;
  if (M == 0) return MOEQ_OK;
  if (int rc = check_device()) return rc;
  return launch_status(moeq::launch_shared_gemm_bf16(a, w, M, N, K, epilogue, out,
                                                     as_stream(stream)));
}

}  // extern "C"
