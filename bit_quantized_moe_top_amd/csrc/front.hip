// moe_route_quant_permute: the layer's front end (routing, FP8 quantization of
// x, permutation plan and the copy of the routed rows into plan order) as one
// launch for small batches.
//
// At decode-sized T the separate launches are almost pure latency (a few
// microseconds each for a few kilobytes of work).  1024-thread workgroups do
// all of it in three phases separated by two barriers -- one workgroup per row
// when R = T k <= 64 (each routing every token and building the plan for
// itself), else one workgroup for all rows:
//   1. the waves of each row load their 8-element chunks of x into registers;
//      waves t < T route token t (expert ids into LDS); each wave then writes
//      the max |x| of its chunks to LDS;
//   2. the last wave builds the plan (R <= 64; the whole workgroup otherwise)
//      while the others turn their chunks into E4M3 codes, kept in registers
//      and written to x_q;
//   3. the codes go to the k plan positions of their token.
// The barriers order LDS only, so no wave waits for another's global stores.
// The arithmetic is the shared front.hpp code, so the results are bit-identical
// to the separate calls.
#include "front.hpp"

namespace moeq {

namespace {

constexpr int kFrontMaxRows = kFrontSmallT * MOEQ_MAX_TOPK;

constexpr int kFrontChunksPerThread = 4;    // 8-element chunks of x held per lane

// Waves quantizing each row: the rows share the waves equally; the last wave,
// which builds the plan, stays out when the others still cover every chunk of
// a row with kFrontChunksPerThread chunks per lane.  0: too large for one launch.
__host__ __device__ inline int front_waves_per_row(int T, int H) {
  if (T <= 0) return 1;
  const int cpr = H >> 3;
  const int cap = kWave * kFrontChunksPerThread;
  if (T < kPlanWaves && (kPlanWaves - 1) / T * cap >= cpr) return (kPlanWaves - 1) / T;
  const int wpr = kPlanWaves / T;
  return wpr * cap >= cpr ? wpr : 0;
}

// With R <= 64 the launch takes one workgroup per row (T > 1): each routes
// every token and builds the plan in LDS (the routing and the plan are a few
// microseconds of latency, the same in every workgroup), and quantizes and
// places only its own row, so the VALU work of the codes spreads over T CUs;
// workgroup 0 alone stores the routing and the plan.
__host__ __device__ inline bool front_per_row(int T, int k) { return T > 1 && T * k <= kWave; }

template <typename XT, int NS>
__global__ void __launch_bounds__(kPlanThreads)
front_small_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
                   int k, int renormalize, const XT* __restrict__ x, int H, int32_t* ids, float* w,
                   uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, int32_t* plan) {
  // plan LDS: R <= 64: E 64-bit row masks + E offsets; otherwise E * 17 ints
  extern __shared__ __align__(16) int smem[];
  __shared__ int s_ids[kFrontMaxRows];
  __shared__ int s_pos[kFrontMaxRows];
  __shared__ float s_part[kPlanWaves];        // per-wave max |x|
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // every kernel argument in one round of loads ahead of the first branch
  // (the compiler otherwise loads each behind the branch that first needs it)
  asm volatile("" ::"s"(logits), "s"(bias), "s"(x), "s"(ids), "s"(w), "s"(x_q), "s"(x_s),
               "s"(xp_q), "s"(xp_s), "s"(plan), "s"(E), "s"(k), "s"(renormalize), "s"(H),
               "s"(gridDim.x));
  const int R = T * k;
  const int cpr = H >> 3;                     // 8-element chunks per row
  // one row per workgroup (several workgroups), or all rows in one
  const bool per_row = gridDim.x > 1;
  const bool lead = blockIdx.x == 0;          // stores the routing and the plan
  const int wpr = front_waves_per_row(per_row ? 1 : T, H);
  int row, sub;
  if (per_row) {
    row = wave < wpr ? int(blockIdx.x) : T;
    sub = wave;
  } else {
    row = wave / wpr;
    sub = wave - row * wpr;
  }
  const int w0 = per_row ? 0 : row * wpr;     // first wave of the row
  const bool qrow = row < T;                  // this wave quantizes part of row `row`
  const auto chunk = [&](int i) { return (i * wpr + sub) * kWave + lane; };

  // ---- phase 1: chunk loads in flight, routing, per-wave max |x|.  Every
  // global load of the kernel is issued here, unconditionally (clamped
  // indices; lanes without a chunk drop theirs from the maximum), and every
  // global store comes after the last load is consumed: a wait for a load
  // also waits for the stores issued before it.
  XChunk<XT> xc[kFrontChunksPerThread];
  if (T > 0) {                                  // T = 0: x holds no row to read
    const int64_t xrow = min(row, T - 1);
#pragma unroll
    for (int i = 0; i < kFrontChunksPerThread; ++i)
      xc[i].load(x + xrow * H + min(chunk(i), cpr - 1) * 8);
  }
  const bool router = wave < T;                 // T <= kFrontSmallT <= kPlanWaves
  int my_e = 0;
  float my_w = 0.0f;
  if (router)
    my_e = route_token_values<NS>(logits + int64_t(wave) * E, bias, E, k, renormalize, lane, my_w);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kFrontChunksPerThread; ++i) {
    float v[8];
    xc[i].values(v);
    const bool mine = qrow && chunk(i) < cpr;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, mine ? fabsf(v[j]) : 0.0f);
  }
  amax = wave_max(amax);
  if (lane == 0) s_part[wave] = amax;
  if (router && lane < k) {
    if (lead) {
      ids[wave * k + lane] = my_e;
      w[wave * k + lane] = my_w;
    }
    s_ids[wave * k + lane] = my_e;
  }
  lds_barrier();

  // ---- phase 2: plan, and E4M3 codes of this thread's chunks.  The plan wave
  // runs at raised priority: it shares its SIMD with quantizing waves, and the
  // plan, not the codes, is what phase 3 waits for.
  if (R <= kWave && wave == kPlanWaves - 1) {
    __builtin_amdgcn_s_setprio(2);
    plan_build_wave<NS>(s_ids, T, k, E, plan, reinterpret_cast<unsigned long long*>(smem),
                        smem + 2 * E, s_pos, lane, lead);
    __builtin_amdgcn_s_setprio(0);
  }
  float scale = 0.0f;
  uint2 codes[kFrontChunksPerThread] = {};
  if (qrow) {
    float m = 0.0f;
    for (int i = 0; i < wpr; ++i) m = fmaxf(m, s_part[w0 + i]);
    scale = fp8_scale(m);
#pragma unroll
    for (int i = 0; i < kFrontChunksPerThread; ++i) {
      if (chunk(i) < cpr) {
        float v[8];
        xc[i].values(v);
        codes[i] = fp8_codes8(v, scale);
        *reinterpret_cast<uint2*>(x_q + int64_t(row) * H + chunk(i) * 8) = codes[i];
      }
    }
    if (sub == 0 && lane == 0) x_s[row] = scale;
  }
  if (R > kWave) {
    plan_build_workgroup([&](int r) { return s_ids[r]; }, T, k, E, plan, smem);
    __threadfence_block();
    __syncthreads();
    const PlanView pv = plan_view(plan, E, R);
    for (int r = tid; r < R; r += kPlanThreads) s_pos[r] = pv.row_pos[r];
  }
  lds_barrier();

  // ---- phase 3: codes and scale to the plan positions of the row's token
  if (qrow) {
    for (int j = 0; j < k; ++j) {
      const int p = s_pos[row * k + j];
      if (p < 0) continue;
#pragma unroll
      for (int i = 0; i < kFrontChunksPerThread; ++i)
        if (chunk(i) < cpr)
          *reinterpret_cast<uint2*>(xp_q + int64_t(p) * H + chunk(i) * 8) = codes[i];
      if (sub == 0 && lane == 0) xp_s[p] = scale;
    }
  }
}

template <typename XT, int NS>
hipError_t launch_small(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, const XT* x, int H, int32_t* ids, float* w,
                        uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, int32_t* plan,
                        hipStream_t stream) {
  const int R = T * k;
  const size_t lds = size_t(E) * (R <= kWave ? 3 : 1 + kPlanWaves) * sizeof(int);
  auto fn = front_small_kernel<XT, NS>;
  hipError_t err;
  if (lds > 64 * 1024 &&
      (err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds))) != hipSuccess)
    return err;
  hipLaunchKernelGGL(fn, dim3(front_per_row(T, k) ? unsigned(T) : 1u), dim3(kPlanThreads), lds,
                     stream, logits, bias, T, E, k, renormalize, x, H, ids, w, x_q, x_s, xp_q,
                     xp_s, plan);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_front(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, const void* x, int x_dtype, int H, int32_t* ids, float* w,
                        uint8_t* x_q, float* x_s, uint8_t* xp_q, float* xp_s, void* plan,
                        hipStream_t stream) {
  if (T > kFrontSmallT || front_waves_per_row(front_per_row(T, k) ? 1 : T, H) == 0) {
    // routing, then the plan, then x quantized once per token straight into
    // x_q and its k plan positions (rows of <= 4096 elements)
    hipError_t err;
    if ((err = launch_route_topk(logits, bias, T, E, k, renormalize, ids, w, stream)) != hipSuccess)
      return err;
    if (row_quant_cpl(H) != 0)
      return launch_permute_quant(ids, T, k, E, x, x_dtype, H, x_q, x_s, xp_q, xp_s, plan, stream);
    if ((err = launch_quant_fp8(x, x_dtype, T, H, H, x_q, x_s, stream)) != hipSuccess) return err;
    return launch_permute(ids, T, k, E, x_q, x_s, H, xp_q, xp_s, plan, stream);
  }
  int32_t* p = static_cast<int32_t*>(plan);
  return with_route_slots(E, [&](auto ns) {
    constexpr int NS = decltype(ns)::value;
    if (x_dtype == MOEQ_BF16)
      return launch_small<uint16_t, NS>(logits, bias, T, E, k, renormalize,
                                        static_cast<const uint16_t*>(x), H, ids, w, x_q, x_s,
                                        xp_q, xp_s, p, stream);
    return launch_small<float, NS>(logits, bias, T, E, k, renormalize,
                                   static_cast<const float*>(x), H, ids, w, x_q, x_s, xp_q, xp_s,
                                   p, stream);
  });
}

}  // namespace moeq
