// moe_permute kernels: a stable counting sort of the routed rows by expert,
// then the gather of the quantized activations into that order.
//
// Row r = t*k + j sits, within its expert, at its rank among the rows of that
// expert with smaller r.  Ranks come from ballots inside a wave (wave_rank in
// front.hpp) and from per-wave / per-chunk counts combined in a fixed order, so
// the plan never depends on scheduling or atomic arrival order (integer
// histogram atomics only count).
//
// R <= 1024 routed rows: one 1024-thread workgroup builds the whole plan
//   (plan_build_workgroup), then gather_kernel copies the rows.
// Larger R, three kernels:
//   chunk_rank_kernel   one workgroup per chunk of 1024 rows: each row's rank
//                       inside its chunk (parked in row_pos) and the chunk's
//                       per-expert counts (plan scratch);
//   plan_scan_kernel    one workgroup: per-expert totals -> offsets, active list,
//                       tiles; per-chunk counts -> per-chunk bases;
//   place_kernel        position = chunk base + rank, written to sorted_rows /
//                       row_pos (place_gather_kernel: one workgroup per row,
//                       which also copies the row's activation bytes and scale).
#include "front.hpp"

namespace moeq {

namespace {

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ plan) {
  extern __shared__ int smem[];
  plan_build_workgroup([&](int r) { return ids[r]; }, T, k, E, plan, smem);
}

// one thread per 16-byte chunk of a destination row
__global__ void __launch_bounds__(256)
gather_kernel(const uint8_t* __restrict__ x_q, const float* __restrict__ x_s, int H, int k,
              const int32_t* __restrict__ plan, int E, int R, uint8_t* __restrict__ xp_q,
              float* __restrict__ xp_s) {
  const PlanView pv = plan_view(const_cast<int32_t*>(plan), E, R);
  const int chunks = H / 16;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int n_rows = pv.offsets[E];       // rows actually placed (R minus dropped ids)
  const int64_t p = idx / chunks;
  const int ch = int(idx - p * chunks);
  if (p >= n_rows) return;
  const int t = pv.sorted_rows[p] / k;
  const uint4 v = reinterpret_cast<const uint4*>(x_q + int64_t(t) * H)[ch];
  reinterpret_cast<uint4*>(xp_q + p * H)[ch] = v;
  if (ch == 0) xp_s[p] = x_s[t];
}

__global__ void __launch_bounds__(kPlanThreads)
chunk_rank_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ plan) {
  extern __shared__ int wcnt[];           // [kPlanWaves][E]
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcnt[i] = 0;
  __syncthreads();
  const int r = c * kPlanChunk + tid;
  int e = (r < R) ? ids[r] : -1;
  if (e >= E) e = -1;
  int gsize;
  const int rank = wave_rank(e, lane, &gsize);
  if (gsize > 0) wcnt[wave * E + e] = gsize;
  __syncthreads();
  for (int x = tid; x < E; x += kPlanThreads) {
    int base = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int g = wcnt[w * E + x];
      wcnt[w * E + x] = base;
      base += g;
    }
    pv.scratch[c * E + x] = base;
  }
  __syncthreads();
  if (r < R) pv.row_pos[r] = (e >= 0) ? wcnt[wave * E + e] + rank : -1;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_scan_kernel(int T, int k, int E, int32_t* __restrict__ plan) {
  extern __shared__ int cnt[];            // [E]
  __shared__ int scan_tmp[kPlanWaves];
  __shared__ int placed;
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int n_chunks = plan_chunks(R);
  const int tid = threadIdx.x;
  if (tid == 0) placed = 0;
  __syncthreads();
  // E <= kPlanThreads: thread x owns expert x.  Up to kRegChunks chunk counts
  // stay in registers, all loaded before any is used and none reloaded after
  // the base stores (a load issued after a store also waits for the store).
  constexpr int kRegChunks = 16;
  const bool in_regs = n_chunks <= kRegChunks;
  int nc[kRegChunks];
  if (tid < E) {
    int s = 0;
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) nc[c] = c < n_chunks ? pv.scratch[c * E + tid] : 0;
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) s += nc[c];
    } else {
      for (int c = 0; c < n_chunks; ++c) s += pv.scratch[c * E + tid];
    }
    cnt[tid] = s;
    atomicAdd(&placed, s);
  }
  __syncthreads();
  plan_finish_counts(cnt, scan_tmp, T, k, E, R - placed, plan);
  if (tid < E) {
    int base = cnt[tid];                  // offsets[tid]
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) {
        if (c < n_chunks) pv.scratch[c * E + tid] = base;
        base += nc[c];
      }
    } else {
      for (int c = 0; c < n_chunks; ++c) {
        const int n = pv.scratch[c * E + tid];
        pv.scratch[c * E + tid] = base;
        base += n;
      }
    }
  }
}

// position of routed row r: its chunk's base for its expert plus its rank in
// the chunk (parked in row_pos by chunk_rank_kernel); -1 for a dropped id
__device__ __forceinline__ int place_row(const int32_t* ids, int r, int E, PlanView& pv) {
  const int e = ids[r];
  if (e < 0 || e >= E) return -1;
  const int pos = pv.scratch[(r / kPlanChunk) * E + e] + pv.row_pos[r];
  pv.sorted_rows[pos] = r;
  pv.row_pos[r] = pos;
  return pos;
}

// plan only: one thread per routed row
__global__ void __launch_bounds__(256)
place_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ plan) {
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < R) place_row(ids, r, E, pv);
}

// with the gather: one workgroup per routed row, 16 bytes per thread per step
__global__ void __launch_bounds__(256)
place_gather_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                    int32_t* __restrict__ plan, const uint8_t* __restrict__ x_q,
                    const float* __restrict__ x_s, int H, uint8_t* __restrict__ xp_q,
                    float* __restrict__ xp_s) {
  __shared__ int s_pos;
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int r = blockIdx.x;
  if (threadIdx.x == 0) s_pos = place_row(ids, r, E, pv);
  __syncthreads();
  const int pos = s_pos;
  if (pos < 0) return;
  const int t = r / k;
  const uint4* src = reinterpret_cast<const uint4*>(x_q + int64_t(t) * H);
  uint4* dst = reinterpret_cast<uint4*>(xp_q + int64_t(pos) * H);
  for (int c = threadIdx.x; c < H / 16; c += 256) dst[c] = src[c];
  if (threadIdx.x == 0) xp_s[pos] = x_s[t];
}

// Quantization of x fused with the scatter (moe_route_quant_permute at larger
// T), for rows the quarter form below does not take: one wave per token
// quantizes its row in registers (RowQuant), writes the
// codes and scale to x_q / x_s and to the k plan positions of the token's
// rows.  kPlace: the positions are placed here (chunk base + rank, after
// chunk_rank_kernel and plan_scan_kernel); otherwise the plan is complete and
// row_pos is read.
template <typename XT, int CPL, bool kPlace>
__global__ void __launch_bounds__(256)
quant_scatter_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                     int32_t* __restrict__ plan, const XT* __restrict__ x, int H,
                     uint8_t* __restrict__ x_q, float* __restrict__ x_s,
                     uint8_t* __restrict__ xp_q, float* __restrict__ xp_s) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                   // wave-uniform
  PlanView pv = plan_view(plan, E, T * k);
  // x's loads first: place_row stores, and a load issued after a store also
  // waits for it
  RowQuant<XT, CPL> rq;
  rq.load(x + int64_t(t) * H, H, lane);
  int pos = -1;
  if (lane < k) pos = kPlace ? place_row(ids, t * k + lane, E, pv) : pv.row_pos[t * k + lane];
  rq.finish(H, lane);
  rq.store(x_q + int64_t(t) * H, H, lane);
  if (lane == 0) x_s[t] = rq.scale;
  for (int j = 0; j < k; ++j) {
    const int p = readlane(pos, j);
    if (p < 0) continue;
    rq.store(xp_q + int64_t(p) * H, H, lane);
    if (lane == 0) xp_s[p] = rq.scale;
  }
}

// The same with one 256-thread workgroup per token, each wave quantizing and
// scattering a quarter of the row (QuarterRowQuant): four times the waves, and
// their stores, in flight.  Wave 0 places (or reads) the k positions, after its
// loads are issued.
template <typename XT, int CPQ, bool kPlace>
__global__ void __launch_bounds__(256)
quant_scatter_quarter_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                             int32_t* __restrict__ plan, const XT* __restrict__ x, int H,
                             uint8_t* __restrict__ x_q, float* __restrict__ x_s,
                             uint8_t* __restrict__ xp_q, float* __restrict__ xp_s) {
  __shared__ float part[4];
  __shared__ int s_pos[MOEQ_MAX_TOPK];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x;
  PlanView pv = plan_view(plan, E, T * k);
  QuarterRowQuant<XT, CPQ> rq;
  rq.load(x + int64_t(t) * H, H, w, lane);
  if (w == 0 && lane < k)
    s_pos[lane] = kPlace ? place_row(ids, t * k + lane, E, pv) : pv.row_pos[t * k + lane];
  rq.finish(w, lane, part);               // its barrier also publishes s_pos
  rq.store(x_q + int64_t(t) * H, lane);
  if (threadIdx.x == 0) x_s[t] = rq.scale;
  for (int j = 0; j < k; ++j) {
    const int p = s_pos[j];
    if (p < 0) continue;
    rq.store(xp_q + int64_t(p) * H, lane);
    if (threadIdx.x == 0) xp_s[p] = rq.scale;
  }
}

hipError_t set_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, const uint8_t* x_q,
                          const float* x_s, int H, uint8_t* xp_q, float* xp_s, void* plan,
                          hipStream_t stream) {
  const int R = T * k;
  int32_t* p = static_cast<int32_t*>(plan);
  hipError_t err;
  if (R <= kPlanChunk) {
    const size_t lds = size_t(E) * (1 + kPlanWaves) * sizeof(int);
    if ((err = set_lds(reinterpret_cast<const void*>(&plan_kernel), lds)) != hipSuccess) return err;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, stream, ids, T, k, E, p);
    if ((err = hipGetLastError()) != hipSuccess || x_q == nullptr || R == 0) return err;
    const int64_t blocks = (int64_t(R) * (H / 16) + 255) / 256;
    hipLaunchKernelGGL(gather_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, x_q, x_s, H, k,
                       p, E, R, xp_q, xp_s);
    return hipGetLastError();
  }
  const size_t lds_rank = size_t(E) * kPlanWaves * sizeof(int);
  if ((err = set_lds(reinterpret_cast<const void*>(&chunk_rank_kernel), lds_rank)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(chunk_rank_kernel, dim3(plan_chunks(R)), dim3(kPlanThreads), lds_rank, stream,
                     ids, T, k, E, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kPlanThreads), size_t(E) * sizeof(int), stream,
                     T, k, E, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (x_q == nullptr)
    hipLaunchKernelGGL(place_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, ids, T, k, E, p);
  else
    hipLaunchKernelGGL(place_gather_kernel, dim3(R), dim3(256), 0, stream, ids, T, k, E, p, x_q, x_s,
                       H, xp_q, xp_s);
  return hipGetLastError();
}

hipError_t launch_permute_quant(const int32_t* ids, int T, int k, int E, const void* x,
                                int x_dtype, int H, uint8_t* x_q, float* x_s, uint8_t* xp_q,
                                float* xp_s, void* plan, hipStream_t stream) {
  if (row_quant_cpl(H) == 0) return hipErrorInvalidValue;
  const int R = T * k;
  int32_t* p = static_cast<int32_t*>(plan);
  hipError_t err;
  const bool place = R > kPlanChunk;
  if (!place) {
    const size_t lds = size_t(E) * (1 + kPlanWaves) * sizeof(int);
    if ((err = set_lds(reinterpret_cast<const void*>(&plan_kernel), lds)) != hipSuccess) return err;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, stream, ids, T, k, E, p);
  } else {
    const size_t lds_rank = size_t(E) * kPlanWaves * sizeof(int);
    if ((err = set_lds(reinterpret_cast<const void*>(&chunk_rank_kernel), lds_rank)) != hipSuccess)
      return err;
    hipLaunchKernelGGL(chunk_rank_kernel, dim3(plan_chunks(R)), dim3(kPlanThreads), lds_rank,
                       stream, ids, T, k, E, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kPlanThreads), size_t(E) * sizeof(int),
                       stream, T, k, E, p);
  }
  if ((err = hipGetLastError()) != hipSuccess || T == 0) return err;
  if (const int cpq = quarter_quant_cpq(H)) {
    auto go = [&](auto xt, auto cpq_tag) {
      using XT = typename decltype(xt)::type;
      constexpr int CPQ = decltype(cpq_tag)::value;
      const XT* xx = static_cast<const XT*>(x);
      if (place)
        hipLaunchKernelGGL((quant_scatter_quarter_kernel<XT, CPQ, true>), dim3(unsigned(T)),
                           dim3(256), 0, stream, ids, T, k, E, p, xx, H, x_q, x_s, xp_q, xp_s);
      else
        hipLaunchKernelGGL((quant_scatter_quarter_kernel<XT, CPQ, false>), dim3(unsigned(T)),
                           dim3(256), 0, stream, ids, T, k, E, p, xx, H, x_q, x_s, xp_q, xp_s);
      return hipGetLastError();
    };
    struct Bf16 { using type = uint16_t; };
    struct F32 { using type = float; };
    if (x_dtype == MOEQ_BF16)
      return cpq == 1 ? go(Bf16{}, SlotsTag<1>{}) : go(Bf16{}, SlotsTag<2>{});
    return cpq == 1 ? go(F32{}, SlotsTag<1>{}) : go(F32{}, SlotsTag<2>{});
  }
  const dim3 grid(unsigned((T + 3) / 4));
  return with_row_quant_cpl(H, [&](auto cpl) {
    constexpr int CPL = decltype(cpl)::value;
    if (x_dtype == MOEQ_BF16) {
      const uint16_t* xb = static_cast<const uint16_t*>(x);
      if (place)
        hipLaunchKernelGGL((quant_scatter_kernel<uint16_t, CPL, true>), grid, dim3(256), 0, stream,
                           ids, T, k, E, p, xb, H, x_q, x_s, xp_q, xp_s);
      else
        hipLaunchKernelGGL((quant_scatter_kernel<uint16_t, CPL, false>), grid, dim3(256), 0, stream,
                           ids, T, k, E, p, xb, H, x_q, x_s, xp_q, xp_s);
    } else {
      const float* xf = static_cast<const float*>(x);
      if (place)
        hipLaunchKernelGGL((quant_scatter_kernel<float, CPL, true>), grid, dim3(256), 0, stream,
                           ids, T, k, E, p, xf, H, x_q, x_s, xp_q, xp_s);
      else
        hipLaunchKernelGGL((quant_scatter_kernel<float, CPL, false>), grid, dim3(256), 0, stream,
                           ids, T, k, E, p, xf, H, x_q, x_s, xp_q, xp_s);
    }
    return hipGetLastError();
  });
}

}  // namespace moeq
