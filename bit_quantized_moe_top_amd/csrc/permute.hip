// moe_permute kernels.
//
// plan_kernel -- a single 1024-thread workgroup builds the whole plan:
//   1. histogram of expert ids in LDS (integer atomics: the counts do not depend
//      on arrival order);
//   2. workgroup scans -> offsets[E+1], the active-expert list and the list of
//      MOEQ_TILE_M-row tiles;
//   3. a stable scatter: the rows are visited in chunks of 1024 (16 waves x 64
//      consecutive rows).  Inside a wave, lanes holding the same expert find each
//      other with ballots (one ballot per distinct expert, leader = lowest lane),
//      which gives each lane its rank among the equal lanes below it.  Per-wave
//      group sizes go to LDS; a per-expert pass turns them into bases in wave
//      order.  The position of row r is therefore
//        offsets[e] + (rows of e in earlier chunks) + (in earlier waves) + rank,
//      i.e. exactly its rank in increasing-r order: no dependence on scheduling.
// gather_kernel -- xp_q[p] = x_q[sorted_rows[p] / k] (16 B per thread), xp_s.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;

// exclusive scan over one value per thread of a 1024-thread workgroup; returns
// the exclusive prefix and writes the total to *total.  `tmp` holds 16 ints.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int wave_base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int c = tmp[w];
    if (w < wave) wave_base += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return wave_base + incl - v;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ plan) {
  extern __shared__ int smem[];
  int* cnt = smem;                        // [E]  counts, later running bases
  int* wcnt = smem + E;                   // [kPlanWaves][E] per-wave group sizes / bases
  __shared__ int scan_tmp[kPlanWaves];
  __shared__ int dropped;
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += kPlanThreads) cnt[e] = 0;
  if (tid == 0) dropped = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kPlanThreads) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else atomicAdd(&dropped, 1);
  }
  __syncthreads();

  // scans over experts (E <= 1024: one expert per thread)
  const int c = tid < E ? cnt[tid] : 0;
  int total_rows, n_active, n_tiles;
  const int off = block_exclusive_scan(c, scan_tmp, &total_rows);
  const int act = block_exclusive_scan(c > 0 ? 1 : 0, scan_tmp, &n_active);
  const int nt = (c + MOEQ_TILE_M - 1) / MOEQ_TILE_M;
  const int tile0 = block_exclusive_scan(nt, scan_tmp, &n_tiles);
  if (tid < E) {
    pv.offsets[tid] = off;
    if (c > 0) pv.active[act] = tid;
    for (int i = 0; i < nt; ++i) {
      pv.tile_expert[tile0 + i] = tid;
      pv.tile_row0[tile0 + i] = off + i * MOEQ_TILE_M;
    }
    cnt[tid] = off;                       // running base of expert tid
  }
  if (tid == 0) {
    pv.offsets[E] = total_rows;
    plan[kPlanR] = R;
    plan[kPlanE] = E;
    plan[kPlanActive] = n_active;
    plan[kPlanTiles] = n_tiles;
    plan[kPlanT] = T;
    plan[kPlanK] = k;
    plan[kPlanDropped] = dropped;
  }
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = 0; r0 < R; r0 += kPlanThreads) {
    for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcnt[i] = 0;
    __syncthreads();
    const int r = r0 + tid;
    int e = (r < R) ? ids[r] : -1;
    if (e >= E) e = -1;
    int rank = 0;
    uint64_t remaining = __ballot(e >= 0);
    while (remaining) {                   // one iteration per distinct expert in the wave
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int ev = __shfl(e, leader, kWave);
      const uint64_t same = __ballot(e == ev);
      if (e == ev) {
        rank = __popcll(same & below);
        if (lane == leader) wcnt[wave * E + e] = __popcll(same);
      }
      remaining &= ~same;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kPlanThreads) {
      int base = cnt[x];
      for (int w = 0; w < kPlanWaves; ++w) {
        const int g = wcnt[w * E + x];
        wcnt[w * E + x] = base;
        base += g;
      }
      cnt[x] = base;
    }
    __syncthreads();
    if (r < R) {
      if (e >= 0) {
        const int pos = wcnt[wave * E + e] + rank;
        pv.sorted_rows[pos] = r;
        pv.row_pos[r] = pos;
      } else {
        pv.row_pos[r] = -1;
      }
    }
    __syncthreads();
  }
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

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, const uint8_t* x_q,
                          const float* x_s, int H, uint8_t* xp_q, float* xp_s, void* plan,
                          hipStream_t stream) {
  const int R = T * k;
  const size_t lds = size_t(E) * (1 + kPlanWaves) * sizeof(int);
  if (lds > 64 * 1024) {
    const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&plan_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (a != hipSuccess) return a;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, stream, ids, T, k, E,
                     static_cast<int32_t*>(plan));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_q == nullptr || R == 0) return err;
  const int64_t threads = int64_t(R) * (H / 16);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, x_q, x_s, H, k,
                     static_cast<const int32_t*>(plan), E, R, xp_q, xp_s);
  return hipGetLastError();
}

}  // namespace moeq
