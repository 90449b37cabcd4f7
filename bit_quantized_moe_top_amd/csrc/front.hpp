// Device routines of the layer's front end -- routing, per-row FP8 quantization
// and the permutation plan -- shared by the stand-alone kernels and the fused
// small-batch kernel, so that every path computes bit-identical results.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

// ------------------------------------------------------------------ routing
constexpr int kRouteSlots = MOEQ_MAX_EXPERTS / kWave;   // scores held per lane

__device__ __forceinline__ bool route_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// wave-wide best (score, expert) pair, in every lane (DPP steps as wave_reduce)
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp<CTRL, ROW_MASK>(v, v);
  const int oi = dpp<CTRL, ROW_MASK>(i, i);
  if (route_better(ov, oi, v, i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppQuadSwap1>(v, i);
  argmax_step<kDppQuadSwap2>(v, i);
  argmax_step<kDppRowHalfMirror>(v, i);
  argmax_step<kDppRowMirror>(v, i);
  argmax_step<kDppRowBcast15, 0xA>(v, i);
  argmax_step<kDppRowBcast31, 0xC>(v, i);
  v = readlane(v, 63);
  i = readlane(i, 63);
}

// One wave routes one token.  Expert e's score lives in lane e % 64, slot e / 64.
// k rounds of a wave-wide argmax pick the experts best first; the order (score
// descending, expert index ascending) makes ties go to the lower index and the
// result independent of the reduction order.  Lanes j < k write slot j.
// Returns the expert chosen in slot `lane` (valid for lane < k).
__device__ __forceinline__ int route_token_wave(const float* row, const float* bias, int E, int k,
                                                int renormalize, int32_t* ids_row, float* w_row,
                                                int lane) {
  float s[kRouteSlots];
#pragma unroll
  for (int j = 0; j < kRouteSlots; ++j) {
    const int e = j * kWave + lane;
    float v = -INFINITY;
    if (e < E) {
      v = row[e];
      if (bias) v = v + bias[e];
    }
    s[j] = v;
  }
  uint32_t used = 0;                                    // slots already selected (bit j)
  float sel_v[MOEQ_MAX_TOPK];
  int sel_e[MOEQ_MAX_TOPK];
#pragma unroll
  for (int r = 0; r < MOEQ_MAX_TOPK; ++r) {
    sel_v[r] = -INFINITY;
    sel_e[r] = 0;
    if (r >= k) continue;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kRouteSlots; ++j) {
      const int e = j * kWave + lane;
      if (e < E && !((used >> j) & 1u) && route_better(s[j], e, bv, bi)) { bv = s[j]; bi = e; }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
    sel_v[r] = bv;
    sel_e[r] = bi;
  }
  const float smax = sel_v[0];
  float den = 0.0f;
  if (renormalize) {
#pragma unroll
    for (int r = 0; r < MOEQ_MAX_TOPK; ++r)
      if (r < k) den += expf(sel_v[r] - smax);
  } else {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kRouteSlots; ++j)
      if (j * kWave + lane < E) part += expf(s[j] - smax);
    den = wave_sum(part);
  }
  float v = sel_v[0];
  int e = sel_e[0];
#pragma unroll
  for (int r = 1; r < MOEQ_MAX_TOPK; ++r)
    if (r == lane) { v = sel_v[r]; e = sel_e[r]; }
  if (lane < k) {
    ids_row[lane] = e;
    w_row[lane] = expf(v - smax) / den;
  }
  return e;
}

// ------------------------------------------------------- FP8 quantization
// 8 consecutive elements (16 B of bf16 or 32 B of fp32) -> fp32
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = u2f(w[i] << 16);
    v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// scale = fp32(amax / 448) (IEEE division); 8 codes of x / scale (IEEE
// division, E4M3 round-to-nearest-even, saturating) packed little-endian
__device__ __forceinline__ float fp8_scale(float amax) { return __fdiv_rn(amax, 448.0f); }
__device__ __forceinline__ uint2 fp8_codes8(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
  if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_e4m3(__fdiv_rn(v[i], s)) << (8 * i);
      hi |= f32_to_e4m3(__fdiv_rn(v[4 + i], s)) << (8 * i);
    }
  }
  return make_uint2(lo, hi);
}

// One wave quantizes one row of K elements (K % 8 == 0).
template <typename T>
__device__ __forceinline__ void quant_row_wave(const T* row, int K, uint8_t* qrow, float* scale,
                                               int lane) {
  float amax = 0.0f;
  for (int c = lane * 8; c < K; c += kWave * 8) {
    float v[8];
    load8(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  const float s = fp8_scale(amax);
  if (lane == 0) *scale = s;
  for (int c = lane * 8; c < K; c += kWave * 8) {
    float v[8];
    load8(row + c, v);
    *reinterpret_cast<uint2*>(qrow + c) = fp8_codes8(v, s);
  }
}

// A 1024-thread workgroup quantizes T <= 16 rows: each row gets 16 / T waves
// (its 8-element chunks strided over them), whose partial max|x| meet in LDS.
template <typename T>
__device__ __forceinline__ void quant_rows_workgroup(const T* x, int rows, int K, uint8_t* q,
                                                     float* scale, float* s_part /* 16 floats */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wpr = rows > 0 ? 16 / rows : 16;
  const int row = wave / wpr, sub = wave - row * wpr;
  const bool active = row < rows;
  const T* xr = x + int64_t(active ? row : 0) * K;
  const int step = wpr * kWave * 8;
  float amax = 0.0f;
  if (active) {
    for (int c = (sub * kWave + lane) * 8; c < K; c += step) {
      float v[8];
      load8(xr + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) s_part[wave] = amax;
  __syncthreads();
  if (active) {
    float m = 0.0f;
    for (int w = 0; w < wpr; ++w) m = fmaxf(m, s_part[row * wpr + w]);
    const float s = fp8_scale(m);
    if (sub == 0 && lane == 0) scale[row] = s;
    uint8_t* qr = q + int64_t(row) * K;
    for (int c = (sub * kWave + lane) * 8; c < K; c += step) {
      float v[8];
      load8(xr + c, v);
      *reinterpret_cast<uint2*>(qr + c) = fp8_codes8(v, s);
    }
  }
}

// ---------------------------------------------------------- plan building
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanChunk = kPlanThreads;                // rows ranked per pass

// exclusive scan of one value per thread of a 1024-thread workgroup; writes the
// total to *total.  `tmp` holds kPlanWaves ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
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

// Rank of each lane's expert among the lanes below it holding the same expert
// (e < 0: no expert).  One ballot per distinct expert in the wave, leader =
// lowest lane, so the result does not depend on scheduling.  The leader of each
// group also gets the group size.
__device__ __forceinline__ int wave_rank(int e, int lane, int* group_size) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  *group_size = 0;
  uint64_t remaining = __ballot(e >= 0);
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int ev = readlane(e, leader);
    const uint64_t same = __ballot(e == ev);
    if (e == ev) {
      rank = __popcll(same & below);
      if (lane == leader) *group_size = __popcll(same);
    }
    remaining &= ~same;
  }
  return rank;
}

// Writes offsets, the active list, the tile list and the header from per-expert
// counts cnt[E] (LDS).  Leaves cnt[e] = offsets[e].  1024 threads, E <= 1024.
__device__ __forceinline__ void plan_finish_counts(int* cnt, int* scan_tmp, int T, int k, int E,
                                                   int dropped, int32_t* plan) {
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int tid = threadIdx.x;
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
    cnt[tid] = off;
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
    for (int i = kPlanDropped + 1; i < kPlanHeader; ++i) plan[i] = 0;
  }
  __syncthreads();
}

// The whole plan in one 1024-thread workgroup.  ids(r) returns the expert of
// routed row r.  smem: E * (1 + kPlanWaves) ints of LDS.
template <typename IdsF>
__device__ __forceinline__ void plan_build_workgroup(IdsF ids, int T, int k, int E, int32_t* plan,
                                                     int* smem) {
  int* cnt = smem;                        // [E]  counts, then running bases
  int* wcnt = smem + E;                   // [kPlanWaves][E] per-wave group sizes -> bases
  __shared__ int scan_tmp[kPlanWaves];
  __shared__ int dropped;
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += kPlanThreads) cnt[e] = 0;
  if (tid == 0) dropped = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kPlanThreads) {
    const int e = ids(r);
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else atomicAdd(&dropped, 1);
  }
  __syncthreads();
  plan_finish_counts(cnt, scan_tmp, T, k, E, dropped, plan);

  for (int r0 = 0; r0 < R; r0 += kPlanChunk) {
    for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcnt[i] = 0;
    __syncthreads();
    const int r = r0 + tid;
    int e = (r < R) ? ids(r) : -1;
    if (e >= E) e = -1;
    int gsize;
    const int rank = wave_rank(e, lane, &gsize);
    if (gsize > 0) wcnt[wave * E + e] = gsize;
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

}  // namespace moeq
