// Device routines of the layer's front end -- routing, per-row FP8 quantization
// and the permutation plan -- shared by the stand-alone kernels and the fused
// small-batch kernel, so that every path computes bit-identical results.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

template <int N>
struct SlotsTag { static constexpr int value = N; };

// ------------------------------------------------------------------ routing
// Scores are held in registers, NS per lane (expert e in lane e % 64, slot
// e / 64); NS = 64-expert slots covering E, rounded up to a power of two.
__host__ __device__ constexpr int route_slots_for(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
}

// Order-preserving 32-bit key of a score: a larger float gives a larger key
// (-0 is first made +0, so equal scores give equal keys).  Every float,
// -inf included, gets a key above 0, which marks "no candidate".
__device__ __forceinline__ uint32_t score_key(float v) {
  const uint32_t b = f2u(v + 0.0f);
  return b ^ ((b >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return u2f(k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

// The best candidate of the wave: the largest key, ties to the lowest expert
// index.  Returns the expert index (every lane); the rare tie takes a second
// reduction over the tied lanes' indices.
__device__ __forceinline__ int wave_best(uint32_t key, int idx, uint32_t* best_key) {
  const uint32_t kmax = static_cast<uint32_t>(
      wave_reduce(int(key), [](int a, int b) { return int(max(uint32_t(a), uint32_t(b))); }, 0));
  const uint64_t tied = __ballot(key == kmax);
  *best_key = kmax;
  if (__popcll(tied) == 1) return readlane(idx, __ffsll(static_cast<unsigned long long>(tied)) - 1);
  return wave_reduce(key == kmax ? idx : 0x7FFFFFFF, [](int a, int b) { return min(a, b); },
                     0x7FFFFFFF);
}

// One wave routes one token.  k rounds of a wave-wide argmax pick the experts
// best first; the order (score descending, expert index ascending) makes ties go
// to the lower index and the result independent of the reduction order.
// Returns the expert chosen in slot `lane` and its weight in w_out (valid for
// lane < k); nothing is stored.
template <int NS>
__device__ __forceinline__ int route_token_values(const float* row, const float* bias, int E,
                                                  int k, int renormalize, int lane, float& w_out) {
  // every load issued before the first use (clamped indices, no branch around
  // them), so the NS slots cost one memory latency, not NS in a row; the bias
  // is added only when given (adding 0 would turn -0 into +0)
  float s[NS], b[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) s[j] = row[min(j * kWave + lane, E - 1)];
  if (bias) {
#pragma unroll
    for (int j = 0; j < NS; ++j) b[j] = bias[min(j * kWave + lane, E - 1)];
#pragma unroll
    for (int j = 0; j < NS; ++j) s[j] = s[j] + b[j];
  }
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (j * kWave + lane >= E) s[j] = -INFINITY;
  uint32_t key[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) key[j] = (j * kWave + lane < E) ? score_key(s[j]) : 0u;
  float sel_v[MOEQ_MAX_TOPK];
  int sel_e[MOEQ_MAX_TOPK];
#pragma unroll
  for (int r = 0; r < MOEQ_MAX_TOPK; ++r) {
    sel_v[r] = -INFINITY;
    sel_e[r] = 0;
    if (r >= k) continue;
    // this lane's best remaining slot (the lower slot, i.e. expert, on ties)
    uint32_t ck = 0;
    int ci = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (key[j] > ck) { ck = key[j]; ci = j * kWave + lane; }
    uint32_t bk;
    const int bi = wave_best(ck, ci, &bk);
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (j == (bi >> 6)) key[j] = 0u;              // taken
    }
    sel_v[r] = key_score(bk);
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
    for (int j = 0; j < NS; ++j)
      if (j * kWave + lane < E) part += expf(s[j] - smax);
    den = wave_sum(part);
  }
  float v = sel_v[0];
  int e = sel_e[0];
#pragma unroll
  for (int r = 1; r < MOEQ_MAX_TOPK; ++r)
    if (r == lane) { v = sel_v[r]; e = sel_e[r]; }
  w_out = expf(v - smax) / den;
  return e;
}

// route_token_values, with lanes j < k writing slot j to ids_row and w_row.
template <int NS>
__device__ __forceinline__ int route_token_wave(const float* row, const float* bias, int E, int k,
                                                int renormalize, int32_t* ids_row, float* w_row,
                                                int lane) {
  float wt;
  const int e = route_token_values<NS>(row, bias, E, k, renormalize, lane, wt);
  if (lane < k) {
    ids_row[lane] = e;
    w_row[lane] = wt;
  }
  return e;
}

// Calls fn(SlotsTag<NS>{}) with NS = route_slots_for(E).
template <typename F>
__host__ __forceinline__ auto with_route_slots(int E, F&& fn) {
  switch (route_slots_for(E)) {
    case 1: return fn(SlotsTag<1>{});
    case 2: return fn(SlotsTag<2>{});
    case 4: return fn(SlotsTag<4>{});
    case 8: return fn(SlotsTag<8>{});
    default: return fn(SlotsTag<16>{});
  }
}

// ------------------------------------------------------- FP8 quantization
// 8 consecutive elements (16 B of bf16 or 32 B of fp32) -> fp32
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  bf16x8_to_f32(*reinterpret_cast<const uint4*>(p), v);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// 8 consecutive elements of x held in registers as loaded (bf16 or fp32)
template <typename XT>
struct XChunk;
template <>
struct XChunk<uint16_t> {
  uint4 raw;
  __device__ __forceinline__ void load(const uint16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void values(float (&v)[8]) const { bf16x8_to_f32(raw, v); }
};
template <>
struct XChunk<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void values(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// A row of x quantized by one wave with the row held in registers: lane l
// takes the 8-element chunks l, l + 64, ... (CPL of them; K <= 512 CPL).
// The codes stay in `codes` for the caller to store wherever they go.
template <typename XT, int CPL>
struct RowQuant {
  XChunk<XT> xc[CPL];
  uint2 codes[CPL];
  float scale;
  __device__ __forceinline__ void run(const XT* row, int K, int lane) {
    load(row, K, lane);
    finish(K, lane);
  }
  // the row's loads (to be issued ahead of other memory work)
  __device__ __forceinline__ void load(const XT* row, int K, int lane) {
    const int chunks = K >> 3;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + kWave * i < chunks) xc[i].load(row + (lane + kWave * i) * 8);
  }
  // max |x|, the scale and the codes of the loaded row
  __device__ __forceinline__ void finish(int K, int lane) {
    const int chunks = K >> 3;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (lane + kWave * i < chunks) {
        float v[8];
        xc[i].values(v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      }
    }
    scale = fp8_scale(wave_max(amax));
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (lane + kWave * i < chunks) {
        float v[8];
        xc[i].values(v);
        codes[i] = fp8_codes8(v, scale);
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* q_row, int K, int lane) const {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + kWave * i < (K >> 3))
        *reinterpret_cast<uint2*>(q_row + (lane + kWave * i) * 8) = codes[i];
  }
};

// A row quantized by the four waves of a 256-thread workgroup: wave q takes the
// quarter [q K/4, (q + 1) K/4) (K % 32 == 0, K/4 <= 512 CPQ), lane l its 8-element
// chunks l, l + 64, ...; the four waves' partial maxima meet in LDS at one
// barrier.  The maximum of the partial maxima is the row maximum, so the scale
// and codes equal RowQuant's; a row's work is spread over four waves, which
// keeps four times as many of them, and their loads and stores, in flight.
template <typename XT, int CPQ>
struct QuarterRowQuant {
  XChunk<XT> xc[CPQ];
  uint2 codes[CPQ];
  float scale;
  int c0, chunks;          // the quarter's first element and its 8-element chunks
  __device__ __forceinline__ void load(const XT* row, int K, int q, int lane) {
    const int qlen = K >> 2;
    c0 = q * qlen;
    chunks = qlen >> 3;
#pragma unroll
    for (int i = 0; i < CPQ; ++i)
      if (lane + kWave * i < chunks) xc[i].load(row + c0 + (lane + kWave * i) * 8);
  }
  // called by every thread of the workgroup (one barrier); part: 4 floats of LDS
  __device__ __forceinline__ void finish(int q, int lane, float* part) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPQ; ++i) {
      if (lane + kWave * i < chunks) {
        float v[8];
        xc[i].values(v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) part[q] = amax;
    __syncthreads();
    scale = fp8_scale(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])));
#pragma unroll
    for (int i = 0; i < CPQ; ++i) {
      if (lane + kWave * i < chunks) {
        float v[8];
        xc[i].values(v);
        codes[i] = fp8_codes8(v, scale);
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* q_row, int lane) const {
#pragma unroll
    for (int i = 0; i < CPQ; ++i)
      if (lane + kWave * i < chunks)
        *reinterpret_cast<uint2*>(q_row + c0 + (lane + kWave * i) * 8) = codes[i];
  }
};

// 8-element chunks per lane of a quarter row (QuarterRowQuant), 0 where rows of K
// take RowQuant instead: the quarters need K % 32 == 0, and for K below 1024 a
// quarter leaves most lanes of its wave idle.  (Used where each row is stored
// k + 1 times, the quantization fused with the scatter: there the four waves'
// stores in flight pay -- 35.1 against 36.9 us for the T = 2048 front end --
// while the plain quantization of h, one store per row, ran slower this way:
// 23.9 against 20.4 us for 12288 rows of 2048.)
__host__ __device__ inline int quarter_quant_cpq(int K) {
  if (K % 32 != 0 || K < 1024) return 0;
  const int c = (K / 4 + 8 * kWave - 1) / (8 * kWave);
  return c <= 1 ? 1 : c <= 2 ? 2 : 0;
}

// chunks per lane for a row of K elements held by one wave (0: K too large)
__host__ __device__ inline int row_quant_cpl(int K) {
  const int c = (K + 8 * kWave - 1) / (8 * kWave);
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 0;
}
template <typename F>
__host__ inline hipError_t with_row_quant_cpl(int K, F&& fn) {
  switch (row_quant_cpl(K)) {
    case 1: return fn(SlotsTag<1>{});
    case 2: return fn(SlotsTag<2>{});
    case 4: return fn(SlotsTag<4>{});
    case 8: return fn(SlotsTag<8>{});
    default: return hipErrorInvalidValue;
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

// Workgroup barrier that orders LDS accesses only (no wait for global stores).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS accesses: the LDS unit serves one wave's operations in
// issue order, so a wavefront-scope fence (a compiler barrier, no wait) makes
// every lane's earlier LDS writes visible to the wave's later reads.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The whole plan for R = T k <= 64 routed rows, built by one wave.  Every
// routed row sets its bit (1 << r) in its expert's 64-bit LDS mask (atomic
// OR, so arrival order does not matter); a row's rank within its expert is the
// number of mask bits below it (stable order), an expert's count the mask's
// population.  Wave scans over the experts (lane x % 64, pass x / 64) give the
// offsets, and ballots the active list.  With at most 64 rows every active
// expert owns exactly one tile.  The result equals plan_build_workgroup's.
// NS: passes of 64 experts covering E.  s_mask: E 64-bit words of LDS, s_off:
// E ints of LDS; s_pos[r] receives row_pos[r].  With write_plan false the plan
// is only computed (s_pos), not stored.
template <int NS>
__device__ __forceinline__ void plan_build_wave(const int* s_ids, int T, int k, int E,
                                                int32_t* plan, unsigned long long* s_mask,
                                                int* s_off, int* s_pos, int lane,
                                                bool write_plan = true) {
  const int R = T * k;
  PlanView pv = plan_view(plan, E, R);
  const int e = lane < R ? s_ids[lane] : -1;
  const bool valid = lane < R && e >= 0 && e < E;
  const int dropped = __popcll(__ballot(lane < R && !valid));
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (lane + j * kWave < E) s_mask[lane + j * kWave] = 0ull;
  lds_wave_sync();
  if (valid) atomicOr(&s_mask[e], 1ull << lane);
  lds_wave_sync();

  // all NS mask reads first, then the NS scans (independent of each other,
  // so their cross-lane steps interleave), then the running carries: one LDS
  // round trip instead of one per pass
  int c[NS], incl[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int x = lane + j * kWave;
    c[j] = x < E ? __popcll(s_mask[x]) : 0;
  }
  const uint64_t mine = valid ? s_mask[e] : 0ull;   // this row's expert's rows
#pragma unroll
  for (int j = 0; j < NS; ++j) incl[j] = wave_inclusive_scan(c[j]);
  int carry = 0, act_carry = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int x = lane + j * kWave;
    const int off = carry + incl[j] - c[j];
    carry += readlane(incl[j], kWave - 1);
    const uint64_t nz = __ballot(c[j] > 0);
    if (x < E) {
      if (write_plan) pv.offsets[x] = off;
      s_off[x] = off;
    }
    if (c[j] > 0 && write_plan) {
      const int a = act_carry + __popcll(nz & ((1ull << lane) - 1ull));
      pv.active[a] = x;
      pv.tile_expert[a] = x;
      pv.tile_row0[a] = off;
    }
    act_carry += __popcll(nz);
  }
  if (lane == 0 && write_plan) {
    pv.offsets[E] = carry;
    plan[kPlanR] = R;
    plan[kPlanE] = E;
    plan[kPlanActive] = act_carry;
    plan[kPlanTiles] = act_carry;
    plan[kPlanT] = T;
    plan[kPlanK] = k;
    plan[kPlanDropped] = dropped;
  }
  if (lane > kPlanDropped && lane < kPlanHeader && write_plan) plan[lane] = 0;
  lds_wave_sync();
  if (lane < R) {
    int p = -1;
    if (valid) {
      p = s_off[e] + __popcll(mine & ((1ull << lane) - 1ull));
      if (write_plan) pv.sorted_rows[p] = lane;
    }
    if (write_plan) pv.row_pos[lane] = p;
    s_pos[lane] = p;
  }
}

}  // namespace moeq
