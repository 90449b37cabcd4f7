// pack_int4_g128 kernel.  16 consecutive lanes own one 128-wide group: each lane
// loads 8 consecutive fp32 weights (32 B), the group's max |w| is reduced over
// the 16 lanes, s = max/7 (IEEE division), codes = clamp(rne(w / s), -8, 7), and
// each lane stores its 8 codes as one little-endian 32-bit word of nibbles
// (code + 8, first code in the least significant nibble).  With bfloat16
// scales the stored scale is bf16(max/7) (RNE) and the codes are taken
// against that stored value.  tile_int4_kernel moves packed rows into the
// GEMMs' tiled order.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

template <typename ST>
__global__ void __launch_bounds__(256)
pack_int4_kernel(const float* __restrict__ w, int64_t n_groups, int groups_per_row,
                 uint32_t* __restrict__ packed, ST* __restrict__ scales) {
  const int64_t gid = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool valid = gid < n_groups;
  float v[8];
  float amax = 0.0f;
  if (valid) {
    // group gid covers w[gid*128 .. gid*128+127] (rows are contiguous, K = 128*groups_per_row)
    const float4* p = reinterpret_cast<const float4*>(w + gid * 128 + sub * 8);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  if (!valid) return;
  float s = __fdiv_rn(amax, 7.0f);
  ST stored;
  if constexpr (sizeof(ST) == 2) {
    stored = f32_to_bf16(s);
    s = bf16_to_f32(stored);
  } else {
    stored = s;
  }
  uint32_t word = 0x88888888u;           // all-zero codes
  if (s > 0.0f) {
    word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = rintf(__fdiv_rn(v[i], s));
      c = fminf(fmaxf(c, -8.0f), 7.0f);
      word |= uint32_t(int(c) + 8) << (4 * i);
    }
  }
  packed[gid * 16 + sub] = word;
  if (sub == 0) scales[gid] = stored;
  (void)groups_per_row;
}

// Packed rows [rows][K/2] -> the tiled order [rows/16][K/128][16][64] (16-row
// blocks stored group after group).  One thread per 16 output bytes, numbered in
// output order u: piece c = u % 4 of row r = (u / 4) % 16 of group
// g = (u / 64) % G of block b = u / (64 G), read from row 16 b + r, bytes
// 64 g + 16 c.  Grid-stride over u.
__global__ void __launch_bounds__(256)
tile_int4_kernel(const uint4* __restrict__ in, int64_t units, int G, uint4* __restrict__ out) {
  const int64_t row_units = int64_t(G) * 4;                 // 16-byte pieces per row
  for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * 256) {
    const int c = int(u & 3), r = int((u >> 2) & 15);
    const int64_t bg = u >> 6;                               // block * G + group
    const int64_t b = bg / G, g = bg - b * G;
    out[u] = in[(16 * b + r) * row_units + 4 * g + c];
  }
}

}  // namespace

hipError_t launch_tile_int4(const uint8_t* packed, int64_t rows, int K, uint8_t* tiled,
                            hipStream_t stream) {
  const int64_t units = rows * (K / 32);
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 255) / 256;
  const unsigned grid = unsigned(blocks < 65536 * 16 ? blocks : 65536 * 16);
  hipLaunchKernelGGL(tile_int4_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(packed), units, K / 128,
                     reinterpret_cast<uint4*>(tiled));
  return hipGetLastError();
}

template <typename ST>
hipError_t launch_pack(const float* w, int64_t rows, int K, uint8_t* packed, ST* scales,
                       hipStream_t stream) {
  const int64_t n_groups = rows * (K / 128);
  if (n_groups == 0) return hipSuccess;
  const int64_t kMaxGrid = 0x7FFFFFFF;
  for (int64_t g0 = 0; g0 < n_groups; g0 += kMaxGrid * 16) {
    const int64_t ng = (n_groups - g0 < kMaxGrid * 16) ? (n_groups - g0) : kMaxGrid * 16;
    hipLaunchKernelGGL(pack_int4_kernel<ST>, dim3(unsigned((ng + 15) / 16)), dim3(256), 0, stream,
                       w + g0 * 128, ng, K / 128, reinterpret_cast<uint32_t*>(packed + g0 * 64),
                       scales + g0);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_pack_int4(const float* w, int64_t rows, int K, uint8_t* packed, void* scales,
                            int bf16_scales, hipStream_t stream) {
  if (bf16_scales)
    return launch_pack(w, rows, K, packed, static_cast<uint16_t*>(scales), stream);
  return launch_pack(w, rows, K, packed, static_cast<float*>(scales), stream);
}

}  // namespace moeq
