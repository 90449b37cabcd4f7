// Streaming-read measurement kernel (not a step of the layer): reads a buffer
// the way a well-fed stream does -- 16 bytes per lane, consecutive lanes on
// consecutive addresses, kInFlight independent loads per thread per step,
// grid-stride over the buffer, each load non-temporal like the grouped GEMMs'
// streamed weight loads -- and stores the XOR of everything it read, one word
// per wave, so the loads cannot be dropped.  Its bytes per second are the
// device's practical HBM read ceiling against which the grouped GEMMs' weight
// streams are measured.
#include "common.hpp"
#include "kernels.hpp"

namespace moeq {

namespace {

constexpr int kInFlight = 16;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ void __launch_bounds__(256)
read_probe_kernel(const uint4* __restrict__ p, int64_t n, uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  uint32_t acc = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride * kInFlight) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = (i + u * stride < n) ? load_nt(p + i + u * stride) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(MOEQ_READ_PROBE_BLOCKS), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moeq
