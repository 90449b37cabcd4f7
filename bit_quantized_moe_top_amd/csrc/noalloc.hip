// moe_expert_mlp_w4a8_noalloc: the routed experts' MLP for callers that cannot
// allocate device memory.  The intermediates of moe_expert_mlp_w4a8 (h, its
// E4M3 codes h_q and row scales h_s) live in `scratch`, a file-scope device
// array of kScratchBytes that each GPU holds from the library's first use on
// it until the process ends; the caller passes only inputs and the output o.
//
// The array's name is a host-side stand-in in host code: its device address on
// the current device comes from hipGetSymbolAddress, taken once per device on
// the entry point's first call there and kept; kernels only ever receive that
// address.  Every call on one GPU shares its array, so calls that overlap on a
// GPU (different streams, or host threads) race on it; calls on one stream are
// ordered.  Nothing here must start at zero: every byte a call reads from the
// array was written earlier by the same call.
#include <mutex>

#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;      // MOEQ_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MOEQ_NOALLOC_SCRATCH_BYTES, "header and library agree");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];        // device address of `scratch` per device (null: not yet)

// The current device's copy of `scratch`, or null if its address is unavailable.
void* scratch_ptr(int dev) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

namespace moeq {

size_t noalloc_mlp_bytes(int R, int I) {
  return align256(size_t(R) * I * 2) + align256(size_t(R) * I) + align256(size_t(R) * 4);
}

// Runs launch_expert_mlp with h, h_q, h_s carved from the current device's
// scratch array.  The caller has validated every argument and checked that
// noalloc_mlp_bytes(R, I) <= kScratchBytes.
hipError_t launch_expert_mlp_noalloc(int wfmt, const uint8_t* xp_q, const float* xp_s,
                                     const void* plan, int E, int R, const uint8_t* w13,
                                     const void* s13, const uint8_t* w2, const void* s2, int H,
                                     int I, uint16_t* o, hipStream_t stream) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint8_t* base = static_cast<uint8_t*>(scratch_ptr(dev));
  if (!base) return hipErrorInvalidSymbol;
  uint16_t* h = reinterpret_cast<uint16_t*>(base);
  uint8_t* h_q = base + align256(size_t(R) * I * 2);
  float* h_s = reinterpret_cast<float*>(h_q + align256(size_t(R) * I));
  return launch_expert_mlp(wfmt, xp_q, xp_s, plan, E, R, w13, s13, w2, s2, H, I, h, h_q, h_s, o,
                           stream);
}

}  // namespace moeq
