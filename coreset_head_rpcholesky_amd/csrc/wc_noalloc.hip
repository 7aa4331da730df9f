// wc_forward for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation): the workspace is a device array of
// this library, `scratch`, of kScratchBytes bytes, instead of a buffer the caller passes.
//
// Each device that runs this code holds its own copy of the array (at its own address) from
// the load of this library's code on that device until the process ends.  Its address is
// taken once per device with hipGetSymbolAddress, with that device current, and only that
// address reaches the kernels: in host code `scratch` names a host-side stand-in, not device
// memory.  Every call on one device shares that device's array: calls that overlap on one
// device (two streams, or two host threads) race on it and must be ordered by the caller.
// Nothing in the forward reads workspace it has not written in the same call, so the contents
// a previous call left behind need no clearing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/wc.h"
#include "wc_host.h"

namespace {

constexpr size_t kScratchBytes = WC_NOALLOC_MAX_WORKSPACE;  // per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" {

wc_status wc_forward_noalloc(const wc_problem* p, const void* Q, const void* K, const void* V,
                             const float* u_forced, uint64_t seed, void* O, int32_t* pivots,
                             int32_t* rank, uint32_t* flags, void* stream) {
  wc_status st = wc::forward_check(p, Q, K, V, u_forced, O, pivots, rank, flags);
  if (st != WC_OK || p->heads == 0) return st;
  size_t need = 0;
  if ((st = wc_workspace_bytes(p, &need)) != WC_OK) return st;
  if (need > kScratchBytes) return WC_ERR_WORKSPACE;  // above the fixed maximum
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WC_ERR_DEVICE;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    void* ptr = nullptr;
    d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    d.ptr = d.err == hipSuccess ? ptr : nullptr;
  });
  if (d.err != hipSuccess || d.ptr == nullptr) return WC_ERR_DEVICE;
  return wc_forward(p, Q, K, V, u_forced, seed, O, pivots, rank, flags, d.ptr, kScratchBytes, stream);
}

}  // extern "C"
