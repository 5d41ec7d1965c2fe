// Library-owned scratch memory for the entry point that allocates nothing
// (tp_mlp_shard_noalloc): a file-scope device array per GPU, in the same
// layout as a caller's workspace (the few-token path's arrival counters in the
// first kWsCounterBytes, split-K partials after them).
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address.  The address is looked up once per device with
// hipGetSymbolAddress (with that device current) and cached; kernels only
// ever receive that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace tpmlp {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_dev[kMaxDevices];

// Zero the counter area (one thread per 16 bytes).
__global__ void zero_counters(uint4 *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t static_scratch(hipStream_t stream, void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch &d = g_dev[dev];
  std::call_once(d.once, [&] {
    void *p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err != hipSuccess) return;
    // The counters must start at zero; every later call leaves them zero.  A
    // fill kernel (not a memset) keeps this first call capturable.
    const int64_t n = (int64_t)(kWsCounterBytes / 16);
    hipLaunchKernelGGL(zero_counters, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (uint4 *)p, n);
    d.err = hipGetLastError();
    if (d.err == hipSuccess) d.ptr = p;
  });
  if (d.err != hipSuccess) return d.err;
  *ptr = d.ptr;
  return hipSuccess;
}

}  // namespace tpmlp
