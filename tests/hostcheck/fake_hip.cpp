// Stand-in for the HIP runtime entry points that libtpmlp's host code calls
// (test infrastructure, CPU only): kernel registration, the launch sequence
// the compiler emits for a triple-chevron launch, and the few API calls the
// library makes.  Launches are handed to the bounds model instead of a GPU.
#include <hip/hip_runtime_api.h>

#include <map>
#include <mutex>
#include <string>

#include "model.hpp"

namespace {

std::map<const void *, std::string> &functions() {
  static std::map<const void *, std::string> m;
  return m;
}

struct CallConfig {
  dim3 grid, block;
  size_t shmem;
  hipStream_t stream;
};
thread_local CallConfig g_cfg;
thread_local hipError_t g_last = hipSuccess;
int g_module_handle;

}  // namespace

extern "C" {

void **__hipRegisterFatBinary(const void *) { return (void **)&g_module_handle; }

void __hipUnregisterFatBinary(void **) {}

void __hipRegisterFunction(void **, const void *hostFunction, char *, const char *deviceName,
                           unsigned int, uint3 *, uint3 *, dim3 *, dim3 *, int *) {
  functions()[hostFunction] = deviceName;
}

void __hipRegisterVar(void **, void *var, char *, char *deviceVar, int, size_t size, int, int) {
  hostcheck::register_symbol(var, size, deviceVar);
}

}  // extern "C"

hipError_t __hipPushCallConfiguration(dim3 gridDim, dim3 blockDim, size_t sharedMem,
                                      hipStream_t stream) {
  g_cfg = CallConfig{gridDim, blockDim, sharedMem, stream};
  return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3 *gridDim, dim3 *blockDim, size_t *sharedMem,
                                     hipStream_t *stream) {
  *gridDim = g_cfg.grid;
  *blockDim = g_cfg.block;
  *sharedMem = g_cfg.shmem;
  *stream = g_cfg.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void *function_address, dim3 numBlocks, dim3 dimBlocks,
                           void **args, size_t, hipStream_t) {
  auto it = functions().find(function_address);
  if (it == functions().end()) {
    g_last = hipErrorInvalidDeviceFunction;
    return g_last;
  }
  if (numBlocks.x == 0 || numBlocks.y == 0 || numBlocks.z == 0 || dimBlocks.x == 0 ||
      dimBlocks.x * dimBlocks.y * dimBlocks.z > 1024) {
    g_last = hipErrorInvalidConfiguration;
    return g_last;
  }
  hostcheck::on_launch(it->second.c_str(), numBlocks.x, numBlocks.y, numBlocks.z, dimBlocks.x,
                       dimBlocks.y, dimBlocks.z, args);
  return hipSuccess;
}

hipError_t hipGetLastError(void) {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}

const char *hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "error (host model)";
}

hipError_t hipGetDevice(int *deviceId) {
  *deviceId = 0;
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void **devPtr, const void *symbol) {
  *devPtr = hostcheck::symbol_address(symbol);
  return *devPtr ? hipSuccess : hipErrorInvalidSymbol;
}
