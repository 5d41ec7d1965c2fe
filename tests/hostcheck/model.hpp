// Host-side bounds model of libtpmlp's kernel launches (test infrastructure).
//
// The library's host code is linked against a stand-in for the HIP runtime
// (fake_hip.cpp) instead of the real one: every kernel launch arrives here
// with its grid, block and arguments, and no GPU is touched.  The caller
// registers the byte ranges of the "device" buffers it passes to the C ABI
// (fake addresses that are never dereferenced); the model then computes, with
// the kernels' own addressing code where it is shared, every address a launch
// would touch and checks that it lies inside the buffer its operand points
// into.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace hostcheck {

// A fake device buffer of `bytes` bytes; returns its base address.
void *fake_alloc(size_t bytes, const char *name);
void reset();  // forget every buffer, launch and finding

struct Stats {
  long launches = 0;       // every kernel launch
  long tiled = 0;          // tiled GEMM launches checked lane by lane
  long decode = 0;         // few-token GEMM launches checked lane by lane
  long checked_other = 0;  // other launches whose extents were checked
  long accesses = 0;       // address ranges checked
  std::vector<std::string> findings;  // violations (first few per launch)
  std::vector<std::string> kernels;   // names of the kernels launched, in order
};
Stats &stats();

// Called by the stand-in runtime for every launch.
void on_launch(const char *name, unsigned gx, unsigned gy, unsigned gz, unsigned bx, unsigned by,
               unsigned bz, void **args);

// A fake address for a registered device variable of `bytes` bytes.
void *symbol_address(const void *host_var);
void register_symbol(const void *host_var, size_t bytes, const char *name);

}  // namespace hostcheck
