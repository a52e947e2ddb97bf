// fa_kernel.h -- internal interface between the C-ABI entry points and the
// gfx950 kernel (not installed, not part of the public ABI).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

enum class DType { kBF16, kF16 };

struct LaunchArgs {
  DType dtype;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be nullptr
  int B, Sq, Skv, Hq, Hkv, D, causal;
  float c;  // scale * log2(e), clamped to >= FLT_MIN
  hipStream_t stream;
};

// Number of workgroups the kernel launches for these sizes.
int64_t grid_blocks(int B, int Sq, int Hq);

// Enqueue the kernel; returns hipGetLastError() after the launch.
hipError_t launch(const LaunchArgs& a);

}  // namespace fa
