// fa_kernel.h -- internal interface between the C-ABI entry points and the
// gfx950 kernel launcher (not installed, not part of the public ABI).
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

// (batch, q-head, 256-row query tile) items of these sizes; the persistent
// kernel runs min(items, compute units) workgroups over them.
int64_t work_items(int B, int Sq, int Hq);
// Query tiles of 256 rows and key tiles of 64 keys.
int query_tiles(int Sq);
// Whether the eight-wave kernel (512-row query tiles, D = 128) runs: when its
// items alone give each of the `cus` compute units one and every item with a
// visible key spans more than 128 keys.
bool use_eight_waves(int B, int Sq, int Skv, int Hq, int D, int causal, int cus);
int key_tiles(int Skv);
// Multiplier m with (hq * m) >> 20 == hq / (Hq / Hkv) for every hq < Hq,
// or false when no 32-bit product does it.
bool group_magic(int Hq, int Hkv, uint32_t* magic);

// Enqueue the kernel (loading the code object on first use on the current
// device); returns the launch status.
hipError_t launch(const LaunchArgs& a);

}  // namespace fa
