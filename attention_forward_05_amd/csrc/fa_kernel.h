// fa_kernel.h -- internal interface between the C-ABI entry points and the
// gfx950 kernel launcher (not installed, not part of the public ABI).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum class DType { kBF16, kF16 };

// Kernel shapes (the values of FA_KERNEL_* in fa.h).
enum Kernel : int { kFourWave = 0, kEightWave = 1, kTileRows = 2, kTileKeys = 3 };

// The launch plan for one call: kernel shape, key ranges per item, whether
// the q-heads of a kv-head are packed into one block of rows (tile kernels),
// and the bytes of partial results the split needs (0 without a split).
struct Plan {
  int kernel;
  int ranges;
  bool packed;
  size_t ws_bytes;
};

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
  // Device memory for the partial results of split key ranges, owned by the
  // caller (nullptr: never split).  The launch fails with FA_ERR_WORKSPACE
  // when the plan splits and ws_bytes is less than it needs.
  void* ws;
  size_t ws_bytes;
};

// (batch, q-head, 256-row query tile) items of these sizes; the persistent
// kernel runs min(items, compute units) workgroups over them.
int64_t work_items(int B, int Sq, int Hq);
// Query tiles of 256 rows and key tiles of 64 keys.
int query_tiles(int Sq);
// Whether the eight-wave kernel (512-row query tiles, D = 64 or 128) runs: when its
// items alone give each of the `cus` compute units one and every item with a
// visible key spans more than 128 keys.
bool use_eight_waves(int B, int Sq, int Skv, int Hq, int D, int causal, int cus);
int key_tiles(int Skv);
// Multiplier m with (hq * m) >> 20 == hq / (Hq / Hkv) for every hq < Hq,
// or false when no 32-bit product does it.
bool group_magic(int Hq, int Hkv, uint32_t* magic);

// Key tiles of the shortest 512-row item with a visible key (0: none).
int64_t min_item_tiles(int Sq, int Skv, int causal);
// log2 of the key ranges each 512-row item is split into (0: no split).
int split_log2(int B, int Sq, int Skv, int Hq, int D, int causal, int cus);
// Bytes of fp32 partial results (O and LSE) of `ranges` key ranges.
size_t split_ws_bytes(int B, int Sq, int Hq, int D, int ranges);
// The plan for these sizes on a device with `cus` compute units; with
// allow_split false (no workspace) key ranges are never split.
Plan make_plan(int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, int cus,
               bool allow_split);

// Enqueue the kernel(s) (loading the code object on first use on the current
// device); returns an fa_status (FA_OK, FA_ERR_WORKSPACE, FA_ERR_HIP).
int launch(const LaunchArgs& a);

// Merge the partial results of `nsplit` key ranges (O fp32
// [nsplit][B][Hq][Sq][D], LSE fp32 [nsplit][B][Hq][Sq]) into o (BSHD, the
// input dtype) and lse ([B][Hq][Sq], may be null); D = 64, 128 or 256.
hipError_t launch_combine(DType dtype, const float* part_o, const float* part_lse, void* o,
                          float* lse, int nsplit, int B, int Hq, int Sq, int D,
                          hipStream_t stream);

// Enqueue a tile kernel (fa_tile.hip): rows or keys split over its four
// waves, q-heads of a kv-head packed or not, `nsplit` key ranges per item
// (partial results to part_o / part_lse when nsplit > 1, else to o / lse).
hipError_t launch_tile(const LaunchArgs& a, bool keys, bool packed, int nsplit, float* part_o,
                       float* part_lse);

// The backward pass (fa_bwd.hip and the generated gradient kernels).
struct BwdLaunchArgs {
  DType dtype;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* ws;  // workspace: l2 = LSE * log2(e), then delta, each [B][Hq][Sq] fp32
  int B, Sq, Skv, Hq, Hkv, D, causal;
  float scale;
  float c;  // scale * log2(e), clamped to >= FLT_MIN
  hipStream_t stream;
};
// Enqueue the backward: the delta kernel (fa_bwd.hip), then the dK/dV and
// dQ kernels (generated, in the code object).  Returns an fa_status.
int launch_bwd(const BwdLaunchArgs& a);
// The delta kernel alone: l2 and delta of every query row into a.ws.
hipError_t launch_bwd_delta(const BwdLaunchArgs& a);
// The dK/dV and dQ kernels for D = 192 and 256 (fa_bwd_wide.hip), after the
// delta kernel.
hipError_t launch_bwd_wide(const BwdLaunchArgs& a);

// Argument checks shared by every forward entry point (no HIP call); on
// FA_OK fills `a` (everything but ws / ws_bytes).
int check_fwd_args(DType dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
                   hipStream_t stream, LaunchArgs* a);

}  // namespace fa
