// fa_noalloc.hip -- fa_fwd_noalloc: the forward pass of fa_fwd_ws with the
// library's own fixed scratch buffer in place of a caller workspace, for
// callers that cannot allocate device memory around the call.
//
// The buffer is a file-scope device array: each device the library runs on
// holds one copy of it from the load of this library's device code until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host that name is a stand-in, not a device address): the first call on a
// device looks up that device's copy with hipGetSymbolAddress and every
// launch uses the address it returned.

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_kernel.h"

namespace {

constexpr size_t kScratchBytes = 64ull << 20;  // FA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "header and library agree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null: not looked up)

int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_noalloc(int dtype, const void* q, const void* k, const void* v, void* o,
                              float* lse, int B, int Sq, int Skv, int Hq, int Hkv, int D,
                              int causal, float scale, hipStream_t stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID;
  fa::LaunchArgs a;
  const int st = fa::check_fwd_args(dtype == FA_DTYPE_BF16 ? fa::DType::kBF16 : fa::DType::kF16,
                                    q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale,
                                    stream, &a);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  const int sst = scratch_for_current_device(&ws);
  if (sst != FA_OK) return sst;
  a.ws = ws;
  a.ws_bytes = kScratchBytes;
  // a split that needs more than the scratch holds is refused with
  // FA_ERR_WORKSPACE before anything is enqueued
  return fa::launch(a);
}
