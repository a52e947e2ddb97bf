// fa_combine.hip -- merges the per-key-range partial results of the split
// attention kernel into O and LSE.
//
// Key range s of a query row left O_s (normalised over its own keys, fp32)
// and LSE_s (natural log-sum-exp of its scaled logits; -inf when the range
// held no visible key).  The whole row's result is the online-softmax merge
// of those partial results (kernbench GQA prefill page, `_merge_running`),
// written with normalised parts:
//
//     LSE = m + ln sum_s exp(LSE_s - m),   m = max_s LSE_s
//     O   = sum_s exp(LSE_s - LSE) * O_s
//
// and a row with no visible key at all gets O = 0, LSE = -inf.  O is rounded
// once to the output dtype (round to nearest even).
//
// Half a wave (32 lanes) per query row, four head dimensions per lane
// (D = 128); the number of ranges is a template parameter so that every
// range's loads are issued before the first is used.

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kLanesPerRow = kD / 4;
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

__device__ inline void store4(__hip_bfloat16* p, const float (&a)[4]) {
  __hip_bfloat162 lo = __float22bfloat162_rn(make_float2(a[0], a[1]));
  __hip_bfloat162 hi = __float22bfloat162_rn(make_float2(a[2], a[3]));
  uint2 u;
  u.x = *reinterpret_cast<uint32_t*>(&lo);
  u.y = *reinterpret_cast<uint32_t*>(&hi);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ inline void store4(__half* p, const float (&a)[4]) {
  __half2 lo = __floats2half2_rn(a[0], a[1]);
  __half2 hi = __floats2half2_rn(a[2], a[3]);
  uint2 u;
  u.x = *reinterpret_cast<uint32_t*>(&lo);
  u.y = *reinterpret_cast<uint32_t*>(&hi);
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename T, int NS>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
               T* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Sq) {
  const int64_t rows = (int64_t)B * Hq * Sq;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  if (r >= rows) return;
  const int lane = threadIdx.x % kLanesPerRow;
  // row r = (b * Hq + hq) * Sq + i, the layout of the partial buffers
  const int i = (int)(r % Sq);
  const int64_t bh = r / Sq;
  const int hq = (int)(bh % Hq);
  const int b = (int)(bh / Hq);

  float ls[NS];
  float4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ls[s] = part_lse[(int64_t)s * rows + r];
    v[s] = *reinterpret_cast<const float4*>(part_o + ((int64_t)s * rows + r) * kD + 4 * lane);
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) m = fmaxf(m, ls[s]);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float w = expf(ls[s] - m);  // 0 for a range without keys
      wsum += w;
      acc[0] += w * v[s].x;
      acc[1] += w * v[s].y;
      acc[2] += w * v[s].z;
      acc[3] += w * v[s].w;
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] *= inv;
    out_lse = m + logf(wsum);
  }
  store4(o + (((int64_t)b * Sq + i) * Hq + hq) * kD + 4 * lane, acc);
  if (lse != nullptr && lane == 0) lse[r] = out_lse;
}

template <typename T>
hipError_t launch_t(const float* part_o, const float* part_lse, T* o, float* lse, int nsplit,
                    int B, int Hq, int Sq, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Hq * Sq;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(kThreads);
  const void* fn;
  switch (nsplit) {
    case 2: fn = reinterpret_cast<const void*>(&combine_kernel<T, 2>); break;
    case 4: fn = reinterpret_cast<const void*>(&combine_kernel<T, 4>); break;
    case 8: fn = reinterpret_cast<const void*>(&combine_kernel<T, 8>); break;
    case 16: fn = reinterpret_cast<const void*>(&combine_kernel<T, 16>); break;
    default: return hipErrorInvalidValue;
  }
  void* args[] = {&part_o, &part_lse, &o, &lse, &B, &Hq, &Sq};
  // the launch's own status (an unrelated earlier error is not reported)
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_combine(DType dtype, const float* part_o, const float* part_lse, void* o, float* lse,
                          int nsplit, int B, int Hq, int Sq, hipStream_t stream) {
  if (dtype == DType::kBF16)
    return launch_t(part_o, part_lse, static_cast<__hip_bfloat16*>(o), lse, nsplit, B, Hq, Sq, stream);
  return launch_t(part_o, part_lse, static_cast<__half*>(o), lse, nsplit, B, Hq, Sq, stream);
}

}  // namespace fa
