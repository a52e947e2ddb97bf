// fa_combine.hip -- merges the per-key-range partial results of split
// attention kernels into O and LSE.
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
// D/4 lanes per query row, four head dimensions per lane; the ranges are
// visited in groups of eight whose loads are all issued before the first is
// used.

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 8;  // ranges whose loads are issued together

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

template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
               T* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Sq, int ns) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerBlock = kThreads / kLanesPerRow;
  const int64_t rows = (int64_t)B * Hq * Sq;
  if ((int)threadIdx.x >= kRowsPerBlock * kLanesPerRow) return;  // D = 192: 5 rows of 48 lanes
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  if (r >= rows) return;
  const int lane = threadIdx.x % kLanesPerRow;
  // row r = (b * Hq + hq) * Sq + i, the layout of the partial buffers
  const int i = (int)(r % Sq);
  const int64_t bh = r / Sq;
  const int hq = (int)(bh % Hq);
  const int b = (int)(bh / Hq);

  float m = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += kGroup) {
    float ls[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      ls[j] = (s0 + j < ns) ? part_lse[(int64_t)(s0 + j) * rows + r] : -INFINITY;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) m = fmaxf(m, ls[j]);
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += kGroup) {
      float ls[kGroup];
      float4 v[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const bool ok = s0 + j < ns;
        ls[j] = ok ? part_lse[(int64_t)(s0 + j) * rows + r] : -INFINITY;
        v[j] = ok ? *reinterpret_cast<const float4*>(part_o + ((int64_t)(s0 + j) * rows + r) * D +
                                                     4 * lane)
                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const float w = expf(ls[j] - m);  // 0 for a range without keys
        wsum += w;
        acc[0] += w * v[j].x;
        acc[1] += w * v[j].y;
        acc[2] += w * v[j].z;
        acc[3] += w * v[j].w;
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] *= inv;
    out_lse = m + logf(wsum);
  }
  store4(o + (((int64_t)b * Sq + i) * Hq + hq) * D + 4 * lane, acc);
  if (lse != nullptr && lane == 0) lse[r] = out_lse;
}

template <typename T, int D>
hipError_t launch_d(const float* part_o, const float* part_lse, T* o, float* lse, int nsplit,
                    int B, int Hq, int Sq, hipStream_t stream) {
  constexpr int kRowsPerBlock = kThreads / (D / 4);
  const int64_t rows = (int64_t)B * Hq * Sq;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  void* args[] = {&part_o, &part_lse, &o, &lse, &B, &Hq, &Sq, &nsplit};
  // the launch's own status (an unrelated earlier error is not reported)
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel<T, D>), grid,
                         dim3(kThreads), args, 0, stream);
}

template <typename T>
hipError_t launch_t(const float* part_o, const float* part_lse, T* o, float* lse, int nsplit,
                    int B, int Hq, int Sq, int D, hipStream_t stream) {
  if (nsplit < 1) return hipErrorInvalidValue;
  switch (D) {
    case 64: return launch_d<T, 64>(part_o, part_lse, o, lse, nsplit, B, Hq, Sq, stream);
    case 128: return launch_d<T, 128>(part_o, part_lse, o, lse, nsplit, B, Hq, Sq, stream);
    case 192: return launch_d<T, 192>(part_o, part_lse, o, lse, nsplit, B, Hq, Sq, stream);
    case 256: return launch_d<T, 256>(part_o, part_lse, o, lse, nsplit, B, Hq, Sq, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_combine(DType dtype, const float* part_o, const float* part_lse, void* o, float* lse,
                          int nsplit, int B, int Hq, int Sq, int D, hipStream_t stream) {
  if (dtype == DType::kBF16)
    return launch_t(part_o, part_lse, static_cast<__hip_bfloat16*>(o), lse, nsplit, B, Hq, Sq, D,
                    stream);
  return launch_t(part_o, part_lse, static_cast<__half*>(o), lse, nsplit, B, Hq, Sq, D, stream);
}

}  // namespace fa
