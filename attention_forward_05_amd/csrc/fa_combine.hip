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
// One 64-lane wave per query row, two head dimensions per lane (D = 128).

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerBlock = 4;

__device__ inline void store2(__hip_bfloat16* p, float a, float b) {
  p[0] = __float2bfloat16(a);
  p[1] = __float2bfloat16(b);
}
__device__ inline void store2(__half* p, float a, float b) {
  p[0] = __float2half(a);
  p[1] = __float2half(b);
}

template <typename T>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
               T* __restrict__ o, float* __restrict__ lse, int nsplit, int B, int Hq, int Sq) {
  const int64_t rows = (int64_t)B * Hq * Sq;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
  if (r >= rows) return;
  const int lane = threadIdx.x % 64;
  // row r = (b * Hq + hq) * Sq + i, the layout of the partial buffers
  const int i = (int)(r % Sq);
  const int64_t bh = r / Sq;
  const int hq = (int)(bh % Hq);
  const int b = (int)(bh / Hq);

  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_lse[(int64_t)s * rows + r]);
  float acc0 = 0.0f, acc1 = 0.0f, out_lse = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float ls = part_lse[(int64_t)s * rows + r];
      const float w = expf(ls - m);          // 0 for a range without keys
      wsum += w;
      const float2 v = *reinterpret_cast<const float2*>(part_o + ((int64_t)s * rows + r) * kD + 2 * lane);
      acc0 += w * v.x;
      acc1 += w * v.y;
    }
    const float inv = 1.0f / wsum;
    acc0 *= inv;
    acc1 *= inv;
    out_lse = m + logf(wsum);
  }
  store2(o + (((int64_t)b * Sq + i) * Hq + hq) * kD + 2 * lane, acc0, acc1);
  if (lse != nullptr && lane == 0) lse[r] = out_lse;
}

}  // namespace

hipError_t launch_combine(DType dtype, const float* part_o, const float* part_lse, void* o, float* lse,
                          int nsplit, int B, int Hq, int Sq, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Hq * Sq;
  const unsigned blocks = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == DType::kBF16) {
    hipLaunchKernelGGL(combine_kernel<__hip_bfloat16>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream,
                       part_o, part_lse, static_cast<__hip_bfloat16*>(o), lse, nsplit, B, Hq, Sq);
  } else {
    hipLaunchKernelGGL(combine_kernel<__half>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream,
                       part_o, part_lse, static_cast<__half*>(o), lse, nsplit, B, Hq, Sq);
  }
  return hipGetLastError();
}

}  // namespace fa
