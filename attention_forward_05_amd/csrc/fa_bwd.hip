// fa_bwd.hip -- the first kernel of the attention backward pass on gfx950:
// per query row, delta = rowsum(O * dO) and l2 = LSE * log2(e), the two row
// statistics the gradient kernels read.
//
// The JAX Pallas FlashAttention3 page's backward, with the scale applied to
// the logits and its base-2 residual replaced by this library's natural-log
// LSE (p = exp2(c*q.k - l2), c = scale*log2(e)):
//   delta   = rowsum(O * dO)                          (`_attention_bwd`)
//   P       = exp2(c*S - l2),  dP = dO.V^T,  dS = P * (dP - delta)
//   dQ      = scale * dS.K                            (`kernel_dq`)
//   dK, dV  = scale * dS^T.Q,  P^T.dO, summed over the q-heads of a kv-head
//                                                     (`kernel_dkv`)
// The dK/dV and dQ kernels are generated gfx950 assembly
// (attention_forward_05_amd/asm/fa_bwd_gen.py) for D = 64 and 128, and HIP
// C++ (fa_bwd_wide.hip) for D = 192 and 256, launched from fa_launch.cpp
// after this one.  A row without a visible key (LSE = -inf) gets l2 = -inf;
// the causal mask hides every key from it, so its P is 0.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"
#include "fa_mfma.h"

namespace fa {

struct BwdArgs {
  const void* o;
  const void* dout;
  const float* lse;
  float* l2;     // [B][Hq][Sq]: LSE * log2(e)
  float* delta;  // [B][Hq][Sq]: rowsum(O * dO)
  int B, Sq, Hq;
};

namespace {

using namespace mfma;

// delta[(b*Hq + hq)*Sq + i] = sum_d O[b,i,hq,d] * dO[b,i,hq,d] in fp32 and
// l2[...] = LSE[...] * log2(e).  Rows are taken in memory order (b, i, hq),
// so a wave reads contiguous bytes; L lanes per row (a power of two) with E
// 16-byte chunks each, and each lane group takes kRowsPerGroup rows a
// block's width apart, their loads issued together.
constexpr int kRowsPerGroup = 4;

template <int D>
struct DeltaShape {
  static constexpr int kChunks = D / 8;                      // 16-byte chunks per row
  static constexpr int L = D == 192 ? 8 : kChunks;           // lanes per row
  static constexpr int E = kChunks / L;                      // chunks per lane
  static constexpr int G = 256 / L;                          // rows per pass of the block
  static_assert(L * E == kChunks && (L & (L - 1)) == 0, "lanes per row");
};

template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdArgs a) {
  using S = DeltaShape<D>;
  constexpr int L = S::L, E = S::E, G = S::G;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int lane = threadIdx.x % L;
  const int64_t r0 = (int64_t)blockIdx.x * G * kRowsPerGroup + threadIdx.x / L;
  s16x8 o8[kRowsPerGroup][E], d8[kRowsPerGroup][E];
#pragma unroll
  for (int u = 0; u < kRowsPerGroup; ++u) {
    const int64_t r = r0 + (int64_t)u * G;  // memory row (b, i, hq)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (r < rows) {
        const int64_t off = r * D + 8 * (lane * E + e);
        o8[u][e] = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.o) + off);
        d8[u][e] = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.dout) + off);
      } else {
        o8[u][e] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        d8[u][e] = o8[u][e];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerGroup; ++u) {
    const int64_t r = r0 + (int64_t)u * G;
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int x = 0; x < 8; ++x) acc += T::widen(o8[u][e][x]) * T::widen(d8[u][e][x]);
#pragma unroll
    for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (r < rows && lane == 0) {
      const int hq = (int)(r % a.Hq);
      const int64_t bi = r / a.Hq;
      const int i = (int)(bi % a.Sq);
      const int64_t b = bi / a.Sq;
      const int64_t s = (b * a.Hq + hq) * a.Sq + i;  // statistics row (b, hq, i)
      a.delta[s] = acc;
      a.l2[s] = a.lse[s] * kLog2e;
    }
  }
}

template <typename T, int D>
hipError_t launch_delta_d(const BwdArgs& in, hipStream_t stream) {
  BwdArgs a = in;
  void* args[] = {&a};
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int rows_per_block = DeltaShape<D>::G * kRowsPerGroup;
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_delta_kernel<T, D>),
                         dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(256),
                         args, 0, stream);
}

}  // namespace

hipError_t launch_bwd_delta(const BwdLaunchArgs& in) {
  BwdArgs a;
  a.o = in.o;
  a.dout = in.dout;
  a.lse = in.lse;
  a.l2 = in.ws;
  a.delta = in.ws + (size_t)in.B * in.Hq * in.Sq;
  a.B = in.B;
  a.Sq = in.Sq;
  a.Hq = in.Hq;
  const bool bf = in.dtype == DType::kBF16;
  if (in.D == 64) return bf ? launch_delta_d<BF16, 64>(a, in.stream) : launch_delta_d<F16, 64>(a, in.stream);
  if (in.D == 128) return bf ? launch_delta_d<BF16, 128>(a, in.stream) : launch_delta_d<F16, 128>(a, in.stream);
  if (in.D == 192) return bf ? launch_delta_d<BF16, 192>(a, in.stream) : launch_delta_d<F16, 192>(a, in.stream);
  if (in.D == 256) return bf ? launch_delta_d<BF16, 256>(a, in.stream) : launch_delta_d<F16, 256>(a, in.stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
