// fa_mfma.h -- device helpers shared by the HIP C++ kernels (fa_tile.hip,
// fa_bwd.hip): the gfx950 32x32x16 MFMA for bf16 and fp16 inputs, rounding
// to the input dtype, and the LDS tile layout with its transposing reads.
//
// v_mfma_f32_32x32x16 (64 lanes):
//   A (32x16): lane l holds A[l%32][8(l/32) .. 8(l/32)+7]
//   B (16x32): lane l holds B[8(l/32) .. +7][l%32]
//   C (32x32): lane l, register i holds C[8(i/4) + 4(l/32) + i%4][l%32]
// A C result whose rows are the contraction index of the next product is
// used directly as that product's B operand: the 16 rows of k-step t sit in
// lane half h as rows 16t + {4h..4h+3, 8+4h..8+4h+3} (registers 8t..8t+7);
// the other operand is read in the same row order (read_a_rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace mfma {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

struct BF16 {
  static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // round to nearest even
  static __device__ __forceinline__ short cvt(float x) {
    return __builtin_bit_cast(short, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float widen(short x) {
    return static_cast<float>(__builtin_bit_cast(__bf16, x));
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mma(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ short cvt(float x) {
    return __builtin_bit_cast(short, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float widen(short x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// LDS row pitch, in 16-bit elements, of a tile with rows of D elements:
// D itself, except D = 192, whose rows are padded to 256 so that the XOR
// swizzle below (of the low four chunk-index bits) keeps every chunk inside
// its row (chunks 0..23 map to 0..31).
template <int D>
constexpr int lds_pitch() {
  return D == 192 ? 256 : D;
}

// 16-byte chunk swizzle of an LDS tile with rows of D 16-bit elements.
// Row reads (16 consecutive rows at one chunk) and transposing reads (4
// consecutive rows x 4 consecutive chunks per 16 lanes) both hit distinct
// banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) return ((r >> 1) & 7) ^ (((r >> 1) & 1) << 2);
  else return (r & 15) ^ ((r & 3) << 2);
}
template <int D>
__device__ __forceinline__ int lds_off(int r, int chunk) {
  return r * (2 * lds_pitch<D>()) + ((chunk ^ swz<D>(r)) << 4);
}

// ds_read_b64_tr_b16 on a generic pointer into LDS: within each group of 16
// lanes, lane i receives element i of the four 16-element rows whose four
// 8-byte pieces lanes 4r..4r+3 address.
__device__ __forceinline__ s16x4 read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// A operand of k-step `ts` from an LDS tile X [rows][D] read transposed:
// A[m][k] = X[row0 + k'][col0 + m] for m = the lane's 32-column block index,
// with the k order of a C result used as B operand (rows 16ts + {4h..4h+3,
// 8+4h..8+4h+3}).  col0 is a multiple of 32.
template <int D>
__device__ __forceinline__ s16x8 read_a_rows(const char* tile, int row0, int ts, int col0,
                                             int lane) {
  const int h = lane >> 5;
  const int r = row0 + 16 * ts + 4 * h + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const s16x4 lo = read_tr(tile + lds_off<D>(r, col >> 3) + (col & 7) * 2);
  const s16x4 hi = read_tr(tile + lds_off<D>(r + 8, col >> 3) + (col & 7) * 2);
  return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// A operand (or B operand) of k-step t from an LDS tile X [rows][D] read by
// rows: lane l gets X[row0 + l%32][16t + 8(l/32) .. +7].
template <int D>
__device__ __forceinline__ s16x8 read_rows(const char* tile, int row0, int t, int lane) {
  return *reinterpret_cast<const s16x8*>(tile + lds_off<D>(row0 + (lane & 31), 2 * t + (lane >> 5)));
}

// Scheduling hints for the compiler: within the enclosing basic block,
// order a chain of N MFMAs whose operands come from N*R LDS reads so that
// the reads of the first AHEAD MFMAs are issued before the first MFMA and
// each MFMA is followed by the reads of a later one (the reads' latency then
// hides behind the MFMAs instead of stalling each one).  EXTRA more reads of
// the block (operands read before the chain) go first.
template <int N, int AHEAD, int GROUP, int R = 1, int EXTRA = 0>
__device__ __forceinline__ void sched_reads_ahead() {
  // masks of __builtin_amdgcn_sched_group_barrier: 0x008 MFMA, 0x100 DS read;
  // R reads per MFMA, AHEAD MFMAs' worth of reads issued first
  if constexpr (EXTRA > 0) __builtin_amdgcn_sched_group_barrier(0x100, EXTRA, GROUP);
#pragma unroll
  for (int i = 0; i < AHEAD && i < N; ++i) __builtin_amdgcn_sched_group_barrier(0x100, R, GROUP);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, GROUP);
    if (i + AHEAD < N) __builtin_amdgcn_sched_group_barrier(0x100, R, GROUP);
  }
}

// Registers 8t..8t+7 of a C result, rounded to the input dtype: the B operand
// of k-step t of the next product.
template <typename T>
__device__ __forceinline__ s16x8 pack_b(const f32x16& c, int t) {
  s16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = T::cvt(c[8 * t + e]);
  return r;
}

}  // namespace mfma
}  // namespace fa
