// fa_kernel.hip -- the fused attention forward kernel for gfx950 (MI355X).
//
// One workgroup owns BM = 256 query rows of one (batch, q-head) and sweeps the
// visible keys in tiles of BN = 64.  Four waves of 64 lanes each own 64 of
// the rows.  Per key tile a wave computes
//
//     S^T = K . Q^T          (MFMA 32x32x16, fp32 accumulate)
//     online softmax of S    (running max m, running sum l, exp2 with the
//                             scale * log2(e) constant folded into one FMA)
//     O^T += V^T . P^T       (MFMA 32x32x16, P rounded to the input dtype)
//
// which is the loop body of the JAX Pallas FlashAttention3 page (`kv_loop`:
// max, alpha = exp2(m_old - m_new), p = exp2(s*log2e - m), acc *= alpha,
// l = l*alpha + sum p, acc += p.V) and of the Croqtile `flash_atten` page
// (the same recurrence with the logit scale folded into the exp2 exponent).
//
// gfx950 layout choices (not taken from the pages, which target other GPUs):
//
// * Transposed products.  With S^T = K.Q^T the 32x32 MFMA accumulator puts
//   one query per lane column: lane l holds query (l % 32) and 16 of the 32
//   keys of a block, the other 16 sit in lane l ^ 32.  Row max and row sum
//   are therefore in-lane plus a single exchange with lane l ^ 32, and the
//   rescale by alpha is one per-lane scalar for the whole O^T column.
// * The S^T accumulator, rounded to bf16/fp16, *is* the B operand of the
//   O^T = V^T.P^T product once the keys of that product are enumerated in the
//   accumulator's row order, so P never goes through LDS.  V is stored
//   transposed in LDS (V^T rows of 64 keys) in that same key order, so each
//   A operand of the second product is one 16-byte LDS read.
// * Q stays in VGPRs for the whole sweep (it is the B operand of S^T = K.Q^T).
// * K and V^T tiles are double-buffered in LDS; the next tile's global loads
//   are in flight while the current tile is computed, one barrier per tile.
//   16-byte chunks are XOR-swizzled so the MFMA operand reads of 16
//   consecutive lanes fall in distinct banks.
// * Causal: key tiles wholly above the diagonal are never loaded; a wave
//   skips tiles that are fully masked for its 64 rows and applies the mask
//   only on tiles that cross its diagonal or the Skv tail.  The grid runs the
//   longest (last) query tiles first, and places all tiles of a (batch,
//   head group) on one XCD so they share that XCD's L2.
//
// MFMA 32x32x16 lane layouts used (gfx9 matrix-core convention):
//   A (32 x 16): lane l holds row (l % 32), k = 8*(l / 32) + j, j = 0..7
//   B (16 x 32): lane l holds column (l % 32), k = 8*(l / 32) + j
//   C (32 x 32): lane l holds column (l % 32), register i holds row
//                8*(i / 4) + 4*(l / 32) + (i % 4), i = 0..15

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernel.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 64;            // query rows per wave (two 32-row MFMA blocks)
constexpr int kBM = kWaves * kQW;  // query rows per workgroup
constexpr int kBN = 64;            // keys per tile

// ---------------------------------------------------------------------------
// dtype traits: the MFMA for the dtype and fp32 -> dtype rounding (RNE)
// ---------------------------------------------------------------------------
template <typename T> struct Dt;

template <> struct Dt<__bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // eight fp32 -> eight bf16 (v_cvt_pk_bf16_f32, round to nearest even)
  static __device__ __forceinline__ v8 cvt8(const float* x) {
    v8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
    return r;
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <> struct Dt<_Float16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v8 cvt8(const float* x) {
    v8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
    return r;
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
};

// ---------------------------------------------------------------------------
// geometry per head dimension
// ---------------------------------------------------------------------------
template <int D> struct Geo {
  static constexpr int kSteps = D / 16;          // k-steps of S^T = K.Q^T
  static constexpr int kDBlk = D / 32;           // 32-row blocks of O^T
  static constexpr int kKRow = D * 2;            // bytes of one K row in LDS
  static constexpr int kKTile = kBN * kKRow;     // bytes of a K tile
  static constexpr int kVRow = kBN * 2;          // bytes of one V^T row (64 keys)
  static constexpr int kVTile = D * kVRow;       // bytes of a V^T tile
  static constexpr int kStage = kKTile + kVTile; // one LDS buffer
  // K staging: 16-byte chunks per thread per tile
  static constexpr int kKChunks = kBN * D / 8 / kThreads;  // 4 (D=128) / 2 (D=64)
  static constexpr int kKChunksPerRow = D / 8;
  // V staging: each thread reads 8 keys x (D/32) dims
  static constexpr int kVDims = D / 32;          // 4 / 2
};

// XOR swizzle of the 16-byte chunk index of K row r.  D = 128: rows are 256
// bytes (16 chunks), 16 consecutive rows map a given chunk to 16 distinct
// chunks.  D = 64: rows are 128 bytes (8 chunks); pairs of rows share an XOR
// value and fall in the two halves of a 256-byte bank sweep.
template <int D> __device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// XOR swizzle of the 16-byte chunk index of V^T row d (8 chunks of 128 bytes).
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Value of the lane l ^ 32 (the other half of the same query's keys).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Keys of the 16-byte V^T chunk g (0..7) within a 64-key tile, element j
// (0..7).  Chunk g = 4*kb + 2*th + h feeds k-step (kb, th) of the second
// product for lanes of half h; its keys are the accumulator rows that those
// lanes hold in registers 8*th .. 8*th+7 of S^T block kb.
__device__ __forceinline__ int vchunk_key(int g, int j) {
  return 16 * (g >> 1) + 4 * (g & 1) + 8 * (j >> 2) + (j & 3);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int B, int Sq, int Skv, int Hq,
    int Hkv, int causal, float c /* scale*log2(e), > 0 */, int nq,
    int pairs_per_xcd) {
  typedef Dt<T> dt;
  typedef typename dt::v8 v8;
  typedef Geo<D> G;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * G::kStage];

  // ---- which (query tile, batch, head) this workgroup owns ---------------
  const int bid = blockIdx.x;
  const int npairs = B * Hq;
  int qt, pair;
  if (pairs_per_xcd > 0) {
    // Workgroups are handed to the 8 XCDs round-robin; keep every tile of a
    // contiguous run of (batch, head) pairs on one XCD.
    const int x = bid & 7, s = bid >> 3;
    qt = s / pairs_per_xcd;
    pair = x * pairs_per_xcd + s % pairs_per_xcd;
  } else {
    qt = bid / npairs;
    pair = bid % npairs;
  }
  const int qtile = causal ? nq - 1 - qt : qt;  // longest causal tiles first
  const int b = pair / Hq, hq = pair % Hq;
  const int hk = hq / (Hq / Hkv);
  const int off = Skv - Sq;  // bottom-right alignment of the causal mask

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int q0 = qtile * kBM;
  const int qw0 = q0 + w * kQW;

  // ---- key range of the workgroup and of this wave ------------------------
  const int q_last_blk = min(q0 + kBM, Sq) - 1;
  const int kv_end_blk = causal ? min(Skv, q_last_blk + off + 1) : Skv;
  const int n_tiles = kv_end_blk > 0 ? (kv_end_blk + kBN - 1) / kBN : 0;

  const bool wave_active = qw0 < Sq;
  const int q_last_w = min(qw0 + kQW, Sq) - 1;
  const int kv_end_w = causal ? min(Skv, q_last_w + off + 1) : Skv;
  // keys below kv_full_w are visible to every row of the wave
  const int kv_full_w = causal ? min(Skv, qw0 + off + 1) : Skv;

  const int64_t q_row_stride = (int64_t)Hq * D;
  const int64_t kv_row_stride = (int64_t)Hkv * D;
  const T* Kbh = K + (int64_t)b * Skv * kv_row_stride + (int64_t)hk * D;
  const T* Vbh = V + (int64_t)b * Skv * kv_row_stride + (int64_t)hk * D;

  // ---- Q block in registers: B operand of S^T = K.Q^T ---------------------
  // qreg[qb][s] = Q[q][16 s + 8 h .. +8] for q = qw0 + 32 qb + l32
  v8 qreg[2][G::kSteps];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + 32 * qb + l32;
    if (q < Sq) {
      const T* p = Q + ((int64_t)b * Sq + q) * q_row_stride + (int64_t)hq * D + 8 * h;
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s)
        qreg[qb][s] = __builtin_bit_cast(v8, *(const uint4*)(p + 16 * s));
    } else {
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s)
        qreg[qb][s] = __builtin_bit_cast(v8, make_uint4(0, 0, 0, 0));
    }
  }

  // ---- staging of one K / V tile through registers -----------------------
  // K: thread loads kKChunks 16-byte chunks; chunk kc = tid % chunks-per-row
  // of rows tid / chunks-per-row + p * (threads / chunks-per-row).
  constexpr int kRowsPerPass = kThreads / G::kKChunksPerRow;
  const int kc = tid % G::kKChunksPerRow;
  const int kr0 = tid / G::kKChunksPerRow;
  // V: thread reads chunk group vg = tid / 32 (8 keys) at dims vd0 .. vd0+kVDims
  const int vg = tid >> 5;
  const int vd0 = (tid & 31) * G::kVDims;

  uint4 kst[G::kKChunks];
  typedef typename std::conditional<G::kVDims == 4, uint2, uint32_t>::type vword;
  vword vst[8];

  auto stage_load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < G::kKChunks; ++p) {
      const int key = k0 + kr0 + p * kRowsPerPass;
      if (key < Skv)
        kst[p] = *(const uint4*)(Kbh + (int64_t)key * kv_row_stride + 8 * kc);
      else
        kst[p] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = k0 + vchunk_key(vg, j);
      if (key < Skv)
        vst[j] = *(const vword*)(Vbh + (int64_t)key * kv_row_stride + vd0);
      else
        vst[j] = vword{};
    }
  };

  auto stage_store = [&](unsigned char* buf) {
    unsigned char* Ks = buf;
    unsigned char* Vs = buf + G::kKTile;
#pragma unroll
    for (int p = 0; p < G::kKChunks; ++p) {
      const int r = kr0 + p * kRowsPerPass;
      *(uint4*)(Ks + r * G::kKRow + ((kc ^ k_swz<D>(r)) << 4)) = kst[p];
    }
    // transpose 8 keys x kVDims dims into kVDims V^T rows of 8 keys
#pragma unroll
    for (int dd = 0; dd < G::kVDims; ++dd) {
      uint32_t e[8];  // element dd of each of the 8 keys, in the low 16 bits
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t word;
        if constexpr (G::kVDims == 4)
          word = (dd < 2) ? vst[j].x : vst[j].y;
        else
          word = vst[j];
        e[j] = (dd & 1) ? (word >> 16) : (word & 0xffffu);
      }
      uint4 out;
      out.x = e[0] | (e[1] << 16);
      out.y = e[2] | (e[3] << 16);
      out.z = e[4] | (e[5] << 16);
      out.w = e[6] | (e[7] << 16);
      const int d = vd0 + dd;
      *(uint4*)(Vs + d * G::kVRow + ((vg ^ v_swz(d)) << 4)) = out;
    }
  };

  // ---- running state ------------------------------------------------------
  f32x16 oacc[2][G::kDBlk];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < G::kDBlk; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.0f;
  float m_run[2] = {-INFINITY, -INFINITY};  // raw-logit running max
  float l_run[2] = {0.0f, 0.0f};            // this lane's half of the row sum

  if (n_tiles > 0) {
    stage_load(0);
    stage_store(smem);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * kBN;
    if (t + 1 < n_tiles) stage_load(k0 + kBN);

    unsigned char* Ks = smem + (t & 1) * G::kStage;
    unsigned char* Vs = Ks + G::kKTile;

    if (wave_active && k0 < kv_end_w) {
      // ---- S^T = K . Q^T ---------------------------------------------------
      f32x16 sacc[2][2];  // [kb][qb]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][qb][i] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + l32;
        const unsigned char* krow = Ks + r * G::kKRow;
        const int sw = k_swz<D>(r);
#pragma unroll
        for (int s = 0; s < G::kSteps; ++s) {
          v8 a = __builtin_bit_cast(v8, *(const uint4*)(krow + (((2 * s + h) ^ sw) << 4)));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = dt::mfma(a, qreg[qb][s], sacc[kb][qb]);
        }
      }

      // ---- mask (only tiles crossing the wave's diagonal or the tail) ------
      if (k0 + kBN > kv_full_w) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int q = qw0 + 32 * qb + l32;
          const int lim = causal ? min(Skv - 1, q + off) : Skv - 1;  // last visible key
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
              if (key > lim) sacc[kb][qb][i] = -INFINITY;
            }
        }
      }

      // ---- online softmax ----------------------------------------------------
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = sacc[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float mc = m_use * c;
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] * c - mc);
        m_run[qb] = m_new;
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][i], c, -mc));
            sacc[kb][qb][i] = p;
            rs += p;
          }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < G::kDBlk; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
      }

      // ---- O^T += V^T . P^T ------------------------------------------------
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          v8 pb[2];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = sacc[kb][qb][8 * th + j];
            pb[qb] = dt::cvt8(x);
          }
          const int g = 4 * kb + 2 * th + h;
#pragma unroll
          for (int db = 0; db < G::kDBlk; ++db) {
            const int d = db * 32 + l32;
            v8 a = __builtin_bit_cast(
                v8, *(const uint4*)(Vs + d * G::kVRow + ((g ^ v_swz(d)) << 4)));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) oacc[qb][db] = dt::mfma(a, pb[qb], oacc[qb][db]);
          }
        }
    }

    if (t + 1 < n_tiles) stage_store(smem + ((t + 1) & 1) * G::kStage);
    __syncthreads();
  }

  // ---- epilogue: O = O / l (to dtype), LSE = scale*m + ln(l) ----------------
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qw0 + 32 * qb + l32;
    const float lt = l_run[qb] + xor32(l_run[qb]);
    if (q >= Sq) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    T* orow = O + ((int64_t)b * Sq + q) * q_row_stride + (int64_t)hq * D;
#pragma unroll
    for (int db = 0; db < G::kDBlk; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * h;
        uint2 pk;
        pk.x = dt::pack2(oacc[qb][db][4 * i4 + 0] * inv, oacc[qb][db][4 * i4 + 1] * inv);
        pk.y = dt::pack2(oacc[qb][db][4 * i4 + 2] * inv, oacc[qb][db][4 * i4 + 3] * inv);
        *(uint2*)(orow + d) = pk;
      }
    if (LSE != nullptr && h == 0) {
      // ln(sum exp(scale*s)) = ln2 * (c*m + log2(l)), with c = scale*log2(e)
      const float lse = lt > 0.0f
                            ? (m_run[qb] * c + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f
                            : -INFINITY;
      LSE[((int64_t)b * Hq + hq) * Sq + q] = lse;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_t(const LaunchArgs& a) {
  const int nq = (a.Sq + kBM - 1) / kBM;
  const int64_t npairs = (int64_t)a.B * a.Hq;
  const int64_t nblocks = (int64_t)nq * npairs;
  const int pairs_per_xcd = (npairs % 8 == 0) ? (int)(npairs / 8) : 0;
  hipLaunchKernelGGL((fa_fwd_kernel<T, D>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                     a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse,
                     a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.causal, a.c, nq, pairs_per_xcd);
  return hipGetLastError();
}

int64_t grid_blocks(int B, int Sq, int Hq) {
  return (int64_t)((Sq + kBM - 1) / kBM) * B * Hq;
}

hipError_t launch(const LaunchArgs& a) {
  if (a.dtype == DType::kBF16) {
    if (a.D == 128) return launch_t<__bf16, 128>(a);
    return launch_t<__bf16, 64>(a);
  }
  if (a.D == 128) return launch_t<_Float16, 128>(a);
  return launch_t<_Float16, 64>(a);
}

}  // namespace fa
