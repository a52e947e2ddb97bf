// fa_tile.hip -- the tile kernels: the fused attention forward pass written
// in HIP C++ on gfx950 MFMA, for the shapes the generated assembly kernels do
// not take: head dimensions 192 and 256 (the JAX Pallas FlashAttention3
// page's `main` sweeps head_dim 64, 128 and 256, and its forward takes any
// multiple of 64), and decode-shaped calls (a few query
// rows over a long key range, where the q-heads of one kv-head are packed
// into one block of rows so that K and V are read once per kv-head).
//
// The method is the tiled online softmax of that page's `kv_loop` (running
// max m, running sum l, rescaled accumulator) in the exp2 form of the
// Croqtile `flash_atten` page (c = scale * log2(e) folded into the
// exponent), over one range of key tiles per work item; with more than one
// range per item the partial results go to a workspace and combine_kernel
// merges them (kernbench GQA prefill page, `_merge_running`).
//
// Layout of the products (v_mfma_f32_32x32x16, 64 lanes):
//   A (32x16): lane l holds A[l%32][8(l/32) .. 8(l/32)+7]
//   B (16x32): lane l holds B[8(l/32) .. +7][l%32]
//   C (32x32): lane l, register i holds C[8(i/4) + 4(l/32) + i%4][l%32]
// S^T = K.Q^T puts one query row on each lane (l%32), so row max, row sum
// and the rescale of O are per-lane scalars plus one exchange between the
// two half-waves.  O^T = V^T.P^T takes P^T straight from the C registers of
// S^T as its B operand: the 16 keys of one k-step sit in a lane half as keys
// {4h..4h+3, 8+4h..8+4h+3}, and V^T's A operand is read in the same key
// order with two transposing LDS reads (ds_read_b64_tr_b16: four
// consecutive key rows at one head dimension per lane).
//
// Two work splits per workgroup of four waves:
//   rows (KEYS = false): wave w owns rows 32w..32w+31 of a 128-row block and
//     every wave runs over every key of the tile (tiles of TK keys);
//   keys (KEYS = true): the four waves share one 32-row block and wave w
//     takes keys 32w..32w+31 of each 128-key tile; their (m, l, O) are
//     merged through LDS at the end.  This is the decode shape.
// Rows are (query, q-head) pairs: row n of an item is query i0 + n / gp of
// q-head h0 + n % gp, with gp = Hq / Hkv when the q-heads of a kv-head are
// packed and 1 otherwise.
//
// K and V tiles go global -> registers -> LDS (16-byte chunks, XOR-swizzled
// so that both the row reads of K and the transposing reads of V are free
// of bank conflicts), two LDS stages: the next tile's loads are in flight
// while the current one is used, with one barrier per tile.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"
#include "fa_mfma.h"

namespace fa {
namespace {

using namespace mfma;

__device__ __forceinline__ float wave_max32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// The slow-path trigger: a lane's sum of p over one tile above 2^8.  Every p
// then stays at most 2^8, far from fp32 and fp16 overflow.
constexpr float kTrigger = 256.0f;

}  // namespace

struct TileArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;       // may be null (final outputs only)
  float* part_o;    // split: [nsplit][B][Hq][Sq][D] fp32 (null: write o / lse)
  float* part_lse;  // split: [nsplit][B][Hq][Sq]
  int B, Sq, Skv, Hq, Hkv, causal;
  float c;          // scale * log2(e)
  int g;            // Hq / Hkv
  int gp;           // rows packing: g (q-heads of a kv-head packed) or 1
  int heads;        // head slots per batch: Hkv when packed, else Hq
  int row_blocks;   // row blocks per (batch, head slot)
  int nsplit;       // key ranges per item
};

namespace {

template <typename T, int D, int TK, bool KEYS>
struct Tile {
  static constexpr int kThreads = 256;
  static constexpr int kRows = KEYS ? 32 : 128;     // rows per item
  static constexpr int kCPR = D / 8;                 // 16-byte chunks per row
  static constexpr int kChunks = TK * kCPR;          // chunks per K (or V) tile
  static constexpr int kNC = kChunks / kThreads;     // chunks per thread per tile
  static constexpr int kTileBytes = TK * lds_pitch<D>() * 2;
  static constexpr int kKB = KEYS ? 1 : TK / 32;     // 32-key blocks per wave per tile
  static constexpr int kND = D / 32;                 // 32-dim blocks of O^T
  static constexpr int kNQ = D / 16;                 // k-steps of S^T
  static constexpr int kStageBytes = 2 * kTileBytes;
  // merge: m and l of 4 waves x 32 rows, then O of 4 x 32 rows (pitch D + 4 floats)
  static constexpr int kMergeBytes = KEYS ? 4 * (256 + 128 * (D + 4)) : 0;
  static constexpr int kLds = (2 * kStageBytes > kMergeBytes) ? 2 * kStageBytes : kMergeBytes;
  static_assert(kChunks % kThreads == 0, "tile chunks per thread");
  static_assert(!KEYS || TK == 128, "the key split gives each wave 32 keys of a 128-key tile");
};

template <typename T, int D, int TK, bool KEYS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
fwd_tile_kernel(TileArgs a) {
  using P = Tile<T, D, TK, KEYS>;
  __shared__ __attribute__((aligned(16))) char lds[P::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- the work item: (batch, head slot, row block, key range), row
  // blocks with the most keys first
  int idx = blockIdx.x;
  const int s = idx % a.nsplit;
  idx /= a.nsplit;
  const int b = idx % a.B;
  idx /= a.B;
  const int hs = idx % a.heads;
  const int rb = a.row_blocks - 1 - idx / a.heads;

  const int gp = a.gp;
  const int hk = (gp > 1) ? hs : hs / a.g;
  const int h0 = (gp > 1) ? hs * a.g : hs;  // first q-head of the item's rows
  const int n0 = rb * P::kRows;             // first packed row of the item
  const int off = a.Skv - a.Sq;             // bottom-right causal offset

  // this lane's row: n = n0 + 32 * (wave in rows mode) + l32
  const int n = n0 + (KEYS ? 0 : 32 * wave) + l32;
  const int qi = n / gp;
  const int qh = h0 + n % gp;
  const bool row_ok = qi < a.Sq;

  // keys of the item: up to the last row's causal limit
  const int last_n = min(n0 + P::kRows, a.Sq * gp) - 1;
  int kend = a.Skv;
  if (a.causal) kend = min(kend, last_n / gp + 1 + off);
  const int ntiles = kend > 0 ? (kend + TK - 1) / TK : 0;
  const int t0 = (int)((int64_t)s * ntiles / a.nsplit);
  const int t1 = (int)((int64_t)(s + 1) * ntiles / a.nsplit);
  const int klimit = a.causal ? qi + off : a.Skv - 1;  // last visible key of this row

  // ---- Q^T as B operand: lane holds Q[row][16t + 8h .. +7]
  s16x8 qf[P::kNQ];
  {
    const short* qp = static_cast<const short*>(a.q) +
                      (((int64_t)b * a.Sq + qi) * a.Hq + qh) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < P::kNQ; ++t) {
      s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
      qf[t] = row_ok ? *reinterpret_cast<const s16x8*>(qp + 16 * t) : z;
      // Q^T is only read (as the B operand) inside the loop: keep it in the
      // accumulator registers so the O accumulators, which the softmax
      // rescales with vector instructions, fit the vector registers
      asm volatile("" : "+a"(qf[t]));
    }
  }

  f32x16 oacc[P::kND];
#pragma unroll
  for (int d = 0; d < P::kND; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.0f;
  float m = -INFINITY;  // running max of c * s (one per row; both half-waves agree)
  float l = 0.0f;       // this lane's part of the running sum

  const int64_t kv_row = (int64_t)a.Hkv * D;  // elements between consecutive keys
  const short* kbase = static_cast<const short*>(a.k) + ((int64_t)b * a.Skv * a.Hkv + hk) * D;
  const short* vbase = static_cast<const short*>(a.v) + ((int64_t)b * a.Skv * a.Hkv + hk) * D;

  u32x4 kreg[P::kNC], vreg[P::kNC];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < P::kNC; ++u) {
      const int c = tid + P::kThreads * u;
      const int r = c / P::kCPR, ch = c % P::kCPR;
      // rows past the last key read the last key's row again: valid, finite
      // data whose logits are masked to -inf, so their p (and P.V terms) are 0
      const int64_t kc = min(t * TK + r, a.Skv - 1);
      kreg[u] = *reinterpret_cast<const u32x4*>(kbase + kc * kv_row + 8 * ch);
      vreg[u] = *reinterpret_cast<const u32x4*>(vbase + kc * kv_row + 8 * ch);
    }
  };
  auto store_tile = [&](int stage) {
    char* kl = lds + stage * P::kStageBytes;
    char* vl = kl + P::kTileBytes;
#pragma unroll
    for (int u = 0; u < P::kNC; ++u) {
      const int c = tid + P::kThreads * u;
      const int r = c / P::kCPR, ch = c % P::kCPR;
      *reinterpret_cast<u32x4*>(kl + lds_off<D>(r, ch)) = kreg[u];
      *reinterpret_cast<u32x4*>(vl + lds_off<D>(r, ch)) = vreg[u];
    }
  };

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int stage = (t - t0) & 1;
    if (t + 1 < t1) load_tile(t + 1);
    const char* kl = lds + stage * P::kStageBytes;
    const char* vl = kl + P::kTileBytes;

    // S^T for this wave's key blocks: the K operands of a block are read
    // from LDS before its MFMA chain, so the reads are in flight together
    f32x16 sacc[P::kKB];
#pragma unroll
    for (int kb = 0; kb < P::kKB; ++kb) {
      const int kr = (KEYS ? 32 * wave : 32 * kb) + l32;
      s16x8 kf[P::kNQ];
#pragma unroll
      for (int q = 0; q < P::kNQ; ++q)
        kf[q] = *reinterpret_cast<const s16x8*>(kl + lds_off<D>(kr, 2 * q + h));
      f32x16 acc = zero16();
#pragma unroll
      for (int q = 0; q < P::kNQ; ++q) acc = T::mma(kf[q], qf[q], acc);
      sacc[kb] = acc;
    }
    sched_reads_ahead<P::kKB * P::kNQ, 4, 0>();

    // mask: only a tile that some row of the wave does not fully see
    // (a wave-uniform test), by setting its hidden logits to -inf
    const int key0 = t * TK;
    const int klast = key0 + (KEYS ? 32 * wave + 31 : TK - 1);
    if (!__all((klast < kend) & (klast <= klimit))) {
#pragma unroll
      for (int kb = 0; kb < P::kKB; ++kb) {
        const int kbase_key = key0 + (KEYS ? 32 * wave : 32 * kb) + 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase_key + 8 * (i >> 2) + (i & 3);
          sacc[kb][i] = ((key < kend) & (key <= klimit)) ? sacc[kb][i] : -INFINITY;
        }
      }
    }
    // p = exp2(c*s - m) against the lazy reference m.  While every lane's
    // sum of its p in this tile stays at most kTrigger, each p is too, and m
    // stays; otherwise (and while a row has no reference yet) the slow path
    // takes the tile's row max, moves m, rescales O and l, and redoes p.
    f32x16 pv[P::kKB];
    float lt = 0.0f;
    float mref = (m == -INFINITY) ? 0.0f : m;
#pragma unroll
    for (int kb = 0; kb < P::kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], a.c, -mref));
        lt += pv[kb][i];
      }
    if (__any(!(lt <= kTrigger) || m == -INFINITY)) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < P::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i] * a.c);
      mt = wave_max32(mt);
      const float mnew = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.0f : mnew));
      m = mnew;
      mref = (m == -INFINITY) ? 0.0f : m;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < P::kND; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      lt = 0.0f;
#pragma unroll
      for (int kb = 0; kb < P::kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pv[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], a.c, -mref));
          lt += pv[kb][i];
        }
    }
    l += lt;

    // P^T packed to the input dtype as B operands, and O^T += V^T . P^T over
    // the 32 keys of each block (two k-steps), the V^T operands of a block
    // read before its MFMAs
#pragma unroll
    for (int kb = 0; kb < P::kKB; ++kb) {
      const int kb_row = KEYS ? 32 * wave : 32 * kb;
      s16x8 vf[2][P::kND];
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
#pragma unroll
        for (int d = 0; d < P::kND; ++d) vf[ts][d] = read_a_rows<D>(vl, kb_row, ts, 32 * d, lane);
      s16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = T::cvt(pv[kb][i]);
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
#pragma unroll
        for (int d = 0; d < P::kND; ++d) oacc[d] = T::mma(vf[ts][d], pf[ts], oacc[d]);
    }
    sched_reads_ahead<P::kKB * 2 * P::kND, 3, 1, 2>();

    if (t + 1 < t1) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int64_t rows_total = (int64_t)a.B * a.Hq * a.Sq;
  if constexpr (!KEYS) {
    const float ltot = l + __shfl_xor(l, 32);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const float lse = ltot > 0.0f ? (m + __builtin_log2f(ltot)) * kLn2 : -INFINITY;
    if (row_ok) {
      const int64_t row = ((int64_t)b * a.Hq + qh) * a.Sq + qi;  // (b, hq, i)
      if (a.part_o) {
        float* po = a.part_o + ((int64_t)s * rows_total + row) * D;
#pragma unroll
        for (int d = 0; d < P::kND; ++d)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 v4 = {oacc[d][4 * j] * inv, oacc[d][4 * j + 1] * inv, oacc[d][4 * j + 2] * inv,
                        oacc[d][4 * j + 3] * inv};
            *reinterpret_cast<f32x4*>(po + 32 * d + 8 * j + 4 * h) = v4;
          }
        if (h == 0) a.part_lse[(int64_t)s * rows_total + row] = lse;
      } else {
        short* op = static_cast<short*>(a.o) + (((int64_t)b * a.Sq + qi) * a.Hq + qh) * D;
#pragma unroll
        for (int d = 0; d < P::kND; ++d)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s16x4 v4 = {T::cvt(oacc[d][4 * j] * inv), T::cvt(oacc[d][4 * j + 1] * inv),
                        T::cvt(oacc[d][4 * j + 2] * inv), T::cvt(oacc[d][4 * j + 3] * inv)};
            *reinterpret_cast<s16x4*>(op + 32 * d + 8 * j + 4 * h) = v4;
          }
        if (h == 0 && a.lse) a.lse[row] = lse;
      }
    }
  } else {
    // merge the four waves' (m, l, O) of the same 32 rows through LDS:
    // per wave, m [32], l [32], O [32][D] fp32 (row pitch D + 4 floats)
    constexpr int kPitch = D + 4;
    float* mo = reinterpret_cast<float*>(lds);               // [4][32]
    float* lo = mo + 4 * 32;                                  // [4][32]
    float* ob = lo + 4 * 32;                                  // [4][32][kPitch]
    const float ltot = l + __shfl_xor(l, 32);
    if (h == 0) {
      mo[wave * 32 + l32] = m;
      lo[wave * 32 + l32] = ltot;
    }
    float* my = ob + (wave * 32 + l32) * kPitch;
#pragma unroll
    for (int d = 0; d < P::kND; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v4 = {oacc[d][4 * j], oacc[d][4 * j + 1], oacc[d][4 * j + 2], oacc[d][4 * j + 3]};
        *reinterpret_cast<f32x4*>(my + 32 * d + 8 * j + 4 * h) = v4;
      }
    __syncthreads();
    // thread -> (row r, dims [dq*D/8, (dq+1)*D/8))
    const int r = tid >> 3, dq = tid & 7;
    constexpr int kDT = D / 8;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = mo[w * 32 + r];
      M = fmaxf(M, mw[w]);
    }
    const float Mref = (M == -INFINITY) ? 0.0f : M;
    float wsum = 0.0f, wt[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = __builtin_amdgcn_exp2f(mw[w] - Mref);
      wsum += wt[w] * lo[w * 32 + r];
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const float lse = wsum > 0.0f ? (M + __builtin_log2f(wsum)) * kLn2 : -INFINITY;
    float out[kDT];
#pragma unroll
    for (int e = 0; e < kDT; ++e) out[e] = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* src = ob + (w * 32 + r) * kPitch + dq * kDT;
#pragma unroll
      for (int e = 0; e < kDT; e += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + e);
        out[e] += wt[w] * v4[0];
        out[e + 1] += wt[w] * v4[1];
        out[e + 2] += wt[w] * v4[2];
        out[e + 3] += wt[w] * v4[3];
      }
    }
    const int nr = n0 + r;
    const int ri = nr / gp, rh = h0 + nr % gp;
    if (ri < a.Sq) {
      const int64_t row = ((int64_t)b * a.Hq + rh) * a.Sq + ri;
      if (a.part_o) {
        float* po = a.part_o + ((int64_t)s * rows_total + row) * D + dq * kDT;
#pragma unroll
        for (int e = 0; e < kDT; e += 4) {
          f32x4 v4 = {out[e] * inv, out[e + 1] * inv, out[e + 2] * inv, out[e + 3] * inv};
          *reinterpret_cast<f32x4*>(po + e) = v4;
        }
        if (dq == 0) a.part_lse[(int64_t)s * rows_total + row] = lse;
      } else {
        short* op = static_cast<short*>(a.o) + (((int64_t)b * a.Sq + ri) * a.Hq + rh) * D + dq * kDT;
#pragma unroll
        for (int e = 0; e < kDT; e += 8) {
          s16x8 v8;
#pragma unroll
          for (int j = 0; j < 8; ++j) v8[j] = T::cvt(out[e + j] * inv);
          *reinterpret_cast<s16x8*>(op + e) = v8;
        }
        if (dq == 0 && a.lse) a.lse[row] = lse;
      }
    }
  }
}

template <typename T, int D, int TK, bool KEYS>
hipError_t launch_one(const TileArgs& a, int items, hipStream_t stream) {
  TileArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_tile_kernel<T, D, TK, KEYS>),
                         dim3((unsigned)(items * a.nsplit)), dim3(256), kargs, 0, stream);
}

template <typename T>
hipError_t launch_t(const TileArgs& a, int D, bool keys, int items, hipStream_t stream) {
  if (keys) {
    if (D == 64) return launch_one<T, 64, 128, true>(a, items, stream);
    if (D == 128) return launch_one<T, 128, 128, true>(a, items, stream);
    return hipErrorInvalidValue;
  }
  if (D == 64) return launch_one<T, 64, 64, false>(a, items, stream);
  if (D == 128) return launch_one<T, 128, 64, false>(a, items, stream);
  if (D == 192) return launch_one<T, 192, 64, false>(a, items, stream);
  if (D == 256) return launch_one<T, 256, 64, false>(a, items, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tile(const LaunchArgs& a, bool keys, bool packed, int nsplit, float* part_o,
                       float* part_lse) {
  TileArgs t;
  t.q = a.q;
  t.k = a.k;
  t.v = a.v;
  t.o = a.o;
  t.lse = a.lse;
  t.part_o = part_o;
  t.part_lse = part_lse;
  t.B = a.B;
  t.Sq = a.Sq;
  t.Skv = a.Skv;
  t.Hq = a.Hq;
  t.Hkv = a.Hkv;
  t.causal = a.causal;
  t.c = a.c;
  t.g = a.Hq / a.Hkv;
  t.gp = packed ? t.g : 1;
  t.heads = packed ? a.Hkv : a.Hq;
  const int rows = keys ? 32 : 128;
  t.row_blocks = (int)(((int64_t)a.Sq * t.gp + rows - 1) / rows);
  t.nsplit = nsplit;
  const int items = a.B * t.heads * t.row_blocks;
  if (a.dtype == DType::kBF16) return launch_t<BF16>(t, a.D, keys, items, a.stream);
  return launch_t<F16>(t, a.D, keys, items, a.stream);
}

}  // namespace fa
