// fa_bwd_wide.hip -- the backward's dK/dV and dQ kernels for head
// dimensions 192 and 256, in HIP C++ on gfx950 MFMA.
//
// The arithmetic is that of the JAX Pallas FlashAttention3 page's backward
// (`kernel_dkv`, `kernel_dq`), with the scale on the logits and this
// library's natural-log LSE (l2 = LSE * log2(e), written with delta by the
// delta kernel of fa_bwd.hip):
//   P  = exp2(c*S - l2),  dP = dO.V^T,  dS = P * (dP - delta)
//   dV = P^T.dO,  dK = scale * dS^T.Q  (summed over the q-heads of a kv-head),
//   dQ = scale * dS.K
// with P and dS rounded to the input dtype before the products that read
// them.
//
// At these head dimensions one wave cannot hold the gradients of 32 keys
// (2 * D * 32 fp32) next to the resident K and V, as the generated kernels
// for D <= 128 do.  Here a workgroup of D/64 waves splits the head dimension
// instead: wave w owns dimensions 64w .. 64w+63 of the resident operands and
// of the gradients.  Each wave computes S and dP of a 32 x 32 block over its
// 64 dimensions; the partial sums meet in LDS, every wave adds them in the
// same order (so all hold the same S and dP), and then multiplies its own
// slice of the gradient products.
//
// Products on v_mfma_f32_32x32x16 (64 lanes; the layouts are listed in
// fa_mfma.h):
//   dK/dV kernel, per 32-row block of Q / dO:
//     S = Q.K^T and dP = dO.V^T as C[rows][keys]: A = Q (dO) rows read from
//     LDS, B = the wave's K^T (V^T) slice, resident;
//     dV^T += dO^T.P, dK^T += Q^T.dS as C[dims][keys]: A = the tile read
//     transposed, B = P (dS) straight from the C registers of S.
//   dQ kernel, per 32-key block of K / V:
//     S^T = K.Q^T and dP^T = V.dO^T as C[keys][rows]: A = K (V) rows read from
//     LDS, B = the wave's Q^T (dO^T) slice, resident;
//     dQ^T += K^T.dS^T as C[dims][rows].
// A workgroup has two halves of D/64 waves: each takes one 32-key (dK/dV)
// or 32-row (dQ) block, and both read the same streamed tiles.  Q / dO
// (K / V) tiles go global -> registers -> LDS (XOR-swizzled rows, D = 192
// padded to 256 dimensions), one stage; barriers around the partial sums'
// reduction and the next block's store.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"
#include "fa_mfma.h"

namespace fa {
namespace {

using namespace mfma;

struct WideArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* l2;     // [B][Hq][Sq]: LSE * log2(e)
  const float* delta;  // [B][Hq][Sq]: rowsum(O * dO)
  void* dq;
  void* dk;
  void* dv;
  int B, Sq, Skv, Hq, Hkv, causal, g;
  float c;      // scale * log2(e)
  float scale;
};

// s_waitcnt vmcnt(0), the other counters left at their maxima
constexpr int kVmcnt0 = 0x0F70;

template <int D>
struct Wide {
  static constexpr int kWaves = D / 64;               // wave w owns dims 64w .. 64w+63
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kCPR = D / 8;                  // 16-byte chunks per row
  static constexpr int kNC = 32 * kCPR / kThreads;    // chunks per thread per 32-row tile
  static constexpr int kTileBytes = 32 * lds_pitch<D>() * 2;
  static constexpr int kStats = 2 * 32 * 4;           // l2 and delta of 32 rows (dK/dV kernel)
  static constexpr int kStage = 2 * kTileBytes + kStats;
  static constexpr int kPart = 2 * 64 * 16 * 4;       // one wave's partial S and dP
  static constexpr int kPds = 2 * 2 * 64 * 16;        // P and dS operands after the reduction
  // a workgroup: two halves of kWaves waves, one stage of tiles and an
  // exchange area (kWaves * kPart + kPds) per half: 88 KB of LDS at D = 192,
  // 104 KB at D = 256
  static_assert(D % 64 == 0 && 32 * kCPR % kThreads == 0, "tile chunks per thread");
};

template <typename T>
__device__ __forceinline__ void store4(void* base, int64_t elem, const f32x16& acc, int i0,
                                       float mul) {
  s16x4 v = {T::cvt(acc[i0] * mul), T::cvt(acc[i0 + 1] * mul), T::cvt(acc[i0 + 2] * mul),
             T::cvt(acc[i0 + 3] * mul)};
  *reinterpret_cast<s16x4*>(static_cast<short*>(base) + elem) = v;
}

// The waves' partial S and dP meet in LDS, four registers (one group) to a
// 16-byte word.  Wave w adds up, in wave order, the groups q with
// q % kWaves == w, turns their registers i = 4q .. 4q+3 into P and dS with
// f(i, s, dp, p, ds), and stores them rounded to the input dtype in the
// layout of B operands; after a barrier every wave reads back the operands
// of both k-steps: pb[t] (P, when kP; pb may be null otherwise) and sb[t]
// (dS).  A wave stores only the groups other waves add up and reads only
// the other waves' parts of its own groups.
template <typename T, int D, bool kP, typename F>
__device__ __forceinline__ void reduce_pds(char* xbase, int w, int lane, const f32x16& s,
                                           const f32x16& dp, s16x8* pb, s16x8 (&sb)[2], F&& f) {
  using W = Wide<D>;
  f32x4* x = reinterpret_cast<f32x4*>(xbase);                // [wave][S, dP][group][lane]
  short* y = reinterpret_cast<short*>(x + W::kWaves * 2 * 4 * 64);  // [dS, P][k-step][lane][8]
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q % W::kWaves != w) {
      x[((2 * w) * 4 + q) * 64 + lane] = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
      x[((2 * w + 1) * 4 + q) * 64 + lane] =
          f32x4{dp[4 * q], dp[4 * q + 1], dp[4 * q + 2], dp[4 * q + 3]};
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q % W::kWaves == w) {
      const f32x4 ms = {s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
      const f32x4 md = {dp[4 * q], dp[4 * q + 1], dp[4 * q + 2], dp[4 * q + 3]};
      f32x4 ss = w == 0 ? ms : x[(0 * 4 + q) * 64 + lane];
      f32x4 dd = w == 0 ? md : x[(1 * 4 + q) * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < W::kWaves; ++ww) {
        ss += ww == w ? ms : x[((2 * ww) * 4 + q) * 64 + lane];
        dd += ww == w ? md : x[((2 * ww + 1) * 4 + q) * 64 + lane];
      }
      s16x4 po, so;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pp, dss;
        f(4 * q + e, ss[e], dd[e], pp, dss);
        so[e] = T::cvt(dss);
        po[e] = T::cvt(pp);
      }
      // registers 4q .. 4q+3 are elements 4(q%2) .. +3 of the B operand of k-step q/2
      *reinterpret_cast<s16x4*>(y + (((q >> 1) * 64) + lane) * 8 + 4 * (q & 1)) = so;
      if constexpr (kP) *reinterpret_cast<s16x4*>(y + (((2 + (q >> 1)) * 64) + lane) * 8 + 4 * (q & 1)) = po;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ts = 0; ts < 2; ++ts) {
    sb[ts] = *reinterpret_cast<const s16x8*>(y + ((ts * 64) + lane) * 8);
    if constexpr (kP) pb[ts] = *reinterpret_cast<const s16x8*>(y + (((2 + ts) * 64) + lane) * 8);
  }
}

// ---------------------------------------------------------------------------
// dK / dV: a workgroup per (64-key block, batch, kv-head), the key blocks in
// order (under a causal mask the first see the most rows); it streams every
// 32-row block of every q-head of its group that sees one of its keys.  Its
// two halves of D/64 waves each take one 32-key block and share the tiles
// (under a causal mask the second half's first row block is hidden from it).
template <typename T, int D>
__global__ void __launch_bounds__(2 * Wide<D>::kThreads) bwd_dkv_wide(WideArgs a) {
  using W = Wide<D>;
  constexpr int kThr = 2 * W::kThreads;             // two key blocks share the tiles
  constexpr int kNC2 = 32 * W::kCPR / kThr;
  constexpr int kExch = W::kWaves * W::kPart + W::kPds;
  __shared__ __attribute__((aligned(16))) char lds[W::kStage + 2 * kExch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int kb = wv / W::kWaves, w = wv % W::kWaves;

  int idx = blockIdx.x;
  const int hk = idx % a.Hkv;
  idx /= a.Hkv;
  const int b = idx % a.B;
  const int jp = 64 * (idx / a.B);
  const int j0 = jp + 32 * kb;
  const int off = a.Skv - a.Sq;
  const int64_t kvrow = (int64_t)a.Hkv * D, qrow = (int64_t)a.Hq * D;

  // K^T and V^T of the wave's dimensions as B operands: lane holds
  // K[j0 + l32][64w + 16t + 8h .. +7]
  const int j = j0 + l32;
  const bool key_ok = j < a.Skv;
  s16x8 kB[4], vB[4];
  {
    const int64_t e = ((int64_t)b * a.Skv + (key_ok ? j : 0)) * kvrow + (int64_t)hk * D + 64 * w + 8 * h;
    const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kB[t] = key_ok ? *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.k) + e + 16 * t) : z;
      vB[t] = key_ok ? *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.v) + e + 16 * t) : z;
    }
  }
  f32x16 dv[2] = {zero16(), zero16()}, dk[2] = {zero16(), zero16()};

  // the 32-row blocks that see a key of the block: from the first row that
  // sees key j0 to the last row, for each q-head of the group
  const int i_first = a.causal ? (jp - off > 0 ? jp - off : 0) : 0;
  const int nib = (a.Sq + 31) / 32;
  const int ib0 = i_first / 32;
  const int per_head = (jp < a.Skv && i_first < a.Sq) ? nib - ib0 : 0;
  const int nsteps = per_head * a.g;

  // The thread's chunks of a tile: row rr[u] (the same in every tile) and
  // element offset coff[u] within that row.  Rows past Sq read row Sq - 1
  // again: finite data whose P and dS the mask sets to 0, so they add nothing
  // to dK and dV.  Offsets from the tile's first row fit 32 bits: the rows
  // stay inside one batch slice of q, below 2 GiB (the entry point checks).
  int rr[kNC2];
  uint32_t coff[kNC2];
#pragma unroll
  for (int u = 0; u < kNC2; ++u) {
    const int c = tid + kThr * u;
    rr[u] = c / W::kCPR;
    coff[u] = 8 * (c % W::kCPR);
  }
  u32x4 qr[kNC2], dr[kNC2];
  float stat = 0.0f;
  // (q-head, row block) of the next tile to load, advanced after each load
  int lhq = hk * a.g, lib = ib0;
  auto load = [&]() {
    const int64_t base = ((int64_t)b * a.Sq + 32 * lib) * qrow + (int64_t)lhq * D;
    const short* qp = static_cast<const short*>(a.q) + base;
    const short* dp = static_cast<const short*>(a.dout) + base;
    const int last = a.Sq - 1 - 32 * lib;  // last row of the tile inside Sq
#pragma unroll
    for (int u = 0; u < kNC2; ++u) {
      const uint32_t e = (uint32_t)min(rr[u], last) * (uint32_t)qrow + coff[u];
      qr[u] = *reinterpret_cast<const u32x4*>(qp + e);
      dr[u] = *reinterpret_cast<const u32x4*>(dp + e);
    }
    if (tid < 64) {  // l2 (lanes 0-31) and delta (32-63) of the 32 rows
      const int64_t row = ((int64_t)b * a.Hq + lhq) * a.Sq + 32 * lib + min(l32, last);
      stat = h == 0 ? a.l2[row] : a.delta[row];
    }
    if (++lib == nib) {
      lib = ib0;
      ++lhq;
    }
  };
  auto store = [&](int stage) {
    char* qt = lds + stage * W::kStage;
#pragma unroll
    for (int u = 0; u < kNC2; ++u) {
      const int c = tid + kThr * u;
      const int r = c / W::kCPR, ch = c % W::kCPR;
      *reinterpret_cast<u32x4*>(qt + lds_off<D>(r, ch)) = qr[u];
      *reinterpret_cast<u32x4*>(qt + W::kTileBytes + lds_off<D>(r, ch)) = dr[u];
    }
    if (tid < 64) reinterpret_cast<float*>(qt + 2 * W::kTileBytes)[tid] = stat;
  };

  if (nsteps > 0) {
    load();
    store(0);
  }
  // Every load so far has landed (the resident operands included).  Said
  // explicitly, so that the loop's first products do not wait for the
  // next tile's loads, which the compiler cannot count across the branches.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  char* xbase = lds + W::kStage + kb * kExch;
  int ib = ib0;  // row block of the tile in LDS
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load();
    const char* qt = lds;
    const char* dt = qt + W::kTileBytes;
    const float* st = reinterpret_cast<const float*>(qt + 2 * W::kTileBytes);

    // partial S and dP over the wave's dimensions, C[rows][keys]
    f32x16 sv = zero16(), dpv = zero16();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sv = T::mma(read_rows<D>(qt, 0, 4 * w + t, lane), kB[t], sv);
      dpv = T::mma(read_rows<D>(dt, 0, 4 * w + t, lane), vB[t], dpv);
    }
    sched_reads_ahead<8, 4, 0>();
    // P and dS: lane = key j, register i = row 8(i/4) + 4h + i%4 of the block
    s16x8 pb[2], sb[2];
    // the block is fully visible (every key to every row): no mask
    // (judged for both key blocks, so that the workgroup takes one branch)
    const bool full = (jp + 63 < a.Skv) & (32 * ib + 31 < a.Sq) &
                      (!a.causal | (jp + 63 <= 32 * ib + off));
    auto pds = [&](int i, float s_, float dp_, float& p_, float& ds_, bool masked) {
      const int rl = 8 * (i >> 2) + 4 * h + (i & 3);
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s_, a.c, -st[rl]));
      if (masked) {
        const int row = 32 * ib + rl;
        const bool vis = key_ok & (row < a.Sq) & (!a.causal | (j <= row + off));
        p_ = vis ? e : 0.0f;
      } else {
        p_ = e;
      }
      ds_ = p_ * (dp_ - st[32 + rl]);
    };
    if (full)
      reduce_pds<T, D, true>(xbase, w, lane, sv, dpv, pb, sb,
                             [&](int i, float s_, float dp_, float& p_, float& ds_) {
                               pds(i, s_, dp_, p_, ds_, false);
                             });
    else
      reduce_pds<T, D, true>(xbase, w, lane, sv, dpv, pb, sb,
                             [&](int i, float s_, float dp_, float& p_, float& ds_) {
                               pds(i, s_, dp_, p_, ds_, true);
                             });
    // dV^T += dO^T.P and dK^T += Q^T.dS over the wave's dimensions
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        dv[d] = T::mma(read_a_rows<D>(dt, 0, ts, 64 * w + 32 * d, lane), pb[ts], dv[d]);
        dk[d] = T::mma(read_a_rows<D>(qt, 0, ts, 64 * w + 32 * d, lane), sb[ts], dk[d]);
      }
    sched_reads_ahead<8, 3, 1, 2, 4>();  // after the four reads of P and dS

    if (s + 1 < nsteps) {
      __syncthreads();  // every wave is done with this block's tiles
      store(0);
    }
    __syncthreads();
    if (++ib == nib) ib = ib0;
  }

  // dK = scale * (dK^T)^T, dV: lane = key, register i = dim 8(i/4) + 4h + i%4 of a 32-dim block
  if (key_ok) {
    const int64_t e = ((int64_t)b * a.Skv + j) * kvrow + (int64_t)hk * D + 64 * w + 4 * h;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        store4<T>(a.dk, e + 32 * d + 8 * q, dk[d], 4 * q, a.scale);
        store4<T>(a.dv, e + 32 * d + 8 * q, dv[d], 4 * q, 1.0f);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup per (64-row block, batch, q-head), the row blocks from the
// last (under a causal mask the last rows see the most keys); it streams the
// 32-key blocks of K and V its rows see.  Its two halves of D/64 waves each
// take one 32-row block and share the tiles (under a causal mask the first
// half's last key block is hidden from it).
template <typename T, int D>
__global__ void __launch_bounds__(2 * Wide<D>::kThreads) bwd_dq_wide(WideArgs a) {
  using W = Wide<D>;
  constexpr int kThr = 2 * W::kThreads;             // two row blocks share the tiles
  constexpr int kNC2 = 32 * W::kCPR / kThr;
  constexpr int kExch = W::kWaves * W::kPart + W::kPds;
  __shared__ __attribute__((aligned(16))) char lds[W::kStage + 2 * kExch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int kb = wv / W::kWaves, w = wv % W::kWaves;

  int idx = blockIdx.x;
  const int hq = idx % a.Hq;
  idx /= a.Hq;
  const int b = idx % a.B;
  const int nip = (a.Sq + 63) / 64;
  const int ip = 64 * (nip - 1 - idx / a.B);  // first row of the pair
  const int i0 = ip + 32 * kb;
  const int hk = hq / a.g;
  const int off = a.Skv - a.Sq;
  const int64_t kvrow = (int64_t)a.Hkv * D, qrow = (int64_t)a.Hq * D;

  // Q^T and dO^T of the wave's dimensions as B operands: lane holds
  // Q[i0 + l32][64w + 16t + 8h .. +7]
  const int i = i0 + l32;
  const bool row_ok = i < a.Sq;
  s16x8 qB[4], oB[4];
  {
    const int64_t e = ((int64_t)b * a.Sq + (row_ok ? i : 0)) * qrow + (int64_t)hq * D + 64 * w + 8 * h;
    const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qB[t] = row_ok ? *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.q) + e + 16 * t) : z;
      oB[t] = row_ok ? *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.dout) + e + 16 * t) : z;
    }
  }
  const int64_t srow = ((int64_t)b * a.Hq + hq) * a.Sq + (row_ok ? i : 0);
  const float l2v = row_ok ? a.l2[srow] : 0.0f;
  const float dlv = row_ok ? a.delta[srow] : 0.0f;
  f32x16 dq[2] = {zero16(), zero16()};

  // the key blocks up to the last key a row of the pair sees
  const int last_row = (ip + 63 < a.Sq ? ip + 63 : a.Sq - 1);
  int kend = a.Skv;
  if (a.causal && last_row + off + 1 < kend) kend = last_row + off + 1;
  const int nsteps = kend > 0 ? (kend + 31) / 32 : 0;

  // The thread's chunks of a tile: key row rr[u] of the tile and element
  // offset coff[u] within that row.  Keys past Skv read key Skv - 1 again:
  // finite data whose dS the mask sets to 0, so they add nothing to dQ.
  // Offsets from the tile's first key fit 32 bits: the keys stay inside one
  // batch slice of k, below 2 GiB (the entry point checks).
  int rr[kNC2];
  uint32_t coff[kNC2];
#pragma unroll
  for (int u = 0; u < kNC2; ++u) {
    const int c = tid + kThr * u;
    rr[u] = c / W::kCPR;
    coff[u] = 8 * (c % W::kCPR);
  }
  u32x4 kr[kNC2], vr[kNC2];
  auto load = [&](int s) {
    const int64_t base = ((int64_t)b * a.Skv + 32 * s) * kvrow + (int64_t)hk * D;
    const short* kp = static_cast<const short*>(a.k) + base;
    const short* vp = static_cast<const short*>(a.v) + base;
    const int last = a.Skv - 1 - 32 * s;  // last key of the tile inside Skv
#pragma unroll
    for (int u = 0; u < kNC2; ++u) {
      const uint32_t e = (uint32_t)min(rr[u], last) * (uint32_t)kvrow + coff[u];
      kr[u] = *reinterpret_cast<const u32x4*>(kp + e);
      vr[u] = *reinterpret_cast<const u32x4*>(vp + e);
    }
  };
  auto store = [&](int stage) {
    char* kt = lds + stage * W::kStage;
#pragma unroll
    for (int u = 0; u < kNC2; ++u) {
      const int c = tid + kThr * u;
      const int r = c / W::kCPR, ch = c % W::kCPR;
      *reinterpret_cast<u32x4*>(kt + lds_off<D>(r, ch)) = kr[u];
      *reinterpret_cast<u32x4*>(kt + W::kTileBytes + lds_off<D>(r, ch)) = vr[u];
    }
  };

  if (nsteps > 0) {
    load(0);
    store(0);
  }
  // Every load so far has landed (the resident operands included).  Said
  // explicitly, so that the loop's first products do not wait for the
  // next tile's loads, which the compiler cannot count across the branches.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  char* xbase = lds + W::kStage + kb * kExch;
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load(s + 1);
    const char* kt = lds;
    const char* vt = kt + W::kTileBytes;

    // partial S^T and dP^T over the wave's dimensions, C[keys][rows]
    f32x16 sv = zero16(), dpv = zero16();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sv = T::mma(read_rows<D>(kt, 0, 4 * w + t, lane), qB[t], sv);
      dpv = T::mma(read_rows<D>(vt, 0, 4 * w + t, lane), oB[t], dpv);
    }
    sched_reads_ahead<8, 4, 0>();
    // dS^T: lane = row i, register r = key 8(r/4) + 4h + r%4 of the block
    s16x8 sb[2];
    // the block is fully visible (every key to every row): no mask
    // (judged for both row blocks, so that the workgroup takes one branch)
    const bool full = (32 * s + 31 < a.Skv) & (ip + 63 < a.Sq) &
                      (!a.causal | (32 * s + 31 <= ip + off));
    auto pds = [&](int r, float s_, float dp_, float& p_, float& ds_, bool masked) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s_, a.c, -l2v));
      if (masked) {
        const int key = 32 * s + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool vis = row_ok & (key < a.Skv) & (!a.causal | (key <= i + off));
        p_ = vis ? e : 0.0f;
      } else {
        p_ = e;
      }
      ds_ = p_ * (dp_ - dlv);
    };
    if (full)
      reduce_pds<T, D, false>(xbase, w, lane, sv, dpv, nullptr, sb,
                              [&](int r, float s_, float dp_, float& p_, float& ds_) {
                                pds(r, s_, dp_, p_, ds_, false);
                              });
    else
      reduce_pds<T, D, false>(xbase, w, lane, sv, dpv, nullptr, sb,
                              [&](int r, float s_, float dp_, float& p_, float& ds_) {
                                pds(r, s_, dp_, p_, ds_, true);
                              });
    // dQ^T += K^T.dS^T over the wave's dimensions
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
        dq[d] = T::mma(read_a_rows<D>(kt, 0, ts, 64 * w + 32 * d, lane), sb[ts], dq[d]);
    sched_reads_ahead<4, 3, 1, 2, 2>();  // after the two reads of dS

    if (s + 1 < nsteps) {
      __syncthreads();  // every wave is done with this block's tiles
      store(0);
    }
    __syncthreads();
  }

  // dQ = scale * (dQ^T)^T: lane = row, register r = dim 8(r/4) + 4h + r%4 of a 32-dim block
  if (row_ok) {
    const int64_t e = ((int64_t)b * a.Sq + i) * qrow + (int64_t)hq * D + 64 * w + 4 * h;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) store4<T>(a.dq, e + 32 * d + 8 * q, dq[d], 4 * q, a.scale);
  }
}

template <typename T, int D>
hipError_t launch_wide_d(const WideArgs& in, hipStream_t stream) {
  using W = Wide<D>;
  WideArgs a = in;
  void* args[] = {&a};
  const unsigned nkp = (unsigned)((a.Skv + 63) / 64), nip = (unsigned)((a.Sq + 63) / 64);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkv_wide<T, D>),
                                 dim3(nkp * (unsigned)a.B * (unsigned)a.Hkv), dim3(2 * W::kThreads), args,
                                 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_wide<T, D>),
                         dim3(nip * (unsigned)a.B * (unsigned)a.Hq), dim3(2 * W::kThreads), args, 0,
                         stream);
}

}  // namespace

hipError_t launch_bwd_wide(const BwdLaunchArgs& in) {
  WideArgs a;
  const size_t rows = (size_t)in.B * in.Hq * in.Sq;
  a.q = in.q;
  a.k = in.k;
  a.v = in.v;
  a.dout = in.dout;
  a.l2 = in.ws;
  a.delta = in.ws + rows;
  a.dq = in.dq;
  a.dk = in.dk;
  a.dv = in.dv;
  a.B = in.B;
  a.Sq = in.Sq;
  a.Skv = in.Skv;
  a.Hq = in.Hq;
  a.Hkv = in.Hkv;
  a.causal = in.causal;
  a.g = in.Hq / in.Hkv;
  a.c = in.c;
  a.scale = in.scale;
  const bool bf = in.dtype == DType::kBF16;
  if (in.D == 192) return bf ? launch_wide_d<BF16, 192>(a, in.stream) : launch_wide_d<F16, 192>(a, in.stream);
  if (in.D == 256) return bf ? launch_wide_d<BF16, 256>(a, in.stream) : launch_wide_d<F16, 256>(a, in.stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
