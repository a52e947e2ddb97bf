// fa_bwd.hip -- the attention backward pass on gfx950 MFMA: given q, k, v,
// the forward's o and (natural-log) lse, and the upstream gradient dO, the
// gradients dQ, dK and dV.
//
// The JAX Pallas FlashAttention3 page's backward, with the scale applied to
// the logits and its base-2 residual replaced by this library's natural-log
// LSE (p = exp2(c*q.k - LSE*log2(e)), c = scale*log2(e)):
//   delta   = rowsum(O * dO)                          (`_attention_bwd`)
//   P       = exp2(c*S - LSE*log2(e)),  dP = dO.V^T,  dS = P * (dP - delta)
//   dQ      = scale * dS.K                            (`kernel_dq`)
//   dK, dV  = scale * dS^T.Q,  P^T.dO, summed over the q-heads of a kv-head
//                                                     (`kernel_dkv`)
// P and dS are rounded to the input dtype before the products that read
// them, as that page casts them (`astype`); every product accumulates in
// fp32 and each gradient is rounded once at the end.  The page has no causal
// backward; here the causal mask (bottom-right, as in the forward) gives P =
// 0 on masked pairs, which is the gradient of the masked forward.
//
// Three kernels, in stream order:
//   bwd_delta_kernel  delta per query row into the workspace;
//   bwd_dkv_kernel    a workgroup per (batch, kv-head, 128 keys): each wave
//                     keeps the K and V rows of its 32 keys in registers and
//                     runs over every q-head of the group and every query
//                     block that sees its keys (Q, dO, LSE and delta blocks
//                     staged through LDS), accumulating dK^T and dV^T;
//   bwd_dq_kernel     a workgroup per (batch, q-head, 128 query rows): each
//                     wave keeps Q and dO of its 32 rows in registers and runs
//                     over the visible key tiles (K, V staged through LDS),
//                     recomputing S^T and dP^T, accumulating dQ^T.
// No atomics: every gradient element has one writer.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernel.h"
#include "fa_mfma.h"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace [B][Hq][Sq]
  int B, Sq, Skv, Hq, Hkv, causal;
  float scale;
  float c;  // scale * log2(e)
};

namespace {

using namespace mfma;

// delta[(b*Hq + hq)*Sq + i] = sum_d O[b,i,hq,d] * dO[b,i,hq,d] in fp32; D/8
// lanes per row, 8 elements each.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdArgs a) {
  constexpr int L = D / 8;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int64_t r = (int64_t)blockIdx.x * (256 / L) + threadIdx.x / L;
  const int lane = threadIdx.x % L;
  float acc = 0.0f;
  if (r < rows) {
    const int i = (int)(r % a.Sq);
    const int64_t bh = r / a.Sq;
    const int hq = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    const int64_t off = (((int64_t)b * a.Sq + i) * a.Hq + hq) * D + 8 * lane;
    const s16x8 o8 = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.o) + off);
    const s16x8 d8 = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.dout) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += T::widen(o8[e]) * T::widen(d8[e]);
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (r < rows && lane == 0) a.delta[r] = acc;
}

// LSE in log2 units for p = exp2(c*s - lse2); a row without a visible key
// (LSE = -inf) gets +inf, so that all its p are 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_dkv_kernel(BwdArgs a) {
  constexpr int BQ = 64;                     // query rows per step
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BQ * D * 2;           // bytes of one Q (or dO) block
  constexpr int NC = BQ * CPR / 256;         // chunks per thread per block
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;
  constexpr int NQ = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  int idx = blockIdx.x;
  const int nkb = (a.Skv + 127) / 128;
  const int kblk = idx % nkb;
  idx /= nkb;
  const int hk = idx % a.Hkv;
  const int b = idx / a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int off = a.Skv - a.Sq;
  const int k0 = kblk * 128;
  const int key = k0 + 32 * wave + l32;  // this lane's key (the C column)
  const bool key_ok = key < a.Skv;

  // K^T and V^T as B operands: lane holds K[key][16t + 8h .. +7]
  s16x8 kf[NQ], vf[NQ];
  {
    // a key past the end reads the last key's row: finite data, and its
    // gradients are not stored
    const int64_t kc = min(key, a.Skv - 1);
    const int64_t kvoff = (((int64_t)b * a.Skv + kc) * a.Hkv + hk) * D + 8 * h;
    const short* kp = static_cast<const short*>(a.k) + kvoff;
    const short* vp = static_cast<const short*>(a.v) + kvoff;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      kf[t] = *reinterpret_cast<const s16x8*>(kp + 16 * t);
      vf[t] = *reinterpret_cast<const s16x8*>(vp + 16 * t);
      // only read (as B operands) in the loop: kept in the accumulator
      // registers, leaving the vector registers to the accumulators and the
      // operands read ahead
      asm volatile("" : "+a"(kf[t]));
      asm volatile("" : "+a"(vf[t]));
    }
  }
  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dka[d] = zero16();
    dva[d] = zero16();
  }

  // query blocks whose rows see a key of [k0, k0 + 128), for every q-head
  const int i_first = a.causal ? max(0, k0 - off) : 0;
  const int qb0 = i_first / BQ;
  const int nqb = (a.Sq + BQ - 1) / BQ;
  const int per_head = (k0 < a.Skv && qb0 < nqb) ? nqb - qb0 : 0;
  const int nsteps = g * per_head;

  u32x4 qreg[NC], dreg[NC];
  float lreg = INFINITY, dlreg = 0.0f;
  auto load_step = [&](int st) {
    const int hq = hk * g + st / per_head;
    const int i0 = (qb0 + st % per_head) * BQ;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + 256 * u;
      const int r = c / CPR, ch = c % CPR;
      // a row past the end reads the last row: finite data whose P is 0
      // (its LSE is taken as +inf below), so it adds nothing
      const int i = min(i0 + r, a.Sq - 1);
      const int64_t e = (((int64_t)b * a.Sq + i) * a.Hq + hq) * D + 8 * ch;
      qreg[u] = *reinterpret_cast<const u32x4*>(static_cast<const short*>(a.q) + e);
      dreg[u] = *reinterpret_cast<const u32x4*>(static_cast<const short*>(a.dout) + e);
    }
    if (tid < BQ) {
      const int i = i0 + tid;
      lreg = INFINITY;
      dlreg = 0.0f;
      if (i < a.Sq) {
        const int64_t row = ((int64_t)b * a.Hq + hq) * a.Sq + i;
        lreg = lse2_of(a.lse[row]);
        dlreg = a.delta[row];
      }
    }
  };
  auto store_step = [&](int stage) {
    char* ql = lds + stage * STAGE;
    char* dl = ql + TILE;
    float* ll = reinterpret_cast<float*>(dl + TILE);
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + 256 * u;
      const int r = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4*>(ql + lds_off<D>(r, ch)) = qreg[u];
      *reinterpret_cast<u32x4*>(dl + lds_off<D>(r, ch)) = dreg[u];
    }
    if (tid < BQ) {
      ll[tid] = lreg;
      ll[BQ + tid] = dlreg;
    }
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int stage = st & 1;
    const int i0 = (qb0 + st % per_head) * BQ;
    if (st + 1 < nsteps) load_step(st + 1);
    const char* ql = lds + stage * STAGE;
    const char* dl = ql + TILE;
    const float* ll = reinterpret_cast<const float*>(dl + TILE);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // S = Q.K^T and dP = dO.V^T, C[query][key]; the A operands (rows of
      // the Q and dO blocks) read ahead of their MFMA chains
      s16x8 qa[NQ], da[NQ];
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        qa[t] = read_rows<D>(ql, 32 * qh, t, lane);
        da[t] = read_rows<D>(dl, 32 * qh, t, lane);
      }
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int t = 0; t < NQ; ++t) s = T::mma(qa[t], kf[t], s);
#pragma unroll
      for (int t = 0; t < NQ; ++t) dp = T::mma(da[t], vf[t], dp);
      sched_reads_ahead<2 * NQ, 4, 0>();
      f32x16 p, ds;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 32 * qh + 8 * j + 4 * h;  // rows row .. row+3 of the block
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ll + row);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(ll + BQ + row);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = i0 + row + e;
          const bool vis = key_ok & ((a.causal == 0) | (key <= qi + off));  // no short-circuit branches
          const float x = vis ? s[4 * j + e] * a.c - l4[e] : -INFINITY;
          const float pv = __builtin_amdgcn_exp2f(x);
          p[4 * j + e] = pv;
          ds[4 * j + e] = pv * (dp[4 * j + e] - d4[e]);
        }
      }
      // dV^T += dO^T.P, then dK^T += Q^T.dS, over the 32 rows (two k-steps
      // each); their A operands read transposed from the dO and Q blocks
      {
        s16x8 dta[2][ND];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
          for (int db = 0; db < ND; ++db) dta[ts][db] = read_a_rows<D>(dl, 32 * qh, ts, 32 * db, lane);
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
          const s16x8 pb = pack_b<T>(p, ts);
#pragma unroll
          for (int db = 0; db < ND; ++db) dva[db] = T::mma(dta[ts][db], pb, dva[db]);
        }
        sched_reads_ahead<2 * ND, 3, 1, 2>();
      }
      {
        s16x8 qta[2][ND];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
          for (int db = 0; db < ND; ++db) qta[ts][db] = read_a_rows<D>(ql, 32 * qh, ts, 32 * db, lane);
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
          const s16x8 sb = pack_b<T>(ds, ts);
#pragma unroll
          for (int db = 0; db < ND; ++db) dka[db] = T::mma(qta[ts][db], sb, dka[db]);
        }
        sched_reads_ahead<2 * ND, 3, 2, 2>();
      }
    }
    if (st + 1 < nsteps) store_step(stage ^ 1);
    __syncthreads();
  }

  // dK^T, dV^T: C[dim][key]; lane's key, dims 32db + 8j + 4h .. +3
  if (key_ok) {
    const int64_t base = (((int64_t)b * a.Skv + key) * a.Hkv + hk) * D + 4 * h;
    short* dkp = static_cast<short*>(a.dk) + base;
    short* dvp = static_cast<short*>(a.dv) + base;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = T::cvt(a.scale * dka[db][4 * j + e]);
          v4[e] = T::cvt(dva[db][4 * j + e]);
        }
        *reinterpret_cast<s16x4*>(dkp + 32 * db + 8 * j) = k4;
        *reinterpret_cast<s16x4*>(dvp + 32 * db + 8 * j) = v4;
      }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_dq_kernel(BwdArgs a) {
  constexpr int TK = 64;
  constexpr int CPR = D / 8;
  constexpr int TILE = TK * D * 2;
  constexpr int NC = TK * CPR / 256;
  constexpr int STAGE = 2 * TILE;
  constexpr int NQ = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  int idx = blockIdx.x;
  const int nqb = (a.Sq + 127) / 128;
  const int qb = nqb - 1 - idx % nqb;  // the longest query blocks first
  idx /= nqb;
  const int hq = idx % a.Hq;
  const int b = idx / a.Hq;
  const int hk = hq / (a.Hq / a.Hkv);
  const int off = a.Skv - a.Sq;
  const int qi = qb * 128 + 32 * wave + l32;  // this lane's query row (the C column)
  const bool row_ok = qi < a.Sq;

  // Q^T and dO^T as B operands: lane holds Q[qi][16t + 8h .. +7]
  s16x8 qf[NQ], df[NQ];
  float lse2 = INFINITY, dl = 0.0f;
  {
    // a row past the end reads the last row (finite; its dQ is not stored)
    const int64_t e = (((int64_t)b * a.Sq + min(qi, a.Sq - 1)) * a.Hq + hq) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      qf[t] = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.q) + e + 16 * t);
      df[t] = *reinterpret_cast<const s16x8*>(static_cast<const short*>(a.dout) + e + 16 * t);
      asm volatile("" : "+a"(qf[t]));  // read-only B operands: accumulator registers
      asm volatile("" : "+a"(df[t]));
    }
    if (row_ok) {
      const int64_t row = ((int64_t)b * a.Hq + hq) * a.Sq + qi;
      lse2 = lse2_of(a.lse[row]);
      dl = a.delta[row];
    }
  }
  f32x16 dqa[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dqa[d] = zero16();

  const int last_i = min(a.Sq, (qb + 1) * 128) - 1;
  const int kend = a.causal ? min(a.Skv, last_i + 1 + off) : a.Skv;
  const int ntiles = kend > 0 ? (kend + TK - 1) / TK : 0;
  const int klimit = a.causal ? qi + off : a.Skv - 1;  // last key this row sees

  const int64_t kv_row = (int64_t)a.Hkv * D;
  const short* kbase = static_cast<const short*>(a.k) + ((int64_t)b * a.Skv * a.Hkv + hk) * D;
  const short* vbase = static_cast<const short*>(a.v) + ((int64_t)b * a.Skv * a.Hkv + hk) * D;
  u32x4 kreg[NC], vreg[NC];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + 256 * u;
      const int r = c / CPR, ch = c % CPR;
      // keys past the end read the last key's row: finite, masked to P = 0
      const int64_t kk = min(t * TK + r, a.Skv - 1);
      kreg[u] = *reinterpret_cast<const u32x4*>(kbase + kk * kv_row + 8 * ch);
      vreg[u] = *reinterpret_cast<const u32x4*>(vbase + kk * kv_row + 8 * ch);
    }
  };
  auto store_tile = [&](int stage) {
    char* kl = lds + stage * STAGE;
    char* vl = kl + TILE;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + 256 * u;
      const int r = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4*>(kl + lds_off<D>(r, ch)) = kreg[u];
      *reinterpret_cast<u32x4*>(vl + lds_off<D>(r, ch)) = vreg[u];
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const char* kl = lds + stage * STAGE;
    const char* vl = kl + TILE;
#pragma unroll
    for (int kb = 0; kb < TK / 32; ++kb) {
      // S^T = K.Q^T and dP^T = V.dO^T, C[key][query]; the A operands (rows
      // of the K and V tiles) read ahead of their MFMA chains
      s16x8 ka[NQ], va[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        ka[u] = read_rows<D>(kl, 32 * kb, u, lane);
        va[u] = read_rows<D>(vl, 32 * kb, u, lane);
      }
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int u = 0; u < NQ; ++u) s = T::mma(ka[u], qf[u], s);
#pragma unroll
      for (int u = 0; u < NQ; ++u) dp = T::mma(va[u], df[u], dp);
      sched_reads_ahead<2 * NQ, 4, 0>();
      s16x8 kta[2][ND];
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
#pragma unroll
        for (int db = 0; db < ND; ++db) kta[ts][db] = read_a_rows<D>(kl, 32 * kb, ts, 32 * db, lane);
      f32x16 ds;
      const int kb0 = t * TK + 32 * kb + 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kb0 + 8 * (i >> 2) + (i & 3);
        const bool vis = (kk < kend) & (kk <= klimit);
        const float x = vis ? s[i] * a.c - lse2 : -INFINITY;
        const float pv = __builtin_amdgcn_exp2f(x);
        ds[i] = pv * (dp[i] - dl);
      }
      // dQ^T += K^T.dS^T over the 32 keys (two k-steps)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        const s16x8 sb = pack_b<T>(ds, ts);
#pragma unroll
        for (int db = 0; db < ND; ++db) dqa[db] = T::mma(kta[ts][db], sb, dqa[db]);
      }
      sched_reads_ahead<2 * ND, 3, 1, 2>();
    }
    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // dQ^T: C[dim][query]; lane's row, dims 32db + 8j + 4h .. +3
  if (row_ok) {
    short* dqp = static_cast<short*>(a.dq) + (((int64_t)b * a.Sq + qi) * a.Hq + hq) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s16x4 q4;
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] = T::cvt(a.scale * dqa[db][4 * j + e]);
        *reinterpret_cast<s16x4*>(dqp + 32 * db + 8 * j) = q4;
      }
  }
}

template <typename T, int D>
hipError_t launch_bwd_d(const BwdArgs& in, hipStream_t stream) {
  BwdArgs a = in;
  void* args[] = {&a};
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int rows_per_block = 256 / (D / 8);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_delta_kernel<T, D>),
                                 dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                                 dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const int64_t nkv = (int64_t)a.B * a.Hkv * ((a.Skv + 127) / 128);
  e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkv_kernel<T, D>), dim3((unsigned)nkv),
                      dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const int64_t nq = (int64_t)a.B * a.Hq * ((a.Sq + 127) / 128);
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<T, D>), dim3((unsigned)nq),
                         dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdLaunchArgs& in) {
  BwdArgs a;
  a.q = in.q;
  a.k = in.k;
  a.v = in.v;
  a.o = in.o;
  a.lse = in.lse;
  a.dout = in.dout;
  a.dq = in.dq;
  a.dk = in.dk;
  a.dv = in.dv;
  a.delta = in.delta;
  a.B = in.B;
  a.Sq = in.Sq;
  a.Skv = in.Skv;
  a.Hq = in.Hq;
  a.Hkv = in.Hkv;
  a.causal = in.causal;
  a.scale = in.scale;
  a.c = in.c;
  const bool bf = in.dtype == DType::kBF16;
  if (in.D == 64) return bf ? launch_bwd_d<BF16, 64>(a, in.stream) : launch_bwd_d<F16, 64>(a, in.stream);
  if (in.D == 128) return bf ? launch_bwd_d<BF16, 128>(a, in.stream) : launch_bwd_d<F16, 128>(a, in.stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
