// fa_api.cpp -- the C-ABI entry points of libfa (declared in include/fa.h).
//
// Argument checks follow the split the JAX Pallas FlashAttention3 page draws
// in `_attention_forward`: malformed arguments (shapes that do not agree, a
// q-head count that is not a multiple of the kv-head count) are errors,
// well-formed requests outside what the kernels implement (head dimensions
// other than 64, 128, 192 and 256 here) are "not implemented".  Unlike that page, any
// sequence lengths >= 1 are accepted; the kernel masks ragged tails.
//
// Every check runs before the first HIP call, so invalid calls never touch
// the device.

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"
#include "fa_kernel.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + bytes) and [r, r + rbytes) overlap?
bool overlap(const void* p, uint64_t bytes, const void* r, uint64_t rbytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t b = reinterpret_cast<uintptr_t>(r);
  return a < b + rbytes && b < a + bytes;
}

}  // namespace

namespace fa {

int check_fwd_args(DType dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
                   hipStream_t stream, LaunchArgs* out) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID;
  if (B < 1 || Sq < 1 || Skv < 1 || Hq < 1 || Hkv < 1 || D < 1) return FA_ERR_INVALID;
  if (Hq % Hkv != 0) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!isfinite(scale)) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID;

  // element counts in 64 bits, rejecting overflow
  uint64_t nq_el, nkv_el, nlse;
  if (__builtin_mul_overflow((uint64_t)B, (uint64_t)Sq, &nq_el) ||
      __builtin_mul_overflow(nq_el, (uint64_t)Hq, &nq_el) ||
      __builtin_mul_overflow(nq_el, (uint64_t)D, &nq_el) ||
      __builtin_mul_overflow((uint64_t)B, (uint64_t)Skv, &nkv_el) ||
      __builtin_mul_overflow(nkv_el, (uint64_t)Hkv, &nkv_el) ||
      __builtin_mul_overflow(nkv_el, (uint64_t)D, &nkv_el) ||
      __builtin_mul_overflow((uint64_t)B, (uint64_t)Hq, &nlse) ||
      __builtin_mul_overflow(nlse, (uint64_t)Sq, &nlse) || nq_el > (UINT64_MAX >> 2) ||
      nkv_el > (UINT64_MAX >> 2) || nlse > (UINT64_MAX >> 3))
    return FA_ERR_INVALID;

  // o must not overlap any input (nor lse)
  const uint64_t qb = nq_el * 2, kvb = nkv_el * 2;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kvb) || overlap(o, qb, v, kvb))
    return FA_ERR_INVALID;
  if (lse && overlap(o, qb, lse, nlse * 4)) return FA_ERR_INVALID;

  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  if (scale < 0.0f) return FA_ERR_UNSUPPORTED;
  // Size limits of the kernel's 32-bit address arithmetic and item decoding:
  // query tiles at most 65535; fewer than 2^24 (batch, q-head, query tile)
  // items; one batch slice of q/o below 2 GiB; key tiles below 65536; B*Sq*Hq
  // and B*Skv below 2^31.
  if (fa::query_tiles(Sq) > 65535 || fa::work_items(B, Sq, Hq) >= (1ll << 24)) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)Sq * (uint64_t)Hq * (uint64_t)D * 2u >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * (uint64_t)Sq * (uint64_t)Hq >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * (uint64_t)Skv >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
  if (fa::key_tiles(Skv) >= 65536) return FA_ERR_UNSUPPORTED;
  uint32_t magic;
  if (!fa::group_magic(Hq, Hkv, &magic)) return FA_ERR_UNSUPPORTED;

  // exponent constant: scale * log2(e), folded so that p = exp2(s*c - m*c).
  // A zero (or sub-FLT_MIN) scale is taken as FLT_MIN: every exp2 argument
  // then rounds to 0 in fp32, which is exactly the scale = 0 result, while
  // masked logits (-inf) still map to -inf instead of 0 * inf.
  double cd = (double)scale * 1.4426950408889634074;
  float c = (float)cd;
  if (!(c >= FLT_MIN)) c = FLT_MIN;
  if (!isfinite(c)) return FA_ERR_UNSUPPORTED;

  LaunchArgs& a = *out;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Sq = Sq;
  a.Skv = Skv;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.causal = causal;
  a.c = c;
  a.stream = stream;
  a.ws = nullptr;
  a.ws_bytes = 0;
  return FA_OK;
}

}  // namespace fa

namespace {

// bytes of q/o and of k/v (valid after check_fwd_args succeeded)
void tensor_bytes(const fa::LaunchArgs& a, uint64_t* qb, uint64_t* kvb, uint64_t* lseb) {
  *qb = (uint64_t)a.B * a.Sq * a.Hq * a.D * 2;
  *kvb = (uint64_t)a.B * a.Skv * a.Hkv * a.D * 2;
  *lseb = (uint64_t)a.B * a.Hq * a.Sq * 4;
}

int fwd(fa::DType dtype, const void* q, const void* k, const void* v, void* o, float* lse,
        int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale, void* ws,
        size_t ws_bytes, hipStream_t stream) {
  fa::LaunchArgs a;
  int st = fa::check_fwd_args(dtype, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale,
                              stream, &a);
  if (st != FA_OK) return st;
  if (ws) {
    // the workspace: 16-byte aligned, overlapping none of the tensors
    if (!aligned16(ws) || ws_bytes == 0) return FA_ERR_INVALID;
    uint64_t qb, kvb, lseb;
    tensor_bytes(a, &qb, &kvb, &lseb);
    if (overlap(ws, ws_bytes, q, qb) || overlap(ws, ws_bytes, k, kvb) ||
        overlap(ws, ws_bytes, v, kvb) || overlap(ws, ws_bytes, o, qb) ||
        (lse && overlap(ws, ws_bytes, lse, lseb)))
      return FA_ERR_INVALID;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
  }
  return fa::launch(a);
}

int bwd(fa::DType dtype, const void* q, const void* k, const void* v, const void* o,
        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int Sq, int Skv,
        int Hq, int Hkv, int D, int causal, float scale, void* ws, size_t ws_bytes,
        hipStream_t stream) {
  // the shape, scale and size checks of the forward pass, on q/k/v with dq
  // as its output (dq must not overlap q, k or v)
  fa::LaunchArgs a;
  int st = fa::check_fwd_args(dtype, q, k, v, dq, nullptr, B, Sq, Skv, Hq, Hkv, D, causal, scale,
                              stream, &a);
  if (st != FA_OK) return st;
  if (!o || !lse || !dout || !dk || !dv) return FA_ERR_INVALID;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return FA_ERR_INVALID;
  uint64_t qb, kvb, lseb;
  tensor_bytes(a, &qb, &kvb, &lseb);
  // outputs (dq, dk, dv) overlap neither each other nor any input
  const void* ins[6] = {q, k, v, o, lse, dout};
  const uint64_t in_bytes[6] = {qb, kvb, kvb, qb, lseb, qb};
  void* outs[3] = {dq, dk, dv};
  const uint64_t out_bytes[3] = {qb, kvb, kvb};
  for (int x = 0; x < 3; ++x) {
    for (int y = 0; y < 6; ++y)
      if (overlap(outs[x], out_bytes[x], ins[y], in_bytes[y])) return FA_ERR_INVALID;
    for (int y = x + 1; y < 3; ++y)
      if (overlap(outs[x], out_bytes[x], outs[y], out_bytes[y])) return FA_ERR_INVALID;
  }
  // (D = 64, 128: the generated gradient kernels; 192, 256: the HIP C++ ones)
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  // the generated gradient kernels address one batch slice of k / v with 32 bits
  if ((uint64_t)Skv * (uint64_t)Hkv * (uint64_t)D * 2u >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
  // the workspace holds two fp32 per query row, [2][B][Hq][Sq]: LSE in log2
  // units and delta
  const uint64_t wsb = 2 * lseb;
  if (!ws || ws_bytes < wsb) return FA_ERR_WORKSPACE;
  if (!aligned16(ws)) return FA_ERR_INVALID;
  for (int y = 0; y < 6; ++y)
    if (overlap(ws, wsb, ins[y], in_bytes[y])) return FA_ERR_INVALID;
  for (int x = 0; x < 3; ++x)
    if (overlap(ws, wsb, outs[x], out_bytes[x])) return FA_ERR_INVALID;

  fa::BwdLaunchArgs b;
  b.dtype = dtype;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.lse = lse;
  b.dout = dout;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.ws = static_cast<float*>(ws);
  b.B = B;
  b.Sq = Sq;
  b.Skv = Skv;
  b.Hq = Hq;
  b.Hkv = Hkv;
  b.D = D;
  b.causal = causal;
  b.scale = scale;
  b.c = a.c;
  b.stream = stream;
  return fa::launch_bwd(b);
}

}  // namespace

extern "C" {

int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int Sq,
           int Skv, int Hq, int Hkv, int D, int causal, float scale, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID;
  return bwd(dtype == FA_DTYPE_BF16 ? fa::DType::kBF16 : fa::DType::kF16, q, k, v, o, lse, dout,
             dq, dk, dv, B, Sq, Skv, Hq, Hkv, D, causal, scale, workspace, workspace_bytes,
             stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
           int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
           hipStream_t stream) {
  return fwd(fa::DType::kBF16, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, nullptr,
             0, stream);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
               hipStream_t stream) {
  return fwd(fa::DType::kF16, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, nullptr,
             0, stream);
}

int fa_fwd_ws(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID;
  return fwd(dtype == FA_DTYPE_BF16 ? fa::DType::kBF16 : fa::DType::kF16, q, k, v, o, lse, B, Sq,
             Skv, Hq, Hkv, D, causal, scale, workspace, workspace_bytes, stream);
}

int fa_fwd_plan(int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, int compute_units,
                int with_workspace, int* kernel, int* key_ranges, size_t* workspace_bytes) {
  if (!kernel || !key_ranges || !workspace_bytes) return FA_ERR_INVALID;
  if (B < 1 || Sq < 1 || Skv < 1 || Hq < 1 || Hkv < 1 || D < 1 || compute_units < 1)
    return FA_ERR_INVALID;
  if (Hq % Hkv != 0) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (with_workspace != 0 && with_workspace != 1) return FA_ERR_INVALID;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  const fa::Plan p =
      fa::make_plan(B, Sq, Skv, Hq, Hkv, D, causal, compute_units, with_workspace != 0);
  *kernel = p.kernel;
  *key_ranges = p.ranges;
  *workspace_bytes = p.ws_bytes;
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK:
      return "success";
    case FA_ERR_INVALID:
      return "invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "unsupported argument (D must be 64, 128, 192 or 256, scale >= 0, sizes within the kernel's limits)";
    case FA_ERR_HIP:
      return "HIP runtime error at kernel launch";
    case FA_ERR_WORKSPACE:
      return "workspace too small for the split key ranges of this call: fa_fwd_ws's workspace, or "
             "fa_fwd_noalloc's fixed 64 MiB scratch buffer (fa_fwd_plan gives the bytes needed)";
    default:
      return "unknown fa_status";
  }
}

}  // extern "C"
