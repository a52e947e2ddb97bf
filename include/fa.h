/*
 * fa.h -- libfa: fused attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * Computes, for every batch b, query head hq and query row i,
 *
 *     O[b,i,hq,:] = sum_j softmax_j( scale * Q[b,i,hq,:] . K[b,j,hk,:] ) * V[b,j,hk,:]
 *     LSE[b,hq,i] = ln sum_j exp( scale * Q[b,i,hq,:] . K[b,j,hk,:] )
 *
 * over the visible keys j, with hk = hq / (Hq / Hkv) (grouped-query heads:
 * each kv-head serves a contiguous group of Hq/Hkv query heads).
 *
 * The operation is the one every page on the tiled online-softmax ("flash")
 * attention forward pass implements: the JAX Pallas Mosaic-GPU
 * FlashAttention3 page (`attention_reference` gives the definition; `kv_loop`
 * the running max m, running sum l and rescaled accumulator; its
 * `_memory_wg` maps q-head to kv-head by integer division), the Croqtile
 * tutorial's non-persistent `flash_atten` (scale folded into an exp2
 * exponent, causal tiles) and the kernbench GQA prefill page
 * (`_merge_running`, the online-softmax merge of partial (m, l, O) triples).
 *
 * Masking: with causal = 0 every key 0 <= j < Skv is visible.  With
 * causal = 1 the mask is aligned bottom-right: key j is visible from query i
 * iff j <= i + (Skv - Sq).  When Sq == Skv this is the pages' j <= i.  A row
 * with no visible key (only possible when Sq > Skv) gets O = 0, LSE = -inf.
 *
 * LSE is the natural-log log-sum-exp of the scaled logits (the JAX page
 * stores the base-2 value m*log2(e) + log2(l); multiply ours by log2(e) to
 * get it).
 *
 * Arithmetic: both products on MFMA with fp32 accumulation; the softmax in
 * fp32 with hardware exp2; the probabilities are rounded to the input dtype
 * (round-to-nearest-even) before the second product; O is rounded once to
 * the input dtype at the end.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every argument check runs on the host before any HIP call,
 * so an invalid call returns without touching the device. */
typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,     /* bad argument: NULL pointer, size < 1, Hq % Hkv != 0,
                              causal not 0/1, scale not finite, pointer not
                              16-byte aligned, o overlapping q/k/v, a workspace
                              overlapping a tensor, size overflow, unknown dtype */
  FA_ERR_UNSUPPORTED = -2, /* valid but not implemented: D not 64, 128, 192 or 256,
                              scale < 0, sizes beyond the kernel's limits
                              (ceil(Sq/256) at most 65535, B*Hq*ceil(Sq/256)
                              below 2^24, ceil(Skv/64) below 65536,
                              Sq*Hq*D*2 bytes, B*Sq*Hq and B*Skv below 2^31) */
  FA_ERR_HIP = -3,         /* the HIP runtime reported an error loading the
                              kernels or at launch */
  FA_ERR_WORKSPACE = -4    /* the call splits its key ranges and the workspace
                              given (or fa_fwd_noalloc's scratch buffer) is
                              smaller than fa_fwd_plan reports */
} fa_status;

/* Element types of q, k, v and o for the entry points that take a dtype. */
enum { FA_DTYPE_BF16 = 0, FA_DTYPE_F16 = 1 };

/*
 * fa_fwd -- bf16 inputs and output.
 *
 *   q    : device pointer, [B, Sq, Hq, D] bf16, contiguous (row-major, "BSHD")
 *   k, v : device pointers, [B, Skv, Hkv, D] bf16, contiguous
 *   o    : device pointer, [B, Sq, Hq, D] bf16, written; must not overlap q, k or v
 *   lse  : device pointer, [B, Hq, Sq] fp32, written; may be NULL (not written)
 *   B, Sq, Skv, Hq, Hkv : sizes >= 1, Hq a multiple of Hkv
 *   D    : head dimension, 64, 128, 192 or 256
 *   causal : 0 (no mask) or 1 (bottom-right aligned causal mask)
 *   scale  : multiplies the logits before the softmax; finite and >= 0
 *            (usually 1/sqrt(D))
 *   stream : HIP stream to enqueue on (NULL = the default stream)
 *
 * All pointers are owned by the caller and must be 16-byte aligned.  The
 * library allocates no device memory.  The only state it keeps is its
 * kernel code and the device's compute-unit count: the first call on a
 * device loads the library's gfx950 code object on that device (under a
 * lock, so concurrent first calls are safe) and keeps it until the process
 * ends; a failed load returns FA_ERR_HIP.  Calls on different streams may
 * run concurrently.  The call is asynchronous: it returns once its kernel is
 * enqueued, and o / lse are valid after the stream has been synchronised.
 *
 * fa_fwd never splits an item's key range (it has no memory for partial
 * results); fa_fwd_ws does, given a workspace.
 *
 * Returns FA_OK or one of the error codes above.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal,
           float scale, hipStream_t stream);

/* fa_fwd_f16 -- identical to fa_fwd, with fp16 q, k, v and o. */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o,
               float* lse, int B, int Sq, int Skv, int Hq, int Hkv, int D,
               int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_ws -- the forward pass with a caller-owned workspace for split key
 * ranges; dtype is FA_DTYPE_BF16 or FA_DTYPE_F16, the other arguments are
 * those of fa_fwd.
 *
 * When a call's work items are fewer than the device's compute units and
 * every item's key range is long, each item's keys are cut into 2, 4, 8, 16,
 * 32 or 64 ranges: the one-device form of the kernbench GQA prefill page's
 * split of the key sequence over PE groups.
 * Each range's partial result (fp32 O normalised over the range's keys and
 * the range's LSE, 4*(D+1) bytes per query row and range) goes to the
 * workspace, and a second kernel on the same stream merges them into o and
 * lse (that page's `_merge_running`).  fa_fwd_plan reports the number of
 * ranges and the workspace bytes the call needs.
 *
 *   workspace       : device memory, 16-byte aligned, overlapping no tensor
 *                     of the call; or NULL: then the call never splits and
 *                     behaves exactly as fa_fwd / fa_fwd_f16.
 *   workspace_bytes : its size in bytes (> 0 when workspace is not NULL).
 *
 * The workspace's contents are undefined after the call; it is in use until
 * the stream passes the call, so calls that run concurrently need distinct
 * workspaces.  A call that splits with workspace_bytes smaller than it needs
 * returns FA_ERR_WORKSPACE before enqueueing anything.
 */
int fa_fwd_ws(int dtype, const void* q, const void* k, const void* v, void* o,
              float* lse, int B, int Sq, int Skv, int Hq, int Hkv, int D,
              int causal, float scale, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/* Bytes of the scratch buffer fa_fwd_noalloc keeps on each device (64 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * fa_fwd_noalloc -- for callers that cannot allocate device memory around
 * the call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the forward pass of fa_fwd_ws, with the library's own
 * scratch buffer of FA_NOALLOC_SCRATCH_BYTES in place of a caller workspace.
 * dtype and the other arguments are those of fa_fwd_ws.
 *
 * The buffer is a device array of the library, one per device, held from the
 * load of the library's device code until the process ends.  The call
 * allocates nothing.  The first call of any entry point on a device loads the
 * library's kernel code there (the HIP runtime allocates for that), so make
 * one call on each device before code that must not allocate.
 *
 * Calls that split their key ranges use the buffer for the partial results
 * and return FA_ERR_WORKSPACE, before enqueueing anything, when the split
 * needs more than FA_NOALLOC_SCRATCH_BYTES (fa_fwd_plan with
 * with_workspace = 1 reports the bytes).  All calls on one device share its
 * buffer, whose contents persist from call to call: two split calls whose
 * kernels overlap on one device (different streams, no ordering between
 * them) race on it and give undefined results.  Calls on one stream are
 * ordered and safe.
 */
int fa_fwd_noalloc(int dtype, const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Sq, int Skv, int Hq, int Hkv, int D,
                   int causal, float scale, hipStream_t stream);

/*
 * fa_bwd -- the backward pass: the gradients dQ, dK, dV of a scalar loss
 * given its gradient dO with respect to the forward output, for the
 * forward these arguments describe.  It follows the JAX Pallas
 * FlashAttention3 page's backward (`_attention_bwd`: delta = rowsum(O * dO);
 * `kernel_dq`: P = exp(scale*q.k - LSE), dP = dO.V^T, dS = P * (dP - delta),
 * dQ = scale * dS.K; `kernel_dkv`: dK = scale * dS^T.Q, dV = P^T.dO, dK and
 * dV of a kv-head summed over the q-heads of its group), with this
 * library's scale and natural-log LSE.  P and dS are rounded to the input
 * dtype before the products that read them, as that page casts them; the
 * gradients are accumulated in fp32 and rounded once.  With causal = 1 the
 * forward's bottom-right mask applies (masked pairs have P = 0); that page
 * has no causal backward.
 *
 *   dtype       : FA_DTYPE_BF16 or FA_DTYPE_F16 (q, k, v, o, dout, dq, dk, dv)
 *   q, k, v     : the forward's inputs (layouts as in fa_fwd)
 *   o, lse      : the forward's outputs, o [B,Sq,Hq,D], lse [B,Hq,Sq] fp32
 *                 (natural log, as fa_fwd writes it; -inf for rows without a
 *                 visible key, which then get dQ = 0)
 *   dout        : dL/dO, [B,Sq,Hq,D]
 *   dq          : written, [B,Sq,Hq,D]
 *   dk, dv      : written, [B,Skv,Hkv,D]
 *   B .. scale  : as in fa_fwd; D = 64, 128, 192 or 256
 *   workspace   : device memory of at least 8*B*Hq*Sq bytes, 16-byte aligned
 *                 (two fp32 per query row: LSE in log2 units and delta);
 *                 contents undefined after
 *   stream      : HIP stream to enqueue on
 *
 * dq, dk, dv and the workspace must overlap neither each other nor any
 * input.  Asynchronous like fa_fwd; the library allocates nothing.  Returns
 * FA_OK, FA_ERR_INVALID (as fa_fwd, plus NULL o/lse/dout/dk/dv and the
 * overlaps above), FA_ERR_UNSUPPORTED (D not 64, 128, 192 or 256, one batch slice of
 * k or v of 2 GiB or more, and fa_fwd's limits), FA_ERR_WORKSPACE
 * (workspace NULL or smaller than 8*B*Hq*Sq bytes) or FA_ERR_HIP.
 */
int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
           int Sq, int Skv, int Hq, int Hkv, int D, int causal, float scale,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Kernel shapes reported by fa_fwd_plan. */
enum {
  FA_KERNEL_FOUR_WAVE = 0,  /* 256-row query tiles, one wave per SIMD (D = 64, 128) */
  FA_KERNEL_EIGHT_WAVE = 1, /* 512-row query tiles, two waves per SIMD (D = 64, 128) */
  FA_KERNEL_TILE_ROWS = 2,  /* 128-row blocks, four waves over the rows: D = 192, 256;
                               calls with Sq <= 64 whose q-heads of one
                               kv-head make more than 32 rows together; and
                               causal D = 64 calls without enough 512-row
                               tiles for the eight-wave kernel whose 256-row
                               tiles fit in one round on the compute units */
  FA_KERNEL_TILE_KEYS = 3   /* one 32-row block, four waves over the keys: calls
                               with Sq <= 64 and Sq * Hq / Hkv <= 32 (decode) */
};
/* With Sq <= 64 the rows of an item are (query, q-head)
 * pairs of the q-heads of one kv-head, so K and V are read once per kv-head. */

/*
 * fa_fwd_plan -- host-only query (no HIP call): what a forward call of these
 * sizes does on a device with `compute_units` compute units (256 on an
 * MI355X).  with_workspace = 0 gives the plan of fa_fwd / fa_fwd_f16 (and of
 * fa_fwd_ws without a workspace), 1 that of fa_fwd_ws with a large enough
 * workspace.
 *
 *   kernel          : written, one of FA_KERNEL_*
 *   key_ranges      : written, 1 (whole key ranges) or 2 .. 64, a power of
 *                     two (split key ranges merged by a second kernel)
 *   workspace_bytes : written, the workspace the split needs (0 without one)
 *
 * Returns FA_OK, FA_ERR_INVALID (NULL output pointer, size or compute_units
 * < 1, Hq % Hkv != 0, causal or with_workspace not 0/1) or
 * FA_ERR_UNSUPPORTED (D not 64, 128, 192 or 256); the outputs are written only on
 * FA_OK.  Size limits of fa_fwd are not checked here.
 */
int fa_fwd_plan(int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal,
                int compute_units, int with_workspace, int* kernel,
                int* key_ranges, size_t* workspace_bytes);

/* fa_strerror -- a static, NUL-terminated description of a status code
 * (never NULL; unknown codes give "unknown fa_status"). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
