"""attention_forward_05_amd -- Python binding of libfa, the gfx950 fused
attention forward library.

This module only marshals arguments: every step of the computation runs in
the HIP kernel behind the C ABI declared in ``include/fa.h``.  The functions
carry the C names (``fa_fwd``, ``fa_fwd_f16``, ``fa_fwd_ws``, ``fa_fwd_plan``,
``fa_strerror``) and take
either torch tensors (their device pointers are passed) or raw integer
addresses.  PyTorch is used for device memory and streams only.

There is no fallback: if ``libfa.so`` is missing or cannot be loaded, or no
GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fa_fwd", "fa_fwd_f16", "fa_fwd_ws", "fa_fwd_noalloc", "fa_fwd_plan", "fa_bwd",
           "attention_bwd", "fa_strerror", "attention",
           "FAError", "library_path", "load", "FA_OK", "FA_ERR_INVALID",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_WORKSPACE", "FA_DTYPE_BF16",
           "FA_DTYPE_F16", "FA_KERNEL_FOUR_WAVE", "FA_KERNEL_EIGHT_WAVE",
           "FA_KERNEL_TILE_ROWS", "FA_KERNEL_TILE_KEYS", "EXPORTED_SYMBOLS"]

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_WORKSPACE = -4
FA_DTYPE_BF16 = 0
FA_DTYPE_F16 = 1
FA_KERNEL_FOUR_WAVE = 0
FA_KERNEL_EIGHT_WAVE = 1
FA_KERNEL_TILE_ROWS = 2
FA_KERNEL_TILE_KEYS = 3

EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_f16", "fa_fwd_ws", "fa_fwd_noalloc", "fa_fwd_plan",
                    "fa_bwd", "fa_strerror")
# bytes of the scratch buffer fa_fwd_noalloc keeps on each device
FA_NOALLOC_SCRATCH_BYTES = 64 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_strerror(status)} (status {status})")


def library_path() -> str:
    return os.path.join(_PKG, "libfa.so")


def load():
    """Load libfa.so (built by ``attention_forward_05_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m attention_forward_05_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("fa_fwd", "fa_fwd_f16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, ctypes.c_float, vp]
        fn.restype = i
    sz = ctypes.c_size_t
    lib.fa_fwd_ws.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, ctypes.c_float, vp,
                              sz, vp]
    lib.fa_fwd_ws.restype = i
    lib.fa_fwd_noalloc.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, ctypes.c_float, vp]
    lib.fa_fwd_noalloc.restype = i
    lib.fa_bwd.argtypes = [i] + [vp] * 9 + [i] * 7 + [ctypes.c_float, vp, sz, vp]
    lib.fa_bwd.restype = i
    ip = ctypes.POINTER(i)
    lib.fa_fwd_plan.argtypes = [i, i, i, i, i, i, i, i, i, ip, ip, ctypes.POINTER(sz)]
    lib.fa_fwd_plan.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, causal, compute_units, with_workspace=False):
    """Host-only query (see include/fa.h): returns (status, kernel,
    key_ranges, workspace_bytes) for these sizes on a device with
    `compute_units` compute units, for fa_fwd (with_workspace False) or
    fa_fwd_ws with a large enough workspace (True); the last three are None
    unless status is FA_OK."""
    kern, ranges, ws = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_size_t(0)
    st = load().fa_fwd_plan(int(B), int(Sq), int(Skv), int(Hq), int(Hkv), int(D), int(causal),
                            int(compute_units), int(bool(with_workspace)), ctypes.byref(kern),
                            ctypes.byref(ranges), ctypes.byref(ws))
    if st != FA_OK:
        return st, None, None, None
    return st, kern.value, ranges.value, ws.value


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, stream):
    fn = getattr(load(), name)
    st = fn(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), int(B), int(Sq),
            int(Skv), int(Hq), int(Hkv), int(D), int(causal), float(scale),
            _stream(stream) if stream != 0 else None)
    return st


def fa_fwd(q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, stream=None) -> int:
    """bf16 forward (see include/fa.h).  Returns the status code.

    ``stream``: None = torch's current stream, 0 = the default (NULL)
    stream, an int = a raw hipStream_t, or a torch.cuda.Stream.
    """
    return _call("fa_fwd", q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, stream)


def fa_fwd_f16(q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, stream=None) -> int:
    """fp16 forward (see include/fa.h).  Returns the status code."""
    return _call("fa_fwd_f16", q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, stream)


def fa_fwd_ws(dtype, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale, workspace,
              workspace_bytes, stream=None) -> int:
    """Forward with a caller-owned workspace for split key ranges (see
    include/fa.h); dtype is FA_DTYPE_BF16 or FA_DTYPE_F16.  Returns the
    status code."""
    st = load().fa_fwd_ws(int(dtype), _addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                          int(B), int(Sq), int(Skv), int(Hq), int(Hkv), int(D), int(causal),
                          float(scale), _addr(workspace), int(workspace_bytes),
                          _stream(stream) if stream != 0 else None)
    return st


def fa_fwd_noalloc(dtype, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, causal, scale,
                   stream=None) -> int:
    """Forward with the library's fixed per-device scratch buffer in place of
    a workspace, for callers that cannot allocate (see include/fa.h).
    Returns the status code."""
    return load().fa_fwd_noalloc(int(dtype), _addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                                 int(B), int(Sq), int(Skv), int(Hq), int(Hkv), int(D),
                                 int(causal), float(scale),
                                 _stream(stream) if stream != 0 else None)


def fa_bwd(dtype, q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Skv, Hq, Hkv, D, causal, scale,
           workspace, workspace_bytes, stream=None) -> int:
    """Backward pass (see include/fa.h).  Returns the status code."""
    return load().fa_bwd(int(dtype), _addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                         _addr(dout), _addr(dq), _addr(dk), _addr(dv), int(B), int(Sq), int(Skv),
                         int(Hq), int(Hkv), int(D), int(causal), float(scale), _addr(workspace),
                         int(workspace_bytes), _stream(stream) if stream != 0 else None)


def attention_bwd(q, k, v, o, lse, dout, causal: bool, scale: float, stream=None):
    """Convenience wrapper: gradients (dq, dk, dv) of the forward on torch
    tensors (q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D], o and dout like q, lse
    [B,Hq,Sq] fp32 from the forward), allocated with torch together with the
    8*B*Hq*Sq-byte workspace.  Raises FAError on a non-zero status."""
    import torch
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if q.dtype == torch.bfloat16:
        dt = FA_DTYPE_BF16
    elif q.dtype == torch.float16:
        dt = FA_DTYPE_F16
    else:
        raise FAError(FA_ERR_UNSUPPORTED, f"attention_bwd: dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        if not t.is_contiguous() or not t.is_cuda:
            raise FAError(FA_ERR_INVALID, f"attention_bwd: {name} must be a contiguous GPU tensor")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(8 * B * Hq * Sq, 16), dtype=torch.uint8, device=q.device)
    if isinstance(stream, torch.cuda.Stream):
        ws.record_stream(stream)
    st = fa_bwd(dt, q, k, v, o, lse, dout, dq, dk, dv, B, Sq, Skv, Hq, Hkv, D, int(bool(causal)),
                scale, ws, ws.numel(), stream)
    if st != FA_OK:
        raise FAError(st, "attention_bwd")
    return dq, dk, dv


def attention(q, k, v, causal: bool, scale: float, with_lse: bool = True, out=None,
              lse=None, stream=None, split: bool = False):
    """Convenience wrapper on torch tensors: q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D]
    (bf16 or fp16, contiguous, on the GPU).  Allocates O (and the fp32 LSE
    [B,Hq,Sq]) with torch unless given, calls the entry point for the dtype
    and raises FAError on a non-zero status.  With split=True the call goes
    through fa_fwd_ws with a torch-allocated workspace of the size
    fa_fwd_plan reports, so that key ranges may be split.  Returns
    (o, lse or None)."""
    import torch
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise FAError(FA_ERR_INVALID, "attention: q, k and v dtypes differ")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise FAError(FA_ERR_INVALID, f"attention: {name} must be a contiguous 4-D GPU tensor")
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise FAError(FA_ERR_INVALID, "attention: k/v shapes do not match q")
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        fn, dt = fa_fwd, FA_DTYPE_BF16
    elif q.dtype == torch.float16:
        fn, dt = fa_fwd_f16, FA_DTYPE_F16
    else:
        raise FAError(FA_ERR_UNSUPPORTED, f"attention: dtype {q.dtype}")
    lse_arg = lse if with_lse else None
    if split:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        st, _, _, nbytes = fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, int(bool(causal)), cus, True)
        if st != FA_OK:
            raise FAError(st, "attention: fa_fwd_plan")
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
        if ws is not None and isinstance(stream, torch.cuda.Stream):
            # torch's allocator may hand the block out again once this
            # function returns: tie its reuse to the stream the call runs on
            ws.record_stream(stream)
        st = fa_fwd_ws(dt, q, k, v, out, lse_arg, B, Sq, Skv, Hq, Hkv, D, int(bool(causal)),
                       scale, ws, nbytes, stream)
    else:
        st = fn(q, k, v, out, lse_arg, B, Sq, Skv, Hq, Hkv, D, int(bool(causal)), scale, stream)
    if st != FA_OK:
        raise FAError(st, "attention")
    return out, (lse if with_lse else None)
