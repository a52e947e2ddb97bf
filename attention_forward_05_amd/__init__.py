"""attention_forward_05_amd -- Python binding of libfa, the gfx950 fused
attention forward library.

This module only marshals arguments: every step of the computation runs in
the HIP kernel behind the C ABI declared in ``include/fa.h``.  The functions
carry the C names (``fa_fwd``, ``fa_fwd_f16``, ``fa_fwd_plan``, ``fa_strerror``) and take
either torch tensors (their device pointers are passed) or raw integer
addresses.  PyTorch is used for device memory and streams only.

There is no fallback: if ``libfa.so`` is missing or cannot be loaded, or no
GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fa_fwd", "fa_fwd_f16", "fa_fwd_plan", "fa_strerror", "attention", "FAError",
           "library_path", "load", "FA_OK", "FA_ERR_INVALID",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_KERNEL_FOUR_WAVE",
           "FA_KERNEL_EIGHT_WAVE", "EXPORTED_SYMBOLS"]

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_KERNEL_FOUR_WAVE = 0
FA_KERNEL_EIGHT_WAVE = 1

EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_f16", "fa_fwd_plan", "fa_strerror")

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
            f"{path} is missing: build it with `python -m attention_forward_05_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("fa_fwd", "fa_fwd_f16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, ctypes.c_float, vp]
        fn.restype = i
    ip = ctypes.POINTER(i)
    lib.fa_fwd_plan.argtypes = [i, i, i, i, i, i, i, ip, ip]
    lib.fa_fwd_plan.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def fa_fwd_plan(B, Sq, Skv, Hq, D, causal, compute_units):
    """Host-only query (see include/fa.h): returns (status, kernel,
    key_ranges) for these sizes on a device with `compute_units` compute
    units; kernel and key_ranges are None unless status is FA_OK."""
    kern, ranges = ctypes.c_int(-1), ctypes.c_int(-1)
    st = load().fa_fwd_plan(int(B), int(Sq), int(Skv), int(Hq), int(D), int(causal),
                            int(compute_units), ctypes.byref(kern), ctypes.byref(ranges))
    if st != FA_OK:
        return st, None, None
    return st, kern.value, ranges.value


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


def attention(q, k, v, causal: bool, scale: float, with_lse: bool = True, out=None,
              lse=None, stream=None):
    """Convenience wrapper on torch tensors: q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D]
    (bf16 or fp16, contiguous, on the GPU).  Allocates O (and the fp32 LSE
    [B,Hq,Sq]) with torch unless given, calls the entry point for the dtype
    and raises FAError on a non-zero status.  Returns (o, lse or None)."""
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
        fn = fa_fwd
    elif q.dtype == torch.float16:
        fn = fa_fwd_f16
    else:
        raise FAError(FA_ERR_UNSUPPORTED, f"attention: dtype {q.dtype}")
    st = fn(q, k, v, out, lse if with_lse else None, B, Sq, Skv, Hq, Hkv, D,
            int(bool(causal)), scale, stream)
    if st != FA_OK:
        raise FAError(st, "attention")
    return out, (lse if with_lse else None)
