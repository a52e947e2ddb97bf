"""CPU oracle for the fused attention forward pass -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the ``attention_forward_05_amd``
package and its HIP library) never does, and the two share no code.

The arithmetic lives in ``oracle.c`` (fp64, two passes per row); this module
builds it with gcc, loads it with ctypes and widens the inputs to float64.
Widening bf16 or fp16 to float64 is exact, so the oracle sees the same input
bits as the GPU path.

Readings of the pages (each one is also listed with its reason in the design
notes):

* LSE base: the JAX Pallas FlashAttention3 page stores ``m*log2(e) + log2(l)``
  (base 2, its ``attention_reference`` residual).  The operation asked for is
  the log-sum-exp of a row, read here as the natural log: ``m + ln(l)``.  The
  two differ by the factor log2(e); a test checks the identity.
* LSE of the *scaled* logits ``scale * q.k`` (the Croqtile page folds the
  scale into the exponent, so its max and sum are of scaled logits).
* Causal mask aligned bottom-right: key j visible from query i iff
  ``j <= i + (Skv - Sq)``; equal to the pages' top-left mask when Sq == Skv.
* A row with no visible key: O = 0, LSE = -inf.
* Grouped-query heads: q-head ``hq`` reads kv-head ``hq // (Hq // Hkv)``
  (contiguous groups, the JAX page's ``lax.div`` and its
  (B, Sq, Hkv, Hq/Hkv, D) reshape).

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, invariants and independent library formulations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP).

    -ffp-contract=off keeps every product and sum a separately rounded fp64
    operation, exactly as written in the source.
    """
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def use_library(path):
    """Point this module at another build of oracle.c (the mutation tests load
    deliberately broken copies).  Returns the previous library handle;
    ``restore_library`` puts it back."""
    global _lib
    old = _load()
    _lib = _configure(ctypes.CDLL(path))
    return old


def restore_library(handle) -> None:
    global _lib
    _lib = handle


def _configure(lib):
    lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp] + [_i64] * 6 + [
        ctypes.c_int, ctypes.c_double]
    lib.oracle_attn_fwd.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [_dp, _dp, _dp] + [_i64] * 6 + [
        ctypes.c_int, ctypes.c_double, _lp, _i64, _dp, _dp]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_partial.argtypes = [_dp, _dp, _dp] + [_i64] * 6 + [
        ctypes.c_int, ctypes.c_double, _i64, _i64, _dp, _dp, _dp]
    lib.oracle_attn_partial.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp,
                                 _dp, _dp, _dp]
    lib.oracle_merge.restype = None
    lib.oracle_attn_bwd.argtypes = [_dp] * 7 + [_i64] * 6 + [ctypes.c_int, ctypes.c_double]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd_rows.argtypes = [_dp] * 4 + [_i64] * 6 + [ctypes.c_int, ctypes.c_double,
                                          _lp, _i64, _dp, _lp, _i64, _dp, _dp]
    lib.oracle_attn_bwd_rows.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    """Widen a torch tensor or array-like to a contiguous float64 array."""
    if hasattr(x, "detach"):  # torch tensor (CPU)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def set_threads(n: int) -> None:
    """Threads for the OpenMP row loop (0 = OpenMP default)."""
    _load().oracle_set_threads(int(n))


def threads() -> int:
    return int(_load().oracle_threads())


def _dims(q, k):
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    return B, Sq, Skv, Hq, Hkv, D


def attn_fwd(q, k, v, causal: bool, scale: float):
    """Full forward.  q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] -> (o [B,Sq,Hq,D], lse [B,Hq,Sq]) in float64."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Skv, Hq, Hkv, D = _dims(q, k)
    if v.shape != k.shape:
        raise ValueError("v shape must equal k shape")
    o = np.empty((B, Sq, Hq, D), np.float64)
    lse = np.empty((B, Hq, Sq), np.float64)
    rc = lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, Sq, Skv, Hq, Hkv, D, int(bool(causal)), float(scale))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd failed ({rc})")
    return o, lse


def attn_bwd(q, k, v, dout, causal: bool, scale: float):
    """Gradients of the forward pass for an upstream gradient dout = dL/dO
    [B,Sq,Hq,D] -> (dq [B,Sq,Hq,D], dk [B,Skv,Hkv,D], dv [B,Skv,Hkv,D]) in
    float64.  The textbook softmax gradient with the JAX page's
    delta = rowsum(O * dO) (see oracle.c, oracle_attn_bwd); dK and dV of a
    kv-head are summed over its q-heads."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Skv, Hq, Hkv, D = _dims(q, k)
    if v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("v must match k and dout must match q")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                             B, Sq, Skv, Hq, Hkv, D, int(bool(causal)), float(scale))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed ({rc})")
    return dq, dk, dv


def attn_bwd_rows(q, k, v, dout, causal: bool, scale: float, qrows, krows):
    """Selected gradients: dQ of the query rows qrows (int [nq, 3] of
    (b, hq, i)) and dK, dV of the key rows krows (int [nk, 3] of (b, hk, j))
    -> (dq [nq, D], dk [nk, D], dv [nk, D]) in float64, the same arithmetic
    as attn_bwd."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Skv, Hq, Hkv, D = _dims(q, k)
    qrows = np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1, 3))
    krows = np.ascontiguousarray(np.asarray(krows, dtype=np.int64).reshape(-1, 3))
    nq, nk = qrows.shape[0], krows.shape[0]
    dq = np.empty((nq, D), np.float64)
    dk = np.empty((nk, D), np.float64)
    dv = np.empty((nk, D), np.float64)
    rc = lib.oracle_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Sq, Skv, Hq, Hkv, D,
                                  int(bool(causal)), float(scale), qrows.ctypes.data_as(_lp), nq,
                                  _ptr(dq), krows.ctypes.data_as(_lp), nk, _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_rows failed ({rc})")
    return dq, dk, dv


def attn_rows(q, k, v, causal: bool, scale: float, rows):
    """Selected rows.  rows: int array [n, 3] of (b, hq, i) -> (o [n, D], lse [n])."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Skv, Hq, Hkv, D = _dims(q, k)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib.oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D,
                              int(bool(causal)), float(scale),
                              rows.ctypes.data_as(_lp), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows failed ({rc})")
    return o, lse


def attn_partial(q, k, v, causal: bool, scale: float, j_lo: int, j_hi: int):
    """Unnormalized (m, l, acc) of every row over keys [j_lo, j_hi).

    m, l: [B,Hq,Sq]; acc: [B,Sq,Hq,D].
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Skv, Hq, Hkv, D = _dims(q, k)
    m = np.empty((B, Hq, Sq), np.float64)
    l = np.empty((B, Hq, Sq), np.float64)
    acc = np.empty((B, Sq, Hq, D), np.float64)
    rc = lib.oracle_attn_partial(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D,
                                 int(bool(causal)), float(scale), int(j_lo), int(j_hi),
                                 _ptr(m), _ptr(l), _ptr(acc))
    if rc != 0:
        raise ValueError(f"oracle_attn_partial failed ({rc})")
    return m, l, acc


def merge(m1, l1, acc1, m2, l2, acc2):
    """Merge two partial triples of n rows (m, l: [n]; acc: [n, D])."""
    lib = _load()
    m1, l1, acc1 = _f64(m1).ravel(), _f64(l1).ravel(), _f64(acc1)
    m2, l2, acc2 = _f64(m2).ravel(), _f64(l2).ravel(), _f64(acc2)
    n = m1.shape[0]
    acc1 = acc1.reshape(n, -1)
    acc2 = np.ascontiguousarray(acc2.reshape(n, -1))
    D = acc1.shape[1]
    m = np.empty(n, np.float64)
    l = np.empty(n, np.float64)
    acc = np.empty((n, D), np.float64)
    lib.oracle_merge(n, D, _ptr(m1), _ptr(l1), _ptr(acc1), _ptr(m2), _ptr(l2),
                     _ptr(acc2), _ptr(m), _ptr(l), _ptr(acc))
    return m, l, acc
