"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
public header declares, and rejects every invalid argument before any HIP
call (so these run without a GPU; no valid call is made here)."""
import ctypes
import os
import re

import pytest

import attention_forward_05_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        from attention_forward_05_amd import build
        build.build()
    return fa.load()


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and as dynamic symbols of the shared object (nm -D)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name


def test_strerror(lib):
    assert fa.fa_strerror(fa.FA_OK) == "success"
    for code in (fa.FA_ERR_INVALID, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        s = fa.fa_strerror(code)
        assert s and s != "unknown fa_status"
    assert fa.fa_strerror(12345) == "unknown fa_status"


# Fake, 16-byte-aligned, far-apart device addresses: validation rejects the
# call before any of them could be dereferenced.
Q, K, V, O, L = (1 << 40), (2 << 40), (3 << 40), (4 << 40), (5 << 40)
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, Sq=128, Skv=128, Hq=4, Hkv=2, D=128,
            causal=1, scale=0.088)


def _call(fn, **over):
    a = dict(GOOD)
    a.update(over)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"], a["Skv"],
              a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"], 0)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(B=0), dict(Sq=0), dict(Skv=0), dict(Hq=0), dict(Hkv=0), dict(D=0),
    dict(B=-1), dict(Sq=-5),
    dict(Hq=3, Hkv=2), dict(Hq=4, Hkv=8),
    dict(causal=2), dict(causal=-1),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=float("-inf")),
    dict(q=Q + 8), dict(k=K + 2), dict(v=V + 4), dict(o=O + 1), dict(lse=L + 2),
    dict(o=Q), dict(o=K + 256), dict(o=V), dict(lse=O + 64),
    dict(B=2**31 - 1, Sq=2**31 - 1, Hq=2**31 - 1, Hkv=1, D=128),
]


@pytest.mark.parametrize("over", INVALID, ids=[str(x) for x in INVALID])
@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f16"])
def test_invalid_arguments(lib, entry, over):
    assert _call(getattr(fa, entry), **over) == fa.FA_ERR_INVALID


UNSUPPORTED = [dict(D=96), dict(D=256), dict(D=32), dict(D=16), dict(scale=-0.1),
               dict(scale=3e38),
               # 2^24 (batch, q-head, query tile) items: beyond the item decoding
               dict(B=16384, Sq=1, Skv=1, Hq=1024, Hkv=1),
               # 65536 key tiles of 64 keys
               dict(Skv=65536 * 64),
               # 65536 query tiles of 256 rows (and a 2 GiB q slice)
               dict(Sq=65536 * 256, Hq=1, Hkv=1, D=64)]


@pytest.mark.parametrize("over", UNSUPPORTED, ids=[str(x) for x in UNSUPPORTED])
@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f16"])
def test_unsupported_arguments(lib, entry, over):
    assert _call(getattr(fa, entry), **over) == fa.FA_ERR_UNSUPPORTED


def test_python_wrapper_raises_on_bad_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.attention(q, q, q, True, 0.125)  # CPU tensors are refused before any call
