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
    for code in (fa.FA_ERR_INVALID, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP, fa.FA_ERR_WORKSPACE):
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


UNSUPPORTED = [dict(D=96), dict(D=512), dict(D=32), dict(D=16), dict(scale=-0.1),
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


# fa_fwd_plan: the kernel-shape rule on the host, with the expected shapes
# worked out by hand from the rule stated in include/fa.h and the launcher:
# eight waves (512-row items, D = 64 or 128) when B*Hq*ceil(Sq/512) >= compute units and the
# shortest item with a visible key spans >= 3 key tiles of 64; else, with
# D = 128, a workspace and fewer items than compute units, the fewest
# power-of-two key ranges (<= 16) that cover the compute units, reduced until
# every range of the shortest item keeps >= 16 key tiles (>= 64 when
# B*Hq*ceil(Sq/256) already covers the compute units).  The workspace of a
# split is ranges * B*Hq*Sq rows * (D + 1) * 4 bytes.
PLAN_CASES = [
    # B, Sq, Skv, Hq, D, causal, cus, kernel, key_ranges
    (2, 4096, 4096, 32, 128, 1, 256, 1, 1),    # 256 items: eight waves, whole ranges
    (4, 1024, 1024, 16, 128, 0, 256, 0, 1),    # 128 items, 16 key tiles: too short to split
    (1, 1000, 16384, 8, 128, 1, 256, 1, 8),    # 16 items; shortest 249 tiles < 16*16
    (1, 512, 8192, 4, 128, 0, 256, 1, 8),      # 4 items; 128 tiles = 16*8
    (1, 512, 16384, 16, 128, 0, 256, 1, 16),   # 16 items; 256 tiles = 16*16
    (3, 300, 4000, 5, 128, 0, 256, 1, 2),      # 15 items; 63 tiles: only 2 ranges
    (1, 2048, 4096, 32, 128, 1, 256, 0, 1),    # 256 four-wave items; ranges would be < 64 tiles
    (1, 2048, 32768, 32, 128, 1, 256, 1, 2),   # 256 four-wave items; 2 ranges of >= 244 tiles
    (1, 2048, 8192, 16, 128, 1, 256, 1, 4),    # 64 items, 128 four-wave ones; 4 ranges of >= 26 tiles
    (2, 700, 5000, 16, 128, 1, 256, 1, 4),     # 64 items; shortest 76 tiles
    (1, 3000, 2600, 16, 128, 1, 256, 0, 1),    # first keyed tile has 2 key tiles
    (1, 512, 8192, 4, 64, 0, 256, 0, 1),       # D = 64: 4 items, four waves, never split
    (1, 4096, 4096, 32, 64, 1, 256, 1, 1),     # D = 64: 256 items, eight waves
    (1, 4096, 4096, 16, 64, 1, 256, 2, 1),     # D = 64 causal: one round of 256-row items: tile kernel
    (1, 4096, 4096, 16, 64, 0, 256, 0, 1),     # D = 64 non-causal: four waves
    (1, 4096, 4096, 24, 64, 1, 256, 0, 1),     # D = 64 causal, 384 items of 256 rows: four waves
    (1, 512, 8192, 4, 128, 0, 4, 1, 1),        # 4 compute units: 4 items fill them
    (1, 200, 100, 256, 128, 1, 256, 0, 1),     # 256 items of 2 key tiles: four waves
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,D,causal,cus,kernel,ranges", PLAN_CASES)
def test_plan(lib, B, Sq, Skv, Hq, D, causal, cus, kernel, ranges):
    ws = 0 if ranges == 1 else ranges * B * Hq * Sq * (D + 1) * 4
    assert fa.fa_fwd_plan(B, Sq, Skv, Hq, 1, D, causal, cus, True) == (fa.FA_OK, kernel, ranges, ws)


@pytest.mark.parametrize("B,Sq,Skv,Hq,D,causal,cus,kernel,ranges", PLAN_CASES)
def test_plan_without_workspace_never_splits(lib, B, Sq, Skv, Hq, D, causal, cus, kernel, ranges):
    """fa_fwd has no memory for partial results: whole key ranges, on the
    eight-wave kernel only where its 512-row items cover the compute units."""
    st, kern, nr, ws = fa.fa_fwd_plan(B, Sq, Skv, Hq, 1, D, causal, cus, False)
    assert (st, nr, ws) == (fa.FA_OK, 1, 0)
    if ranges == 1:
        assert kern == kernel
    else:
        assert kern == fa.FA_KERNEL_FOUR_WAVE  # split cases have too few 512-row items


# The tile kernels (include/fa.h): head dimension 256, and calls with Sq <= 64
# whose q-heads of one kv-head are packed into rows (keys split over the four
# waves when those rows number at most 32).  With a workspace, key ranges
# double while items * ranges stays below the compute units and the shortest
# item keeps >= 4 (keys) / 8 (rows) tiles of 128 / 64 keys per range, at
# most 64 ranges; the key split doubles once more while items * ranges stays
# below twice the compute units and the ranges keep >= 32 tiles.
TILE_PLAN_CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal, kernel, ranges
    # decode, g = 4: 4 rows, 8 items, 128 tiles of 128 keys -> 32 ranges (8 * 32 = 256)
    (1, 1, 16384, 32, 8, 128, 0, 3, 32),
    # decode, g = 8: 8 items, 256 tiles -> 32 ranges of 8 tiles (too short to double again)
    (1, 1, 32768, 64, 8, 128, 1, 3, 32),
    # decode, 128 items, 256 tiles -> 2 ranges cover the units; 128 tiles each -> 4
    (16, 1, 32768, 32, 8, 128, 1, 3, 4),
    # Sq 64, g = 4: 256 packed rows, 2 row blocks x 8 kv-heads = 16 items; the
    # first block's last query 31 sees 16352 keys = 256 tiles of 64 -> 16 ranges
    (1, 64, 16384, 32, 8, 128, 1, 2, 16),
    # D = 256, 8 blocks of 128 rows x 8 heads = 64 items, first block 2 tiles: no split
    (1, 1000, 1000, 8, 8, 256, 1, 2, 1),
    # D = 256, 8 items, 128 tiles of 64 keys -> 16 ranges of 8 tiles
    (1, 256, 8192, 4, 4, 256, 0, 2, 16),
    # D = 192 (rows padded to 256 in LDS): the same plan as D = 256
    (1, 256, 8192, 4, 4, 192, 0, 2, 16),
    # decode at D = 192: the 4 q-heads of a kv-head packed into one row block
    # (the row split: 128-key tiles of the key split do not fit the LDS),
    # 8 items of 128 tiles -> 16 ranges
    (1, 1, 8192, 32, 8, 192, 1, 2, 16),
    # D = 64 decode, g = 8: 4 items, 32 tiles -> 8 ranges (32 < 4 * 2 * 8)
    (2, 1, 4096, 16, 2, 64, 1, 3, 8),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal,kernel,ranges", TILE_PLAN_CASES)
def test_plan_tile_kernels(lib, B, Sq, Skv, Hq, Hkv, D, causal, kernel, ranges):
    ws = 0 if ranges == 1 else ranges * B * Hq * Sq * (D + 1) * 4
    assert fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, causal, 256, True) == (fa.FA_OK, kernel, ranges, ws)
    assert fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, causal, 256, False) == (fa.FA_OK, kernel, 1, 0)


def test_plan_items_without_keys(lib):
    # Sq = 600, Skv = 100, causal: rows 0..499 see no key, so the first
    # 512-row tile reaches only keys 0..11 (1 key tile): four waves.
    # Sq = 1200, Skv = 100: rows below 1100 see nothing, so tiles 0 and 1
    # have no key and tile 2 ends at key 100 (2 key tiles): four waves.
    assert fa.fa_fwd_plan(1, 600, 100, 256, 256, 128, 1, 256, True) == (fa.FA_OK, 0, 1, 0)
    assert fa.fa_fwd_plan(1, 1200, 100, 256, 256, 128, 1, 256, True) == (fa.FA_OK, 0, 1, 0)
    # Sq = 1200, Skv = 300: tile 0 none (rows < 900 see nothing), tile 1
    # (rows 512..1023) ends at key min(1024 - 900, 300) = 124 (2 tiles);
    # Skv = 1100: tile 0 ends at key 412 (7 tiles): eight waves
    assert fa.fa_fwd_plan(1, 1200, 300, 256, 256, 128, 1, 256, True) == (fa.FA_OK, 0, 1, 0)
    assert fa.fa_fwd_plan(1, 1200, 1100, 256, 256, 128, 1, 256, True) == (fa.FA_OK, 1, 1, 0)


@pytest.mark.parametrize("over,status", [
    (dict(B=0), fa.FA_ERR_INVALID), (dict(Sq=0), fa.FA_ERR_INVALID),
    (dict(Skv=-1), fa.FA_ERR_INVALID), (dict(Hq=0), fa.FA_ERR_INVALID),
    (dict(Hkv=0), fa.FA_ERR_INVALID), (dict(Hkv=3), fa.FA_ERR_INVALID),
    (dict(causal=2), fa.FA_ERR_INVALID), (dict(cus=0), fa.FA_ERR_INVALID),
    (dict(ws=2), fa.FA_ERR_INVALID), (dict(ws=-1), fa.FA_ERR_INVALID),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED), (dict(D=32), fa.FA_ERR_UNSUPPORTED),
    (dict(D=512), fa.FA_ERR_UNSUPPORTED),
])
def test_plan_rejects(lib, over, status):
    a = dict(B=1, Sq=512, Skv=8192, Hq=4, Hkv=2, D=128, causal=0, cus=256, ws=1)
    a.update(over)
    kern, ranges, ws = ctypes.c_int(-7), ctypes.c_int(-7), ctypes.c_size_t(7)
    st = lib.fa_fwd_plan(a["B"], a["Sq"], a["Skv"], a["Hq"], a["Hkv"], a["D"], a["causal"],
                         a["cus"], a["ws"], ctypes.byref(kern), ctypes.byref(ranges),
                         ctypes.byref(ws))
    assert st == status
    assert (kern.value, ranges.value, ws.value) == (-7, -7, 7)  # untouched on error
    # NULL output pointers
    assert lib.fa_fwd_plan(1, 512, 8192, 4, 2, 128, 0, 256, 1, None, None, None) == fa.FA_ERR_INVALID


# fa_fwd_ws: the same checks as fa_fwd, plus the dtype and the workspace
WS = 6 << 40


def _call_ws(dtype=0, ws=WS, ws_bytes=1 << 20, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.fa_fwd_ws(dtype, a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"],
                        a["Skv"], a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"], ws,
                        ws_bytes, 0)


@pytest.mark.parametrize("over", INVALID, ids=[str(x) for x in INVALID])
def test_ws_invalid_arguments(lib, over):
    assert _call_ws(**over) == fa.FA_ERR_INVALID


@pytest.mark.parametrize("over", UNSUPPORTED, ids=[str(x) for x in UNSUPPORTED])
def test_ws_unsupported_arguments(lib, over):
    assert _call_ws(**over) == fa.FA_ERR_UNSUPPORTED


def _call_noalloc(dtype=0, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.fa_fwd_noalloc(dtype, a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"],
                             a["Skv"], a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"], 0)


@pytest.mark.parametrize("over", INVALID + [dict(dtype=2), dict(dtype=-1)],
                         ids=[str(x) for x in INVALID + [dict(dtype=2), dict(dtype=-1)]])
def test_noalloc_invalid_arguments(lib, over):
    assert _call_noalloc(**over) == fa.FA_ERR_INVALID


@pytest.mark.parametrize("over", UNSUPPORTED, ids=[str(x) for x in UNSUPPORTED])
def test_noalloc_unsupported_arguments(lib, over):
    assert _call_noalloc(**over) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("args", [
    dict(dtype=2), dict(dtype=-1),                     # unknown dtype
    dict(ws=WS + 8), dict(ws=WS + 1),                  # workspace not 16-byte aligned
    dict(ws_bytes=0),                                  # a workspace of no bytes
    dict(ws=Q), dict(ws=K - 64), dict(ws=V + 4096),    # overlapping q, k, v
    dict(ws=O + 16), dict(ws=L - 16),                  # overlapping o, lse
])
def test_ws_rejects_bad_workspace(lib, args):
    assert _call_ws(**args) == fa.FA_ERR_INVALID


def test_workload_shapes():
    """bench.py's workloads: a name, or an ad-hoc shape string."""
    import workloads
    assert workloads.get(workloads.HEADLINE.name) is workloads.HEADLINE
    w = workloads.get("2,32,8,4096,8192,128,1,f16")
    assert (w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.causal, w.dtype) == (2, 32, 8, 4096, 8192, 128, True, "f16")
    assert w.name == "causal_b2_hq32_hkv8_sq4096_skv8192_d128_f16"
    for bad in ("nope", "2,32,8,4096,8192,128,2,bf16", "2,32,8,4096,8192,128,1,fp8", "1,2,3"):
        with pytest.raises(ValueError):
            workloads.get(bad)
