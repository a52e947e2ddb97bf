"""fa_fwd_noalloc (the entry point for callers that cannot allocate) against
fa_fwd_ws, the entry point it varies: the same kernels, so the same bits.

Two split calls in a row, the second smaller than the first (the scratch
buffer keeps the first call's partial results, which must not leak into the
second), a call that does not split, and a call whose split needs more than
the scratch buffer holds (refused, nothing enqueued)."""
import math

import pytest
import torch

import attention_forward_05_amd as fa
import workloads

pytestmark = pytest.mark.gpu


def _inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed):
    dev = torch.device("cuda:0")
    return [t.to(dev) for t in workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed)]


def _run(entry, dtype, q, k, v, causal, scale):
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), device=q.device)
    dt = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F16
    if entry == "noalloc":
        st = fa.fa_fwd_noalloc(dt, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, int(causal), scale)
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        _, _, _, nbytes = fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, int(causal), cus, True)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = fa.fa_fwd_ws(dt, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, int(causal), scale,
                          ws if nbytes else None, nbytes)
    torch.cuda.synchronize()
    return st, o, lse


def _ranges(B, Sq, Skv, Hq, Hkv, D, causal):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st, _, nr, nbytes = fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, int(causal), cus, True)
    assert st == fa.FA_OK
    return nr, nbytes


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    fa.load()


def test_noalloc_matches_workspace_entry_two_calls():
    """A large split call then a smaller one, each against fa_fwd_ws."""
    shapes = [
        # B, Sq, Skv, Hq, Hkv, D, causal, dtype
        (1, 1, 32768, 64, 8, 128, True, "bf16"),    # decode, many key ranges
        (1, 4, 4096, 32, 8, 128, False, "f16"),     # smaller: fewer rows and ranges
    ]
    sizes = []
    for n, (B, Sq, Skv, Hq, Hkv, D, causal, dtype) in enumerate(shapes):
        nr, nbytes = _ranges(B, Sq, Skv, Hq, Hkv, D, causal)
        assert nr > 1 and 0 < nbytes <= fa.FA_NOALLOC_SCRATCH_BYTES
        sizes.append(nbytes)
        q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, dtype, 500 + n)
        scale = 1.0 / math.sqrt(D)
        st1, o1, l1 = _run("noalloc", dtype, q, k, v, causal, scale)
        st2, o2, l2 = _run("ws", dtype, q, k, v, causal, scale)
        assert st1 == fa.FA_OK and st2 == fa.FA_OK
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {n}"
    assert sizes[1] < sizes[0]


def test_noalloc_without_split_and_eight_wave_split():
    """A call that does not split (the scratch is not touched) and a split
    on the eight-wave kernel, both bit-equal to fa_fwd_ws."""
    for n, (B, Sq, Skv, Hq, Hkv, D, causal, dtype) in enumerate([
            (1, 300, 300, 4, 2, 64, True, "bf16"),
            (1, 512, 8192, 4, 4, 128, False, "bf16")]):
        q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, dtype, 600 + n)
        st1, o1, l1 = _run("noalloc", dtype, q, k, v, causal, 0.1)
        st2, o2, l2 = _run("ws", dtype, q, k, v, causal, 0.1)
        assert st1 == fa.FA_OK and st2 == fa.FA_OK
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_refuses_split_beyond_scratch():
    """A split needing more than the scratch buffer: FA_ERR_WORKSPACE and the
    outputs untouched."""
    B, Sq, Skv, Hq, Hkv, D = 1, 1024, 32768, 8, 1, 128
    nr, nbytes = _ranges(B, Sq, Skv, Hq, Hkv, D, True)
    if nbytes <= fa.FA_NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"this device splits into {nr} ranges, {nbytes} bytes: within the scratch")
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, "bf16", 700)
    o = torch.full_like(q, 3.0)
    lse = torch.full((B, Hq, Sq), 3.0, device=q.device)
    st = fa.fa_fwd_noalloc(fa.FA_DTYPE_BF16, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, 1, 0.088)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_WORKSPACE
    assert torch.all(o == 3.0) and torch.all(lse == 3.0)
