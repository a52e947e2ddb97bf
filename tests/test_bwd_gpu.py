"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 oracle's gradients (oracle.attn_bwd), on the same rounded inputs.

The GPU path starts from its own forward (fa_fwd's O and LSE), as a caller
does.  The bar comes from its arithmetic: P and dS are rounded to the input
dtype (unit roundoff u = 2^-8 bf16, 2^-11 fp16) before the products that read
them, delta is formed from the rounded O, and each gradient is rounded once.
Every gradient element is a sum whose terms carry at most two such roundings
plus the final one, and the rounding errors of different terms are
independent, so the error of a gradient stays a few u of the gradient's own
size: per tensor, rms(dG)/rms(G) <= 4u and max|dG|/max|G| <= 16u.  A
missing or wrong term (mask, scale, GQA sum, sign) moves the gradient by an
O(1) fraction and fails by orders of magnitude, most sharply in fp16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import attention_forward_05_amd as m
    m.load()
    return m


def _inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed, boost=0.0):
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed, k_row_boost_frac=boost)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn((B, Sq, Hq, D), generator=g, dtype=torch.float32).to(q.dtype)
    return q, k, v, do


def run_bwd(fa, q, k, v, do, causal, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, causal, scale)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    return [t.cpu().double().numpy() for t in (dq, dk, dv)]


def check_grads(got, ref, dtype, what):
    u = U[dtype]
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        d = np.abs(g - r)
        rms_r = math.sqrt(float((r * r).mean()))
        max_r = float(np.abs(r).max())
        if max_r == 0.0:
            assert d.max() == 0.0, f"{what} {name}: expected zeros"
            continue
        rel_rms = math.sqrt(float((d * d).mean())) / rms_r
        rel_max = float(d.max()) / max_r
        assert rel_rms <= 4 * u, f"{what} {name}: rms err {rel_rms:.3e} > {4 * u:.3e}"
        assert rel_max <= 16 * u, f"{what} {name}: max err {rel_max:.3e} > {16 * u:.3e}"


BWD_CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal, dtype
    (1, 300, 300, 4, 4, 128, True, "bf16"),
    (1, 300, 300, 4, 4, 128, True, "f16"),
    (2, 200, 517, 8, 2, 128, True, "f16"),     # bottom-right, GQA 4, ragged
    (1, 517, 200, 4, 1, 64, True, "bf16"),     # rows without a visible key, GQA 4
    (1, 333, 1000, 6, 3, 64, False, "f16"),    # non-causal, GQA 2
    (2, 1, 4000, 16, 2, 128, True, "bf16"),    # one query row per sequence, GQA 8
    (1, 1024, 1024, 4, 4, 128, True, "f16"),   # several blocks each way
    (3, 77, 130, 2, 2, 64, False, "bf16"),
    # head dimensions 192 and 256 (the HIP C++ gradient kernels, the head
    # dimension split over the waves)
    (1, 300, 300, 4, 4, 256, True, "bf16"),
    (2, 200, 517, 8, 2, 192, True, "f16"),     # bottom-right, GQA 4, ragged
    (1, 517, 200, 4, 1, 256, True, "f16"),     # rows without a visible key, GQA 4
    (1, 333, 1000, 6, 3, 192, False, "bf16"),  # non-causal, GQA 2
    (2, 1, 4000, 16, 2, 256, True, "bf16"),    # one query row per sequence, GQA 8
    (3, 77, 130, 2, 2, 192, False, "f16"),
    # workgroups of two 32-key (dK/dV) or 32-row (dQ) halves: fewer keys and
    # rows than one half, exact multiples of a pair, and a pair whose second
    # half is past the end
    (1, 20, 12, 2, 1, 256, True, "bf16"),      # Sq, Skv < 32: one half idle
    (2, 128, 128, 4, 4, 192, False, "f16"),    # whole pairs
    (1, 160, 96, 8, 2, 256, True, "f16"),      # last pair half empty, GQA 4
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal,dtype", BWD_CASES)
def test_backward(fa, B, Sq, Skv, Hq, Hkv, D, causal, dtype):
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed=Sq + 3 * Skv + D)
    scale = 1.0 / math.sqrt(D)
    got = run_bwd(fa, q, k, v, do, causal, scale)
    ref = oracle.attn_bwd(q, k, v, do, causal, scale)
    check_grads(got, ref, dtype, f"B{B} Sq{Sq} Skv{Skv} Hq{Hq} Hkv{Hkv} D{D} c{causal} {dtype}")


def test_backward_large_logits(fa):
    """1% of the key rows scaled by 8 (the prefill workload's stress), fp16."""
    q, k, v, do = _inputs(1, 256, 700, 4, 2, 128, "f16", seed=9, boost=0.01)
    scale = 1.0 / math.sqrt(128)
    got = run_bwd(fa, q, k, v, do, True, scale)
    ref = oracle.attn_bwd(q, k, v, do, True, scale)
    check_grads(got, ref, "f16", "kboost")


def test_backward_dead_rows_are_zero(fa):
    """Causal with Sq > Skv: rows without a visible key get dQ = 0 exactly."""
    q, k, v, do = _inputs(1, 300, 100, 2, 2, 128, "bf16", seed=10)
    dq, _, _ = run_bwd(fa, q, k, v, do, True, 0.088)
    assert np.all(dq[:, :200] == 0.0)


FULL_BWD = [workloads.WORKLOADS[2], workloads.WORKLOADS[3],
            workloads.BY_NAME["causal_b1_h16_s4096_d256_bf16"]]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", FULL_BWD, ids=[w.name for w in FULL_BWD])
def test_backward_full_size_sampled(fa, w):
    """The backward of the S = 4096 and S = 8192 causal workloads (and the
    D = 256 one) at full size:
    dQ of sampled query rows and dK, dV of sampled key rows against the
    oracle (which computes LSE and delta of every row first)."""
    q, k, v = workloads.workload_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 1000)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    dq, dk, dv = run_bwd(fa, q, k, v, do, w.causal, w.scale)
    rng = np.random.default_rng(0)
    n = 384
    qrows = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.Hq, n),
                      rng.integers(0, w.Sq, n)], axis=1)
    qrows[:4, 2] = [0, 1, w.Sq - 1, 127]
    krows = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.Hkv, n),
                      rng.integers(0, w.Skv, n)], axis=1)
    krows[:4, 2] = [0, w.Skv - 1, 128, 4095]
    rq, rk, rv = oracle.attn_bwd_rows(q, k, v, do, w.causal, w.scale, qrows, krows)
    got = (dq[qrows[:, 0], qrows[:, 2], qrows[:, 1]],
           dk[krows[:, 0], krows[:, 2], krows[:, 1]],
           dv[krows[:, 0], krows[:, 2], krows[:, 1]])
    check_grads(got, (rq, rk, rv), w.dtype, w.name)


def test_backward_scale_zero(fa):
    """scale = 0: every visible key gets the same weight, so dQ = dK = 0 exactly
    (each is scale times a finite sum) and dV is dO averaged over the rows that
    see each key; against the oracle at the same tolerance."""
    q, k, v, do = _inputs(1, 200, 333, 4, 2, 128, "bf16", seed=11)
    dq, dk, dv = run_bwd(fa, q, k, v, do, True, 0.0)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    ref = oracle.attn_bwd(q, k, v, do, True, 0.0)
    check_grads((dq, dk, dv), ref, "bf16", "scale 0")


def test_backward_one_kv_head(fa):
    """Sixteen q-heads on one kv-head: the dK / dV sum runs over 16 heads' query
    blocks in one workgroup's step sequence."""
    q, k, v, do = _inputs(1, 300, 700, 16, 1, 128, "bf16", seed=12)
    scale = 1.0 / math.sqrt(128)
    got = run_bwd(fa, q, k, v, do, True, scale)
    ref = oracle.attn_bwd(q, k, v, do, True, scale)
    check_grads(got, ref, "bf16", "Hq16 Hkv1")


def test_backward_is_deterministic(fa):
    """Two calls on the same inputs give the same bits (every gradient element
    has one writer and a fixed summation order)."""
    q, k, v, do = _inputs(2, 517, 517, 8, 2, 64, "f16", seed=13)
    a = run_bwd(fa, q, k, v, do, True, 0.125)
    b = run_bwd(fa, q, k, v, do, True, 0.125)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
