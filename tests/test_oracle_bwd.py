"""Pins for the oracle's backward pass (no GPU needed).

oracle.attn_bwd is trusted only once it agrees with what does not come from
itself: central finite differences of the (separately pinned) forward
oracle, a hand-worked example, closed forms, invariants of the softmax
gradient, and PyTorch autograd in float64 on the CPU.  test_oracle_mutants.py
plants mistakes in the backward and checks that these pins catch them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def _inputs(B, Sq, Skv, Hq, Hkv, D, seed, dtype="bf16"):
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn((B, Sq, Hq, D), generator=g, dtype=torch.float32).to(q.dtype)
    return q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy()


def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attn_fwd(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv,Hq,Hkv", [(7, 7, 2, 1), (5, 11, 4, 2), (9, 4, 2, 2)])
def test_finite_differences(causal, Sq, Skv, Hq, Hkv):
    """dL/dx of L = sum(O * dO) by central differences of the forward oracle
    at sampled entries of q, k and v (fp64, step 1e-6: truncation ~1e-12)."""
    D, scale = 8, 0.35
    q, k, v, do = _inputs(1, Sq, Skv, Hq, Hkv, D, seed=Sq * 31 + Skv)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
    rng = np.random.default_rng(Sq + Skv)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num = (_loss(args_p["q"], args_p["k"], args_p["v"], do, causal, scale)
                   - _loss(args_m["q"], args_m["k"], args_m["v"], do, causal, scale)) / (2 * h)
            assert grad[idx] == pytest.approx(num, rel=1e-6, abs=1e-7), (name, idx)


def _exact(s):
    """'3/4', '-3/4*ln(3)', 'ln(3)' -> float."""
    s = str(s)
    if "*ln(" in s:
        a, b = s.split("*ln(")
        return float(Fraction(a)) * math.log(float(Fraction(b[:-1])))
    if s.startswith("ln("):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def test_golden_worked_example():
    path = os.path.join(os.path.dirname(__file__), "golden", "bwd_worked_example.json")
    with open(path) as f:
        ex = json.load(f)
    conv = np.vectorize(_exact, otypes=[np.float64])
    q, k, v, do = (conv(np.array(ex[n], dtype=object)) for n in ("q", "k", "v", "dout"))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, ex["causal"], ex["scale"])
    np.testing.assert_allclose(dq, conv(np.array(ex["expected_dq"], dtype=object)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dk, conv(np.array(ex["expected_dk"], dtype=object)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dv, conv(np.array(ex["expected_dv"], dtype=object)), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key(causal):
    """Skv = 1: the weight is 1 whatever q and k are, so dQ = dK = 0, and
    dV_0 of a kv-head is the sum of dO over its q-heads and rows."""
    B, Sq, Hq, Hkv, D = 2, 1, 4, 2, 16
    q, k, v, do = _inputs(B, Sq, 1, Hq, Hkv, D, seed=3)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, 0.3)
    assert np.all(dq == 0) and np.all(dk == 0)
    g = Hq // Hkv
    expect = do.reshape(B, Sq, Hkv, g, D).sum(axis=(1, 3))
    np.testing.assert_allclose(dv[:, 0], expect, rtol=1e-14, atol=1e-14)


def test_constant_values_give_zero_dq_dk():
    """Every V row equal: O = V_0 for any weights, so dQ = dK = 0."""
    B, Sq, Skv, Hq, Hkv, D = 1, 6, 9, 2, 1, 16
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=4)
    v[:] = v[:, :1]
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True, 0.4)
    np.testing.assert_allclose(dq, 0, atol=1e-13)
    np.testing.assert_allclose(dk, 0, atol=1e-13)
    assert np.abs(dv).max() > 0.1


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero(causal):
    """scale = 0: uniform weights over the visible keys; dQ = dK = 0 and
    dV_j = sum over rows i that see j of dO_i / |J_i|."""
    B, Sq, Skv, H, D = 1, 5, 8, 2, 8
    q, k, v, do = _inputs(B, Sq, Skv, H, H, D, seed=5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    expect = np.zeros_like(dv)
    for i in range(Sq):
        n = min(Skv, i + (Skv - Sq) + 1) if causal else Skv
        expect[:, :n] += do[:, i:i + 1] / n
    np.testing.assert_allclose(dv, expect, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Softmax is unchanged by adding one vector to every key of a kv-head, so
    sum_j dK_j = 0; the weights of a row sum to one, so sum_j dV_j is the sum
    of dO over the rows with a visible key."""
    B, Sq, Skv, Hq, Hkv, D = 2, 7, 12, 4, 2, 16
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=6)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, 0.3)
    np.testing.assert_allclose(dk.sum(axis=1), 0, atol=1e-12)
    g = Hq // Hkv
    np.testing.assert_allclose(dv.sum(axis=1), do.reshape(B, Sq, Hkv, g, D).sum(axis=(1, 3)),
                               rtol=1e-12, atol=1e-12)


def test_no_visible_key_rows():
    """Causal with Sq > Skv: rows without a visible key get dQ = 0 and add
    nothing to dK, dV (equal to the run without those rows)."""
    B, Sq, Skv, H, D = 1, 9, 4, 2, 8
    q, k, v, do = _inputs(B, Sq, Skv, H, H, D, seed=7)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True, 0.3)
    dead = Sq - Skv
    assert np.all(dq[:, :dead] == 0)
    dq2, dk2, dv2 = oracle.attn_bwd(q[:, dead:], k, v, do[:, dead:], True, 0.3)
    np.testing.assert_allclose(dq[:, dead:], dq2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dk, dk2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dv, dv2, rtol=1e-14, atol=1e-15)


def _torch_grads(q, k, v, do, causal, scale, Hq, Hkv):
    g = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    kr = kt.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vr = vt.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    s = scale * torch.matmul(qt, kr.transpose(-1, -2))
    Sq, Skv = q.shape[1], k.shape[1]
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        s = s.masked_fill(j > i + (Skv - Sq), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vr).permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    return qt.grad.permute(0, 2, 1, 3).numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal,scale", [
    (1, 17, 17, 1, 1, 64, True, 0.125),
    (2, 9, 31, 4, 2, 64, True, 0.0884),
    (1, 12, 40, 8, 1, 32, False, 0.5),
    (2, 20, 20, 6, 2, 16, False, 1.0),
])
def test_against_torch_autograd_float64(B, Sq, Skv, Hq, Hkv, D, causal, scale):
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=Sq + Skv)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
    rq, rk, rv = _torch_grads(q, k, v, do, causal, scale, Hq, Hkv)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-10, atol=1e-12)


def test_rows_equal_full():
    """The selected-rows entry gives the same numbers as the full backward."""
    B, Sq, Skv, Hq, Hkv, D = 2, 11, 17, 4, 2, 16
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=8)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True, 0.3)
    qrows = np.array([[0, 0, 0], [1, 3, 10], [0, 2, 5]])
    krows = np.array([[0, 0, 0], [1, 1, 16], [1, 0, 7]])
    dq_r, dk_r, dv_r = oracle.attn_bwd_rows(q, k, v, do, True, 0.3, qrows, krows)
    for n, (b, hq, i) in enumerate(qrows):
        np.testing.assert_array_equal(dq_r[n], dq[b, i, hq])
    for n, (b, hk, j) in enumerate(krows):
        np.testing.assert_array_equal(dk_r[n], dk[b, j, hk])
        np.testing.assert_array_equal(dv_r[n], dv[b, j, hk])
