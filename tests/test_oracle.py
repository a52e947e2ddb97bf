"""Pins for the CPU oracle (no GPU needed).

The oracle is only trusted once it agrees with things that do not come from
itself: closed forms, invariants of the online-softmax merge, special cases
that reduce to a textbook result, and two independent library formulations
(the softmax definition evaluated on whole matrices with SciPy's
``logsumexp``, and PyTorch's CPU ``scaled_dot_product_attention`` in
float64).  The cases are
chosen so that a dropped term, a wrong sign, a wrong index or a transposed
operand in ``oracle.c`` fails at least one of them; ``test_oracle_mutants.py``
checks that claim by compiling broken copies of the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _inputs(B, Sq, Skv, Hq, Hkv, D, seed, dtype="bf16", dist="normal"):
    return workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed, dist=dist)


def _f64(t):
    return t.double().numpy()


def _logits(q, k, scale, Hq, Hkv):
    """scale * q.k with contiguous GQA groups, [B, Hq, Sq, Skv] (NumPy)."""
    q, k = _f64(q), _f64(k)
    g = Hq // Hkv
    k_rep = np.repeat(k, g, axis=2)  # kv-head hq // g serves q-head hq
    return scale * np.einsum("bihd,bjhd->bhij", q, k_rep)


def _bottom_right_mask(Sq, Skv):
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    return j <= i + (Skv - Sq)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_single_key_gives_v0(causal):
    """Skv = 1: the only weight is 1, so O = V0 exactly and LSE = s0."""
    B, Sq, Skv, Hq, Hkv, D = 2, 1, 1, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=1)
    scale = 0.125
    o, lse = oracle.attn_fwd(q, k, v, causal, scale)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // (Hq // Hkv)
            np.testing.assert_array_equal(o[b, 0, hq], _f64(v)[b, 0, hk])
            s0 = scale * float(np.dot(_f64(q)[b, 0, hq], _f64(k)[b, 0, hk]))
            assert lse[b, hq, 0] == pytest.approx(s0, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_v(causal):
    """All keys equal: all logits of a row are equal, so O is the plain mean
    of the visible V rows and LSE = s + ln|J|."""
    B, Sq, Skv, Hq, Hkv, D = 1, 7, 11, 2, 1, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=2)
    k[:] = k[:, :1]  # every key row equals key 0
    scale = 0.3
    o, lse = oracle.attn_fwd(q, k, v, causal, scale)
    vv = _f64(v)
    for hq in range(Hq):
        for i in range(Sq):
            n = min(Skv, i + (Skv - Sq) + 1) if causal else Skv
            np.testing.assert_allclose(o[0, i, hq], vv[0, :n, 0].mean(axis=0),
                                       rtol=1e-13, atol=1e-13)
            s = scale * float(np.dot(_f64(q)[0, i, hq], _f64(k)[0, 0, 0]))
            assert lse[0, hq, i] == pytest.approx(s + math.log(n), rel=1e-13, abs=1e-13)


def test_causal_row0_and_last_row():
    """Square causal: row 0 sees only key 0 (O = V0, LSE = s00); the last row
    sees every key, so it equals the non-causal result."""
    B, S, H, D = 2, 33, 3, 64
    q, k, v = _inputs(B, S, S, H, H, D, seed=3)
    scale = 1 / 8
    oc, lc = oracle.attn_fwd(q, k, v, True, scale)
    on, ln_ = oracle.attn_fwd(q, k, v, False, scale)
    np.testing.assert_array_equal(oc[:, 0], _f64(v)[:, 0])
    s00 = scale * np.einsum("bhd,bhd->bh", _f64(q)[:, 0], _f64(k)[:, 0])
    np.testing.assert_allclose(lc[:, :, 0], s00, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(oc[:, -1], on[:, -1])
    np.testing.assert_array_equal(lc[:, :, -1], ln_[:, :, -1])
    # and a middle row differs (the mask does something)
    assert np.abs(oc[:, S // 2] - on[:, S // 2]).max() > 1e-3


def test_bottom_right_offset():
    """Causal with Sq < Skv: row 0 sees the first Skv-Sq+1 keys, so it equals a
    non-causal run over exactly those keys; the last row sees all keys."""
    B, Sq, Skv, H, D = 1, 5, 19, 2, 64
    q, k, v = _inputs(B, Sq, Skv, H, H, D, seed=4)
    scale = 0.2
    oc, lc = oracle.attn_fwd(q, k, v, True, scale)
    n0 = Skv - Sq + 1
    o0, l0 = oracle.attn_fwd(q[:, :1], k[:, :n0], v[:, :n0], False, scale)
    np.testing.assert_array_equal(oc[:, :1], o0)
    np.testing.assert_array_equal(lc[:, :, :1], l0)
    on, ln_ = oracle.attn_fwd(q, k, v, False, scale)
    np.testing.assert_array_equal(oc[:, -1], on[:, -1])
    # row r sees exactly n0 + r keys
    for r in range(Sq):
        orr, lrr = oracle.attn_fwd(q[:, r:r + 1], k[:, :n0 + r], v[:, :n0 + r], False, scale)
        np.testing.assert_array_equal(oc[:, r:r + 1], orr)
        np.testing.assert_array_equal(lc[:, :, r:r + 1], lrr)


def test_top_left_differs_from_bottom_right():
    """The mask is not top-left: with Sq < Skv row 0 must see more than key 0."""
    q, k, v = _inputs(1, 4, 12, 1, 1, 64, seed=5)
    oc, _ = oracle.attn_fwd(q, k, v, True, 0.125)
    assert np.abs(oc[0, 0, 0] - _f64(v)[0, 0, 0]).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_uniform_weights(causal):
    """scale = 0: every visible logit is 0, so O = mean of visible V and
    LSE = ln|J|."""
    B, Sq, Skv, H, D = 1, 6, 9, 2, 64
    q, k, v = _inputs(B, Sq, Skv, H, H, D, seed=6)
    o, lse = oracle.attn_fwd(q, k, v, causal, 0.0)
    vv = _f64(v)
    for h in range(H):
        for i in range(Sq):
            n = min(Skv, i + (Skv - Sq) + 1) if causal else Skv
            np.testing.assert_allclose(o[0, i, h], vv[0, :n, h].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert lse[0, h, i] == pytest.approx(math.log(n), rel=1e-14)


def test_v_ones_gives_ones_and_weights_sum_to_one():
    """V = 1 gives O = 1 (weights sum to one); independently,
    sum_j exp(s_j - LSE) over the visible keys is 1."""
    B, Sq, Skv, Hq, Hkv, D = 2, 13, 21, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=7)
    v1 = torch.ones_like(v)
    scale = 0.125
    o, lse = oracle.attn_fwd(q, k, v1, True, scale)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    s = _logits(q, k, scale, Hq, Hkv)
    mask = _bottom_right_mask(Sq, Skv)
    w = np.where(mask, np.exp(s - lse[..., None]), 0.0)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-13)


def test_no_visible_key_rows():
    """Causal with Sq > Skv: rows i < Sq - Skv see nothing (O = 0, LSE = -inf);
    row Sq - Skv sees key 0 only."""
    B, Sq, Skv, H, D = 1, 9, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, H, H, D, seed=8)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.125)
    dead = Sq - Skv
    assert np.all(o[:, :dead] == 0.0)
    assert np.all(np.isneginf(lse[:, :, :dead]))
    np.testing.assert_array_equal(o[:, dead], _f64(v)[:, 0])
    assert np.all(np.isfinite(lse[:, :, dead:]))


# --------------------------------------------------------------------------
# hand-worked example (tests/golden/worked_example.json)
# --------------------------------------------------------------------------

def test_golden_worked_example():
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
    with open(path) as f:
        ex = json.load(f)
    q = np.array(ex["q"], np.float64)
    k = np.array(ex["k"], np.float64)
    v = np.array(ex["v"], np.float64)
    o, lse = oracle.attn_fwd(q, k, v, ex["causal"], ex["scale"])

    def value(s):  # "12/7" or "ln(14)", exact forms derived by hand
        from fractions import Fraction
        if s.startswith("ln("):
            return math.log(float(Fraction(s[3:-1])))
        return float(Fraction(s))
    exp_o = np.vectorize(value, otypes=[np.float64])(np.array(ex["expected_o"]))
    exp_lse = np.vectorize(value, otypes=[np.float64])(np.array(ex["expected_lse"]))
    np.testing.assert_allclose(o, exp_o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, exp_lse, rtol=1e-14, atol=1e-14)


def test_golden_folded_constant():
    """The Croqtile page prints the folded exponent constant 0.12751743 for
    D = 128: log2(e)/sqrt(128).  The kernel folds scale*log2(e) the same way."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "folded_constant.txt")
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split("=")
                vals[key.strip()] = val.strip()
    printed = float(vals["printed"])
    c = math.log2(math.e) / math.sqrt(128)
    assert f"{c:.8f}" == vals["printed"]
    assert abs(c - printed) < 5e-9


# --------------------------------------------------------------------------
# merge invariant (kernbench `_merge_running`)
# --------------------------------------------------------------------------

def _flat(m, l, acc):
    """[B,Hq,Sq] + [B,Sq,Hq,D] -> rows in (b, hq, i) order."""
    B, Sq, Hq, D = acc.shape
    return m.reshape(-1), l.reshape(-1), acc.transpose(0, 2, 1, 3).reshape(-1, D)


@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_partials_equals_one_shot(causal):
    B, Sq, Skv, Hq, Hkv, D = 1, 16, 40, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=9)
    scale = 0.125
    o, lse = oracle.attn_fwd(q, k, v, causal, scale)
    cuts = [0, 7, 23, 31, Skv]
    parts = [_flat(*oracle.attn_partial(q, k, v, causal, scale, a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    # left fold
    m, l, acc = parts[0]
    for p in parts[1:]:
        m, l, acc = oracle.merge(m, l, acc, *p)
    # right fold, different association and order
    m2, l2, acc2 = parts[-1]
    for p in reversed(parts[:-1]):
        m2, l2, acc2 = oracle.merge(*p, m2, l2, acc2)
    o_ref = o.transpose(0, 2, 1, 3).reshape(-1, D)
    for (mm, ll, aa) in ((m, l, acc), (m2, l2, acc2)):
        np.testing.assert_allclose(aa / ll[:, None], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(mm + np.log(ll), lse.reshape(-1), rtol=1e-12, atol=1e-13)


def test_merge_identity_commutes_and_associates():
    rng = np.random.default_rng(10)
    n, D = 5, 8
    def rand_triple():
        return rng.normal(size=n), rng.uniform(0.5, 3, size=n), rng.normal(size=(n, D))
    a, b, c = rand_triple(), rand_triple(), rand_triple()
    ident = (np.full(n, -np.inf), np.zeros(n), np.zeros((n, D)))
    for x in (a, b):
        for r in (oracle.merge(*x, *ident), oracle.merge(*ident, *x)):
            np.testing.assert_array_equal(r[0], x[0])
            np.testing.assert_allclose(r[1], x[1], rtol=1e-15)
            np.testing.assert_allclose(r[2], x[2], rtol=1e-15)
    ii = oracle.merge(*ident, *ident)
    assert np.all(np.isneginf(ii[0])) and np.all(ii[1] == 0) and np.all(ii[2] == 0)
    ab, ba = oracle.merge(*a, *b), oracle.merge(*b, *a)
    for x, y in zip(ab, ba):
        np.testing.assert_allclose(x, y, rtol=1e-14)
    l1 = oracle.merge(*oracle.merge(*a, *b), *c)
    r1 = oracle.merge(*a, *oracle.merge(*b, *c))
    for x, y in zip(l1, r1):
        np.testing.assert_allclose(x, y, rtol=1e-13)
    # closed form: merged l is sum_i l_i exp(m_i - max m)
    mm = np.maximum(a[0], b[0])
    np.testing.assert_allclose(ab[1], a[1] * np.exp(a[0] - mm) + b[1] * np.exp(b[0] - mm), rtol=1e-14)


# --------------------------------------------------------------------------
# grouped-query heads
# --------------------------------------------------------------------------

def test_gqa_contiguous_grouping():
    """Hq=4, Hkv=2 equals the Hq=Hkv=4 run with each kv-head repeated for its
    contiguous group (repeat_interleave), and not the interleaved (tiled) one."""
    B, Sq, Skv, Hq, Hkv, D = 2, 9, 12, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=11)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.125)
    kr, vr = k.repeat_interleave(2, dim=2), v.repeat_interleave(2, dim=2)
    o2, lse2 = oracle.attn_fwd(q, kr, vr, True, 0.125)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    kt, vt = k.repeat(1, 1, 2, 1), v.repeat(1, 1, 2, 1)
    o3, _ = oracle.attn_fwd(q, kt, vt, True, 0.125)
    assert np.abs(o - o3).max() > 1e-3


# --------------------------------------------------------------------------
# independent library formulations
# --------------------------------------------------------------------------

def _softmax_definition(q, k, v, causal, scale, Hq, Hkv):
    """Masked softmax attention evaluated from its definition on whole
    matrices: the weights of a row are exp(s_j - LSE) over its visible keys,
    with LSE = logsumexp of the row's visible logits (SciPy's routine), and O
    is the weighted sum of the V rows.  Returns O [B,Sq,Hq,D] and the
    natural-log LSE [B,Hq,Sq]."""
    from scipy.special import logsumexp
    s = _logits(q, k, scale, Hq, Hkv)                     # [B, Hq, Sq, Skv]
    if causal:
        s = np.where(_bottom_right_mask(s.shape[2], s.shape[3]), s, -np.inf)
    lse = logsumexp(s, axis=-1)                           # [B, Hq, Sq]
    w = np.exp(s - lse[..., None])
    v_rep = np.repeat(_f64(v), Hq // Hkv, axis=2)         # [B, Skv, Hq, D]
    o = np.einsum("bhij,bjhd->bihd", w, v_rep)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_against_softmax_definition(causal):
    B, S, Hq, Hkv, D = 2, 24, 4, 2, 64
    q, k, v = _inputs(B, S, S, Hq, Hkv, D, seed=12)
    o, lse = oracle.attn_fwd(q, k, v, causal, 1.0)
    o_ref, lse_ref = _softmax_definition(q, k, v, causal, 1.0, Hq, Hkv)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_base2_residual_identity():
    """The JAX page keeps a base-2 residual: row max (in natural-log units)
    times log2(e) plus log2 of the row's sum of exp(s_j - max).  The oracle's
    natural-log LSE times log2(e) must equal it."""
    B, S, Hq, Hkv, D = 1, 20, 2, 1, 64
    q, k, v = _inputs(B, S, S, Hq, Hkv, D, seed=16)
    _, lse = oracle.attn_fwd(q, k, v, True, 0.3)
    s = _logits(q, k, 0.3, Hq, Hkv)
    s = np.where(_bottom_right_mask(S, S), s, -np.inf)
    m = s.max(axis=-1)
    resid2 = m * math.log2(math.e) + np.log2(np.exp(s - m[..., None]).sum(axis=-1))
    np.testing.assert_allclose(lse * math.log2(math.e), resid2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal,scale", [
    (1, 17, 17, 1, 1, 64, True, 0.125),
    (2, 9, 31, 4, 2, 64, True, 0.0884),
    (2, 31, 9, 4, 4, 128, True, 0.0884),
    (1, 12, 40, 8, 1, 64, False, 0.5),
    (2, 33, 64, 4, 1, 128, True, 1.0),
])
def test_against_torch_sdpa_float64(B, Sq, Skv, Hq, Hkv, D, causal, scale):
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=13 + Sq)
    o, lse = oracle.attn_fwd(q, k, v, causal, scale)
    g = Hq // Hkv
    qt = q.double().permute(0, 2, 1, 3)
    kt = k.double().repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vt = v.double().repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    mask = None
    if causal:
        mask = torch.from_numpy(_bottom_right_mask(Sq, Skv))
    dead = None
    if causal and Sq > Skv:
        dead = Sq - Skv  # SDPA gives NaN on fully masked rows; compare the rest
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale).permute(0, 2, 1, 3).numpy()
    s = torch.from_numpy(_logits(q, k, scale, Hq, Hkv))
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    lse_ref = torch.logsumexp(s, dim=-1).numpy()
    sl = slice(dead, None) if dead else slice(None)
    np.testing.assert_allclose(o[:, sl], ref[:, sl], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, sl], lse_ref[:, :, sl], rtol=1e-12, atol=1e-12)
    if dead:
        assert np.all(o[:, :dead] == 0) and np.all(np.isneginf(lse[:, :, :dead]))


def test_rows_equal_full():
    """The row-sampling entry gives the same numbers as the full forward."""
    B, Sq, Skv, Hq, Hkv, D = 2, 20, 50, 4, 2, 64
    q, k, v = _inputs(B, Sq, Skv, Hq, Hkv, D, seed=14)
    o, lse = oracle.attn_fwd(q, k, v, True, 0.125)
    rows = np.array([[0, 0, 0], [1, 3, 19], [0, 2, 7], [1, 1, 11]])
    orow, lrow = oracle.attn_rows(q, k, v, True, 0.125, rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(orow[r], o[b, i, h])
        assert lrow[r] == lse[b, h, i]


def test_large_logits_are_stable():
    """Keys scaled by 8 on some rows (the long-prefix workload's stress) keep
    the oracle finite and equal to float64 SDPA."""
    B, Sq, Skv, Hq, Hkv, D = 1, 8, 64, 4, 1, 128
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, "f16", 15, k_row_boost_frac=0.1)
    o, lse = oracle.attn_fwd(q, k, v, True, 1 / math.sqrt(128))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    qt = q.double().permute(0, 2, 1, 3)
    kt = k.double().repeat_interleave(Hq, dim=2).permute(0, 2, 1, 3)
    vt = v.double().repeat_interleave(Hq, dim=2).permute(0, 2, 1, 3)
    mask = torch.from_numpy(_bottom_right_mask(Sq, Skv))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=1 / math.sqrt(128)).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)
