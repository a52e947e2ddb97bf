"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (per element, O widened to fp64): max |dO| <= 2e-2, mean |dO| <= 2e-3,
max |dLSE| <= 1e-3, both sides reading the same rounded input bits.

* Every case is compared element by element on every output, the five
  named workloads included: they run at full size in the launch
  configuration the benchmark times, and the oracle evaluates all their
  rows (a few minutes of host time for the largest).  A property that holds
  at any size (V = 1 gives O = 1) is checked on them as well.
* Split key ranges run through fa_fwd_ws with a workspace of the size
  fa_fwd_plan reports; decode-shaped calls (a few query rows over long key
  ranges) among them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

MAX_DO, MEAN_DO, MAX_DLSE = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import attention_forward_05_amd as m
    m.load()
    return m


def run_gpu(fa, q, k, v, causal, scale, with_lse=True, stream=None, split=False):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.attention(qd, kd, vd, causal, scale, with_lse=with_lse, stream=stream,
                          split=split)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), (lse.cpu().double().numpy() if with_lse else None)


def check(o, lse, o_ref, lse_ref, what="", figures=None):
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    do = np.abs(o - o_ref)
    if figures is not None:
        dl_all = 0.0
        if lse is not None:
            live = ~np.isneginf(lse_ref)
            if live.any():
                dl_all = float(np.abs(lse[live] - lse_ref[live]).max())
        figures.append(f"{what}: max|dO| {do.max():.3e}  mean|dO| {do.mean():.3e}  "
                       f"max|dLSE| {dl_all:.3e}  ({o.size} O elements)")
    assert do.max() <= MAX_DO, f"{what}: max|dO| {do.max():.3e}"
    assert do.mean() <= MEAN_DO, f"{what}: mean|dO| {do.mean():.3e}"
    if lse is not None:
        dead = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse), dead), f"{what}: -inf LSE pattern differs"
        if (~dead).any():
            dl = np.abs(lse[~dead] - lse_ref[~dead])
            assert dl.max() <= MAX_DLSE, f"{what}: max|dLSE| {dl.max():.3e}"
    return do.max(), do.mean()


def full_case(fa, B, Sq, Skv, Hq, Hkv, D, causal, dtype="bf16", seed=0, scale=None, dist="normal",
              boost=0.0, split=False):
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype, seed, k_row_boost_frac=boost, dist=dist)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(fa, q, k, v, causal, scale, split=split)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    return check(o, lse, o_ref, lse_ref, f"B{B} Sq{Sq} Skv{Skv} Hq{Hq} Hkv{Hkv} D{D} c{causal} {dtype}")


def compute_units():
    return torch.cuda.get_device_properties(0).multi_processor_count


def plan(fa, B, Sq, Skv, Hq, Hkv, D, causal, with_ws):
    st, kern, ranges, ws = fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, int(causal), compute_units(),
                                          with_ws)
    assert st == fa.FA_OK
    return kern, ranges, ws


# ---------------------------------------------------------------------------
# small / ragged shapes, every output element
# ---------------------------------------------------------------------------

RAGGED = [1, 17, 200, 1000]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq", RAGGED)
@pytest.mark.parametrize("Skv", RAGGED)
def test_ragged_shapes_bf16(fa, Sq, Skv, causal, D):
    full_case(fa, 1, Sq, Skv, 2, 1, D, causal, "bf16", seed=Sq * 7 + Skv)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Skv", [(300, 300), (17, 1000), (1000, 17), (257, 513)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes_f16(fa, Sq, Skv, causal, D):
    full_case(fa, 2, Sq, Skv, 4, 2, D, causal, "f16", seed=Sq + Skv + D)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_d64_long_keys_and_gqa(fa, dtype):
    """D = 64 (the four-wave kernel's second head size) over long, ragged key
    ranges with GQA 4, causal bottom-right."""
    full_case(fa, 2, 700, 3001, 16, 4, 64, True, dtype, seed=31)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_gqa_ratios(fa, g):
    full_case(fa, 2, 333, 700, 8, 8 // g, 128, True, "bf16", seed=100 + g)


@pytest.mark.parametrize("B,Hq", [(3, 5), (1, 12), (2, 16)])
def test_head_counts_not_multiple_of_8(fa, B, Hq):
    # exercises both workgroup orderings (pairs % 8 == 0 and != 0)
    full_case(fa, B, 520, 520, Hq, 1, 64, True, "bf16", seed=B * Hq)


def test_no_visible_key_rows(fa):
    """Causal with Sq > Skv: the first Sq - Skv rows see no key: O = 0 exactly,
    LSE = -inf; the others match the oracle."""
    B, Sq, Skv, H, D = 1, 600, 100, 2, 128
    q, k, v = workloads.make_inputs(B, Sq, Skv, H, H, D, "bf16", 5)
    o, lse = run_gpu(fa, q, k, v, True, 0.088)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, 0.088)
    dead = Sq - Skv
    assert np.all(o[:, :dead] == 0.0)
    assert np.all(np.isneginf(lse[:, :, :dead]))
    check(o, lse, o_ref, lse_ref, "dead rows")


def test_scale_zero(fa):
    """scale = 0: O is the mean of the visible V rows, LSE = ln(count)."""
    B, Sq, Skv, H, D = 1, 130, 300, 2, 64
    q, k, v = workloads.make_inputs(B, Sq, Skv, H, H, D, "bf16", 6)
    o, lse = run_gpu(fa, q, k, v, True, 0.0)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, 0.0)
    check(o, lse, o_ref, lse_ref, "scale 0")
    n = np.arange(Sq) + (Skv - Sq) + 1
    np.testing.assert_allclose(lse[0, 0], np.log(n), atol=1e-4)


def test_lse_null_gives_same_output(fa):
    q, k, v = workloads.make_inputs(1, 400, 400, 4, 4, 128, "bf16", 7)
    o1, _ = run_gpu(fa, q, k, v, True, 0.088, with_lse=True)
    o2, l2 = run_gpu(fa, q, k, v, True, 0.088, with_lse=False)
    assert l2 is None
    np.testing.assert_array_equal(o1, o2)


def test_deterministic_and_side_stream(fa):
    """Two runs give identical bits, also when enqueued on a non-default stream."""
    q, k, v = workloads.make_inputs(2, 700, 900, 8, 2, 128, "bf16", 8)
    o1, l1 = run_gpu(fa, q, k, v, True, 0.088)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = run_gpu(fa, q, k, v, True, 0.088, stream=s)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_uniform_inputs_and_large_logits(fa):
    full_case(fa, 1, 512, 512, 2, 2, 128, True, "bf16", seed=9, dist="uniform")
    full_case(fa, 1, 256, 777, 2, 1, 128, False, "f16", seed=10, scale=1.0)


# ---------------------------------------------------------------------------
# the eight-wave kernel: D = 128 with at least 256 (batch, q-head, 512-row
# query tile) items, i.e. one per compute unit of an MI355X
# ---------------------------------------------------------------------------

X8_CASES = [
    # B, Sq, Skv, Hq, Hkv, causal, dtype
    (1, 512, 512, 256, 256, True, "bf16"),     # one query tile, the whole diagonal
    (1, 1000, 1000, 128, 32, True, "bf16"),    # ragged second tile, GQA 4
    (2, 300, 777, 128, 16, False, "bf16"),     # ragged key tail, GQA 8
    (1, 200, 1500, 256, 32, True, "f16"),      # bottom-right mask, Sq < Skv
    (1, 1500, 1300, 128, 128, True, "bf16"),   # rows (and whole blocks) without a key
    (1, 1600, 1000, 128, 64, True, "bf16"),    # a query tile without any key
    (1, 520, 600, 256, 64, False, "f16"),      # 8-row second query tile
    (1, 1024, 150, 256, 32, False, "bf16"),    # 3-tile items, two per compute unit
    (2, 2048, 200, 128, 128, False, "bf16"),   # 4-tile items, four per compute unit
    (22, 512, 300, 12, 4, True, "bf16"),       # Hq % 8 != 0, GQA 3, 264 items: a short last round
    (8, 1100, 260, 32, 8, False, "f16"),       # 768 items (three rounds), ragged rows and keys
    (1, 700, 3000, 256, 64, True, "bf16"),     # bottom-right, two query tiles of unequal length
]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,causal,dtype", X8_CASES)
def test_eight_wave_shapes(fa, B, Sq, Skv, Hq, Hkv, causal, dtype, D):
    if compute_units() == 256:
        for with_ws in (False, True):
            assert plan(fa, B, Sq, Skv, Hq, Hkv, D, causal, with_ws) == (
                fa.FA_KERNEL_EIGHT_WAVE, 1, 0)
    full_case(fa, B, Sq, Skv, Hq, Hkv, D, causal, dtype, seed=Sq + 3 * Skv + Hkv + D)


@pytest.mark.parametrize("D", [128, 64])
def test_eight_wave_special_arguments(fa, D):
    """The eight-wave kernel with scale 0 (O = mean of the visible V rows,
    LSE = ln(count)), without LSE (same O bits), and twice in a row (same
    bits), on a bottom-right causal shape with 256 items."""
    B, Sq, Skv, Hq, Hkv = 1, 512, 700, 256, 64
    if compute_units() == 256:
        assert plan(fa, B, Sq, Skv, Hq, Hkv, D, True, False)[0] == fa.FA_KERNEL_EIGHT_WAVE
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, "bf16", 61 + D)
    o, lse = run_gpu(fa, q, k, v, True, 0.0)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, 0.0)
    check(o, lse, o_ref, lse_ref, f"scale 0, D {D}")
    n = np.arange(Sq) + (Skv - Sq) + 1
    np.testing.assert_allclose(lse[0, 5], np.log(n), atol=1e-4)
    scale = 1.0 / math.sqrt(D)
    o1, l1 = run_gpu(fa, q, k, v, True, scale)
    o2, l2 = run_gpu(fa, q, k, v, True, scale, with_lse=False)
    o3, l3 = run_gpu(fa, q, k, v, True, scale)
    assert l2 is None
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(o1, o3)
    np.testing.assert_array_equal(l1, l3)


def rounding_bound(o, o_ref, v, dtype):
    """Elementwise bound of the two roundings the kernel does (P and O to the
    input dtype, unit roundoff u = 2^-8 for bf16, 2^-11 for fp16): P rounded
    moves O by at most u * sum_j w_j |V_j| <= u * max|V|, and the final
    rounding by u * |O|.  Returns the largest ratio |dO| / bound (<= 1)."""
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    vmax = float(np.abs(v.double().numpy()).max())
    bound = u * (np.abs(o_ref) + vmax) * (1 + u) + 1e-5
    return float((np.abs(o - o_ref) / bound).max())


@pytest.mark.parametrize("D", [128, 64])
def test_eight_wave_slow_path_bf16(fa, D):
    """bf16 on the eight-wave kernel with 1% of the key rows scaled by 8: the
    reference max moves (the slow path) in bf16 as well.  The softmax is
    nearly one-hot here, so |O| reaches |V| (about 4.5) and bf16 rounding of
    O alone can exceed the 2e-2 bar of the N(0,1) workloads: the bar is the
    rounding bound instead, with the mean and LSE bars unchanged."""
    if compute_units() == 256:
        assert plan(fa, 1, 256, 1024, 256, 8, D, True, False)[0] == fa.FA_KERNEL_EIGHT_WAVE
    B, Sq, Skv, Hq, Hkv = 1, 256, 1024, 256, 8
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, D, "bf16", 24, k_row_boost_frac=0.01)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(fa, q, k, v, True, scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, scale)
    assert rounding_bound(o, o_ref, v, "bf16") <= 1.0
    do = np.abs(o - o_ref)
    assert do.mean() <= MEAN_DO
    assert np.abs(lse - lse_ref).max() <= MAX_DLSE


# ---------------------------------------------------------------------------
# split key ranges: items too few for the compute units, long key ranges; the
# eight-wave kernel writes fp32 partial (O, LSE) per range and a second
# kernel merges them
# ---------------------------------------------------------------------------

SPLIT_CASES = [
    # B, Sq, Skv, Hq, Hkv, causal, dtype, key ranges on 256 compute units
    (1, 1000, 16384, 8, 2, True, "bf16", 8),    # bottom-right, ragged second query tile
    (1, 512, 8192, 4, 4, False, "f16", 8),      # 16 key tiles per range
    (2, 700, 5000, 16, 2, True, "bf16", 4),     # GQA 8, ragged keys, unequal items
    (3, 300, 4000, 5, 5, False, "bf16", 2),     # Hq % 8 != 0, ragged last range
    (1, 2048, 8192, 16, 8, True, "f16", 4),     # causal diagonal inside the last range
    (1, 512, 16384, 16, 4, False, "bf16", 16),  # 16 ranges
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,causal,dtype,ranges", SPLIT_CASES)
def test_split_key_ranges(fa, B, Sq, Skv, Hq, Hkv, causal, dtype, ranges):
    kern, nr, ws = plan(fa, B, Sq, Skv, Hq, Hkv, 128, causal, True)
    assert kern == fa.FA_KERNEL_EIGHT_WAVE
    if compute_units() == 256:
        assert nr == ranges and ws == ranges * B * Hq * Sq * 129 * 4
    full_case(fa, B, Sq, Skv, Hq, Hkv, 128, causal, dtype, seed=Sq + 7 * Skv + Hq, split=True)


def test_split_shape_without_workspace(fa):
    """fa_fwd on a shape fa_fwd_ws would split: whole key ranges, same bar."""
    assert plan(fa, 1, 1000, 16384, 8, 2, 128, True, False)[1] == 1
    full_case(fa, 1, 1000, 16384, 8, 2, 128, True, "bf16", seed=5)


# decode-shaped calls: a few query rows (Sq <= 64) over long key ranges,
# GQA 4 and 8, with a workspace (split key ranges)
DECODE_CASES = [
    # B, Sq, Skv, Hq, Hkv, causal, dtype
    (1, 1, 16384, 32, 8, False, "bf16"),
    (1, 1, 32768, 64, 8, True, "f16"),
    (2, 4, 16384, 32, 8, True, "bf16"),
    (1, 16, 32768, 32, 4, False, "bf16"),
    (1, 16, 16384, 16, 4, True, "f16"),
    (1, 64, 16384, 32, 8, True, "bf16"),
    (1, 64, 32768, 64, 8, False, "f16"),
    (3, 7, 20000, 24, 3, True, "bf16"),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,causal,dtype", DECODE_CASES)
def test_decode_shapes(fa, B, Sq, Skv, Hq, Hkv, causal, dtype, parity_figures):
    q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, 128, dtype, 200 + Sq + Hq)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_gpu(fa, q, k, v, causal, scale, split=True)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    check(o, lse, o_ref, lse_ref, f"decode B{B} Sq{Sq} Skv{Skv} Hq{Hq} Hkv{Hkv} c{causal} {dtype}",
          figures=parity_figures)
    # and without a workspace: whole key ranges, same bar
    o2, lse2 = run_gpu(fa, q, k, v, causal, scale)
    check(o2, lse2, o_ref, lse_ref, "decode (no workspace)")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Hq,Hkv,causal", [(1, 16, 2, True), (3, 12, 4, False),
                                               (20, 8, 1, True), (64, 4, 4, False)])
def test_decode_tile_kernels(fa, D, Sq, Hq, Hkv, causal):
    """The packed tile kernels with and without split key ranges: keys over
    the waves (Sq * Hq / Hkv <= 32) or rows (more), bf16 and fp16."""
    kern, _, _ = plan(fa, 2, Sq, 5000, Hq, Hkv, D, causal, True)
    assert kern == (fa.FA_KERNEL_TILE_KEYS if Sq * (Hq // Hkv) <= 32 else fa.FA_KERNEL_TILE_ROWS)
    for dtype, split in (("bf16", True), ("f16", False)):
        full_case(fa, 2, Sq, 5000, Hq, Hkv, D, causal, dtype, seed=Sq + Hq + D, split=split)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_slow_path(fa, D):
    """Decode shapes with 1% of the key rows scaled by 8, fp16: rows' maxima
    jump inside the key ranges, so the tile kernel's reference max moves
    (its slow path) in both the key and the row split."""
    for Sq, Hq, Hkv in ((1, 32, 8), (16, 16, 2)):
        full_case(fa, 1, Sq, 9000, Hq, Hkv, D, True, "f16", seed=60 + Sq + D, boost=0.01,
                  split=True)


# head dimensions 192 and 256: the tile kernel, four waves over 128-row blocks
# (D = 192 with its LDS rows padded to 256 dimensions)
LARGE_D_CASES = [
    # B, Sq, Skv, Hq, Hkv, causal, dtype, split
    (1, 128, 128, 1, 1, True, "bf16", False),
    (2, 300, 300, 4, 2, True, "bf16", False),     # ragged rows and keys, GQA 2
    (1, 100, 1000, 8, 2, True, "f16", False),     # bottom-right, GQA 4
    (1, 1000, 100, 2, 1, True, "bf16", False),    # rows with no visible key
    (2, 513, 777, 3, 3, False, "f16", False),     # ragged, Hq % 8 != 0
    (1, 256, 8192, 4, 4, False, "bf16", True),    # 16 key ranges merged
    (1, 200, 6000, 6, 2, True, "f16", True),      # split, bottom-right, GQA 3
    (1, 40, 3000, 8, 1, True, "bf16", True),      # few rows: 8 q-heads packed, 320 rows
    (2, 1, 5000, 32, 4, True, "f16", True),       # decode, 8 q-heads packed into rows
]


@pytest.mark.parametrize("D", [192, 256])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,causal,dtype,split", LARGE_D_CASES)
def test_head_dim_large(fa, B, Sq, Skv, Hq, Hkv, causal, dtype, split, D):
    assert plan(fa, B, Sq, Skv, Hq, Hkv, D, causal, split)[0] == fa.FA_KERNEL_TILE_ROWS
    full_case(fa, B, Sq, Skv, Hq, Hkv, D, causal, dtype, seed=Sq + Skv + D, split=split)


@pytest.mark.parametrize("D", [192, 256])
def test_head_dim_large_logits(fa, D):
    """D = 192, 256 with scale 1 on N(0, 1) inputs (nearly one-hot softmax,
    the running max moves often), fp16: within the rounding bound."""
    q, k, v = workloads.make_inputs(1, 200, 700, 2, 1, D, "f16", 77)
    o, lse = run_gpu(fa, q, k, v, True, 1.0)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, 1.0)
    assert rounding_bound(o, o_ref, v, "f16") <= 1.0
    assert np.abs(lse - lse_ref).max() <= MAX_DLSE


def test_long_key_range_few_rows(fa):
    """A key range of about a million keys (16384 key tiles, the ragged last
    one with 63 keys) for three query rows."""
    full_case(fa, 1, 3, (1 << 20) - 1, 8, 2, 128, True, "bf16", seed=41, split=True)


def test_split_without_lse(fa):
    """lse = NULL on the split path: the merge still needs the partial LSEs
    (which the kernel always writes), and O must not change."""
    q, k, v = workloads.make_inputs(1, 1000, 16384, 8, 2, 128, "bf16", 5)
    o1, l1 = run_gpu(fa, q, k, v, True, 0.088, split=True)
    o2, _ = run_gpu(fa, q, k, v, True, 0.088, with_lse=False, split=True)
    assert np.array_equal(o1, o2)


def test_split_streams_own_workspaces(fa):
    """Split calls on two streams, queued without a host wait, each with a
    workspace of its own: the same bits as when run one at a time."""
    dev = torch.device("cuda:0")
    shapes = [(1, 512, 8192, 4, 4, False), (1, 1000, 16384, 8, 2, True), (1, 512, 8192, 4, 4, False)]
    ins = []
    for n, (B, Sq, Skv, Hq, Hkv, causal) in enumerate(shapes):
        q, k, v = workloads.make_inputs(B, Sq, Skv, Hq, Hkv, 128, "bf16", 100 + n)
        ins.append((q.to(dev), k.to(dev), v.to(dev), causal))
    ref = []
    for q, k, v, causal in ins:
        o, lse = fa.attention(q, k, v, causal, 0.088, split=True)
        torch.cuda.synchronize()
        ref.append((o.clone(), lse.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, keep = [], []
    for n, (q, k, v, causal) in enumerate(ins):
        B, Sq, Hq, D = q.shape
        Skv, Hkv = k.shape[1], k.shape[2]
        _, _, nr, nbytes = fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, D, int(causal), compute_units(), True)
        assert nr > 1
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Sq), float("nan"), device=dev)
        st = streams[n % 2]
        st.wait_stream(torch.cuda.current_stream())
        assert fa.fa_fwd_ws(fa.FA_DTYPE_BF16, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D,
                            int(causal), 0.088, ws, nbytes, st) == fa.FA_OK
        outs.append((o, lse))
        keep.append(ws)
    torch.cuda.synchronize()
    for (o, lse), (o_ref, lse_ref) in zip(outs, ref):
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_split_workspace_too_small(fa):
    """A workspace one byte short of what fa_fwd_plan reports: FA_ERR_WORKSPACE,
    nothing enqueued (the outputs keep their contents)."""
    dev = torch.device("cuda:0")
    B, Sq, Skv, Hq, Hkv = 1, 512, 8192, 4, 4
    q, k, v = (t.to(dev) for t in workloads.make_inputs(B, Sq, Skv, Hq, Hkv, 128, "bf16", 3))
    _, _, nr, nbytes = fa.fa_fwd_plan(B, Sq, Skv, Hq, Hkv, 128, 0, compute_units(), True)
    assert nr > 1
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, Sq), 7.0, device=dev)
    st = fa.fa_fwd_ws(fa.FA_DTYPE_BF16, q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, 128, 0, 0.088,
                      ws, nbytes - 16, None)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_WORKSPACE
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)


def test_split_slow_path(fa):
    """Key rows scaled by 8 in every range: the reference max moves inside
    ranges, and the ranges' LSEs differ widely before the merge."""
    full_case(fa, 1, 512, 8192, 4, 2, 128, False, "f16", seed=23, boost=0.01, split=True)


@pytest.mark.parametrize("case", ["scale1", "kboost"])
@pytest.mark.parametrize("D", [128, 64])
def test_eight_wave_slow_path(fa, case, D):
    """Logits large enough that the reference max moves often (the slow
    path): scale 1 on N(0, 1) inputs; 1% of key rows scaled by 8.  fp16:
    with scale 1 the softmax is nearly one-hot and bf16 rounding of P and O
    alone reaches the 2e-2 bound (both kernels measure about 2e-2 there)."""
    if compute_units() == 256:
        assert plan(fa, 1, 512, 512, 256, 128, D, True, False)[0] == fa.FA_KERNEL_EIGHT_WAVE
    if case == "scale1":
        full_case(fa, 1, 512, 512, 256, 128, D, True, "f16", seed=21, scale=1.0)
    else:
        full_case(fa, 1, 256, 1024, 256, 8, D, True, "f16", seed=22, boost=0.01)


# ---------------------------------------------------------------------------
# the five named workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", workloads.WORKLOADS + workloads.SPLIT_WORKLOADS,
                         ids=[w.name for w in workloads.WORKLOADS + workloads.SPLIT_WORKLOADS])
def test_named_workload(fa, w, parity_figures):
    """Every output element of the workload at full size against the oracle
    over all B*Hq*Sq rows (the split workloads through fa_fwd_ws, as the
    benchmark runs them)."""
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gpu(fa, q, k, v, w.causal, w.scale, split=w in workloads.SPLIT_WORKLOADS)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, lse_ref, w.name, figures=parity_figures)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", workloads.HEAD_DIM_WORKLOADS,
                         ids=[w.name for w in workloads.HEAD_DIM_WORKLOADS])
def test_head_dim_workload(fa, w, parity_figures):
    """The head-dimension workloads (D = 64 on the four-wave and the
    eight-wave kernel, D = 192 and 256 on the tile kernel) at full size,
    every output element against the oracle."""
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gpu(fa, q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, lse_ref, w.name, figures=parity_figures)


@pytest.mark.parametrize("w", workloads.WORKLOADS[2:], ids=[w.name for w in workloads.WORKLOADS[2:]])
def test_named_workload_v_ones_property(fa, w):
    """V = 1 makes every output row 1 (the weights of a row sum to one); this
    covers every output element of the full-size workloads."""
    q, k, v = workloads.workload_inputs(w)
    v = torch.ones_like(v)
    o, _ = run_gpu(fa, q, k, v, w.causal, w.scale, with_lse=False)
    d = np.abs(o - 1.0)
    assert d.max() <= MAX_DO and d.mean() <= MEAN_DO, (d.max(), d.mean())
