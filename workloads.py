"""Seeded synthetic inputs for the attention forward pass.

This module holds no attention arithmetic: it only draws the input tensors.
It is the one piece the oracle side and the HIP side share (tests, smoke
check and benchmark call it for both).

The inputs follow the workloads the pages measure on: i.i.d. N(0, 1) query,
key and value tensors (the JAX Pallas FlashAttention3 page's ``main`` draws
``jax.random.normal`` f16 tensors from key 42), rounded once to the working
dtype with round-to-nearest-even.  The five named workloads below give the
shapes; one of them scales 1% of the key rows by 8 to stress the running max.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    dtype: str            # "bf16" or "f16"
    seed: int
    k_row_boost_frac: float = 0.0   # fraction of key rows multiplied by 8

    @property
    def scale(self) -> float:
        # 1/sqrt(D), as an fp32 value (the library takes scale as float).
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch_dtype(self.dtype)

    def as_dict(self) -> dict:
        d = asdict(self)
        d["scale"] = self.scale
        return d


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f16": torch.float16}[name]


# The five workloads, smallest first.  Seeds are 42 + position.
WORKLOADS = [
    Workload("causal_b1_h1_s256_d64_bf16", 1, 1, 1, 256, 256, 64, True, "bf16", 42),
    Workload("noncausal_b4_h16_s1024_d128_bf16", 4, 16, 16, 1024, 1024, 128, False, "bf16", 43),
    Workload("causal_b2_h32_s4096_d128_bf16", 2, 32, 32, 4096, 4096, 128, True, "bf16", 44),
    Workload("causal_gqa_b1_hq32_hkv8_s8192_d128_bf16", 1, 32, 8, 8192, 8192, 128, True, "bf16", 45),
    Workload("causal_gqa_prefill_b1_hq64_hkv8_sq2048_skv32768_d128_f16_kboost",
             1, 64, 8, 2048, 32768, 128, True, "f16", 46, k_row_boost_frac=0.01),
]
# Shapes outside the five above that exercise the split key ranges: few
# (batch, q-head, 512-row query tile) items over long key ranges, the
# short-prefill / long-context case of the kernbench GQA prefill page.
SPLIT_WORKLOADS = [
    Workload("causal_gqa_shortprefill_b1_hq8_hkv1_sq1024_skv32768_d128_bf16",
             1, 8, 1, 1024, 32768, 128, True, "bf16", 47),
    Workload("causal_gqa_shortprefill_b1_hq32_hkv8_sq512_skv16384_d128_bf16",
             1, 32, 8, 512, 16384, 128, True, "bf16", 48),
]
# Decode-shaped calls: one query row per sequence over a long key range, the
# q-heads of each kv-head packed into one block of rows (memory-bound: K and V
# are read once).
DECODE_WORKLOADS = [
    Workload("decode_gqa_b16_hq32_hkv8_sq1_skv32768_d128_bf16",
             16, 32, 8, 1, 32768, 128, True, "bf16", 49),
    Workload("decode_gqa_b1_hq64_hkv8_sq1_skv32768_d128_bf16",
             1, 64, 8, 1, 32768, 128, True, "bf16", 50),
]
# The other head dimensions the JAX Pallas FlashAttention3 page's `main`
# sweeps (64, 256) at its B = 1, 16 heads, S = 4096 causal shape.
HEAD_DIM_WORKLOADS = [
    Workload("causal_b1_h16_s4096_d64_bf16", 1, 16, 16, 4096, 4096, 64, True, "bf16", 51),
    Workload("causal_b1_h16_s4096_d256_bf16", 1, 16, 16, 4096, 4096, 256, True, "bf16", 52),
    # the multiple of 64 between them (the page's forward takes any)
    Workload("causal_b1_h16_s4096_d192_bf16", 1, 16, 16, 4096, 4096, 192, True, "bf16", 54),
    # the headline shape at head dimension 64 (enough 512-row items for the
    # eight-wave kernel)
    Workload("causal_b2_h32_s4096_d64_bf16", 2, 32, 32, 4096, 4096, 64, True, "bf16", 53),
]
BY_NAME = {w.name: w for w in WORKLOADS + SPLIT_WORKLOADS + DECODE_WORKLOADS + HEAD_DIM_WORKLOADS}

# The headline benchmark workload: causal, D=128, bf16, S=4096.
HEADLINE = WORKLOADS[2]


def get(spec: str) -> Workload:
    """A named workload, or an ad-hoc shape "B,Hq,Hkv,Sq,Skv,D,causal,dtype"
    (causal 0 or 1, dtype bf16 or f16) with seeded N(0, 1) inputs."""
    if spec in BY_NAME:
        return BY_NAME[spec]
    f = spec.split(",")
    if len(f) != 8 or f[7] not in ("bf16", "f16") or f[6] not in ("0", "1"):
        raise ValueError(f"not a workload name or B,Hq,Hkv,Sq,Skv,D,causal,dtype: {spec!r}")
    B, Hq, Hkv, Sq, Skv, D = (int(x) for x in f[:6])
    causal = f[6] == "1"
    name = (f"{'causal' if causal else 'noncausal'}_b{B}_hq{Hq}_hkv{Hkv}_sq{Sq}_skv{Skv}"
            f"_d{D}_{f[7]}")
    return Workload(name, B, Hq, Hkv, Sq, Skv, D, causal, f[7], 100)


def make_inputs(B, Sq, Skv, Hq, Hkv, D, dtype="bf16", seed=0,
                k_row_boost_frac=0.0, dist="normal"):
    """Draw q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] on the CPU.

    Draw order: q, k, v as fp32 ``randn`` from one generator seeded with
    ``seed``, each rounded to ``dtype`` (round-to-nearest-even).  With
    ``k_row_boost_frac`` > 0, a fourth draw (``randperm`` over the B*Skv*Hkv
    key rows) picks round(frac * rows) rows that are multiplied by 8; the
    multiplication is exact (a power of two, far from overflow).

    ``dist`` = "normal" (default) or "uniform" (U(-1, 1), for extra tests).
    """
    g = torch.Generator().manual_seed(int(seed))
    td = torch_dtype(dtype)

    def draw(shape):
        if dist == "normal":
            x = torch.randn(shape, generator=g, dtype=torch.float32)
        elif dist == "uniform":
            x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
        else:
            raise ValueError(dist)
        return x.to(td)

    q = draw((B, Sq, Hq, D))
    k = draw((B, Skv, Hkv, D))
    v = draw((B, Skv, Hkv, D))
    if k_row_boost_frac > 0.0:
        nrows = B * Skv * Hkv
        nboost = int(round(k_row_boost_frac * nrows))
        idx = torch.randperm(nrows, generator=g)[:nboost]
        kr = k.view(nrows, D)
        kr[idx] = (kr[idx].float() * 8.0).to(td)
    return q, k, v


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D, w.dtype, w.seed,
                       w.k_row_boost_frac)


def attention_flops(B, Sq, Skv, Hq, D, causal) -> float:
    """Matmul FLOPs of the two products over the visible (query, key) pairs.

    4*B*Hq*Sq*Skv*D without a mask, halved for a square causal mask (the JAX
    page's ``main`` count).  For a bottom-right causal mask with Sq < Skv the
    masked triangle Sq*Sq/2 is subtracted, which gives exactly one half when
    Sq == Skv.
    """
    if not causal:
        return 4.0 * B * Hq * Sq * Skv * D
    if Sq == Skv:
        return 4.0 * B * Hq * Sq * Skv * D / 2.0
    if Sq < Skv:
        return 4.0 * B * Hq * D * (Sq * Skv - Sq * Sq / 2.0)
    # Sq > Skv: rows i < Sq - Skv see nothing; the rest see a triangle plus.
    return 4.0 * B * Hq * D * (Skv * Skv / 2.0)
