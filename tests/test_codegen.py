"""CPU checks of the generated gfx950 assembly (no GPU): the code object
assembles, and properties every kernel must have hold on the generated
text -- the wait states and wait counts that the hardware leaves to
software, register and LDS budgets, and the backward kernels' barrier
structure.  Plus unit checks of the emitter (asm/regs.py) that inserts them.
"""
import os
import re
import subprocess

import pytest

from attention_forward_05_amd.asm import fa_fwd_gen
from attention_forward_05_amd.asm.fa_bwd_gen import GenBwd, VARIANTS as BWD_VARIANTS
from attention_forward_05_amd.asm.regs import Emitter, MFMA_TO_OTHER

LDS_BYTES = 160 * 1024
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "bin", "clang")


@pytest.fixture(scope="module")
def text():
    return fa_fwd_gen.generate_all()


def kernels(text):
    """{name: (body lines, descriptor dict)} of every kernel in the text."""
    out = {}
    for m in re.finditer(r"\t\.globl (\S+)\n", text):
        name = m.group(1)
        i = m.end()
        j = text.index(f"\t.amdhsa_kernel {name}", i)
        k = text.index("\t.end_amdhsa_kernel", j)
        desc = dict(re.findall(r"\.amdhsa_(\w+) (\d+)", text[j:k]))
        body = [l.strip() for l in text[i:j].splitlines()]
        out[name] = ([l for l in body if l and not l.startswith((".", ";"))], desc)
    return out


def test_every_kernel_is_generated(text):
    names = set(kernels(text))
    assert len(names) == 18
    for kind, dt, D in BWD_VARIANTS:
        assert f"fa_bwd_{kind}_{dt}_d{D}_gfx950" in names


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no ROCm clang")
def test_code_object_assembles(text, tmp_path):
    src = tmp_path / "k.s"
    src.write_text(text)
    r = subprocess.run([CLANG, "-x", "assembler", "-target", "amdgcn-amd-amdhsa", "-mcpu=gfx950", "-c",
                        str(src), "-o", str(tmp_path / "k.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]


def test_budgets(text):
    """Registers (VGPR + AGPR) within a SIMD lane's 512, accumulator offset on
    a 4-register boundary, LDS within the compute unit's 160 KB."""
    for name, (_, d) in kernels(text).items():
        total, acc = int(d["next_free_vgpr"]), int(d["accum_offset"])
        assert total <= 512 and acc % 4 == 0 and acc <= total, name
        assert int(d["group_segment_fixed_size"]) <= LDS_BYTES, name


def test_no_packed_fp32_alu(text):
    """No packed fp32 VALU instruction anywhere (they are not to be used)."""
    ops = {l.split()[0] for body, _ in kernels(text).values() for l in body}
    assert not {o for o in ops if re.fullmatch(r"v_pk_(add|mul|fma)_f32", o)}


def test_lds_dma_after_m0_with_a_wait_state(text):
    """Every load into LDS (buffer_load ... lds) comes after an M0 write with
    one instruction between them (the GFX9 wait state between an SALU write
    of M0 and an LDS DMA)."""
    for name, (body, _) in kernels(text).items():
        for i, l in enumerate(body):
            if l.startswith("buffer_load") and l.endswith(" lds"):
                assert body[i - 1].startswith("s_nop") and " m0," in body[i - 2], (name, i, body[i - 2:i + 1])


def test_waves_drain_memory_before_ending(text):
    """s_waitcnt vmcnt(0) right before every s_endpgm: no load into LDS may
    outlive the workgroup that owns the LDS."""
    for name, (body, _) in kernels(text).items():
        for i, l in enumerate(body):
            if l == "s_endpgm":
                assert body[i - 1] == "s_waitcnt vmcnt(0)", name


def test_backward_step_structure():
    """The backward's step loop: three mask variants, each with exactly one
    barrier (every wave of a workgroup runs the same number of steps), and
    as many MFMAs per step as the design gives (dK/dV 4 x 16, dQ 2 x 16 +
    2 x 8 at D = 128)."""
    for kind, dt, D in BWD_VARIANTS:
        g = GenBwd(kind, dt, D)
        txt, _ = g.assemble_text()
        lines = [l.strip() for l in txt.splitlines()]
        heads = [i for i, l in enumerate(lines) if re.match(r"\.Lbwd_\w+_(ff|mf|mm)_\d+:", l)]
        assert len(heads) == 3, (kind, dt, D)
        end = [i for i, l in enumerate(lines) if re.match(r"\.Lbwd_\w+_exit_\d+:", l)][0]
        for a, b in zip(heads, heads[1:] + [end]):
            seg = lines[a:b]
            assert sum(l == "s_barrier" for l in seg) == 1
            nq, nd = D // 16, D // 32
            want = (2 * 2 * nq + 2 * 4 * nd) if kind == "dkv" else (2 * 2 * nq + 2 * 2 * nd)
            assert sum(l.startswith("v_mfma") for l in seg) == want, (kind, dt, D)


# ---- the emitter ------------------------------------------------------------

def test_emitter_pads_mfma_result_reads():
    em = Emitter()
    em.mfma("v_mfma_f32_32x32x16_bf16", "v[0:15]", "v[16:19]", "v[20:23]", "0")
    em.valu("v_mov_b32 v30, v3", dst=["v30"], src=["v3"])
    nops = sum(int(m) + 1 for m in re.findall(r"s_nop (\d+)", em.text()))
    assert nops + 1 >= MFMA_TO_OTHER          # the MFMA itself counts as one


def test_emitter_counts_lds_reads_in_order():
    em = Emitter()
    for r in range(4):
        em.ds_read(f"ds_read_b128 v[{4 * r}:{4 * r + 3}], v40", f"v[{4 * r}:{4 * r + 3}]", "v40")
    em.valu("v_mov_b32 v50, v5", dst=["v50"], src=["v5"])      # the second read's result
    assert "s_waitcnt lgkmcnt(2)" in em.text()


def test_emitter_rejects_an_mfma_result_as_operand():
    em = Emitter()
    em.mfma("v_mfma_f32_32x32x16_bf16", "v[0:15]", "v[16:19]", "v[20:23]", "0")
    with pytest.raises(AssertionError):
        em.mfma("v_mfma_f32_32x32x16_bf16", "v[24:39]", "v[0:3]", "v[20:23]", "0")
