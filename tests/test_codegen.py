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


def test_waves_drain_loads_before_ending(text):
    """Before every s_endpgm, an s_waitcnt vmcnt(0) with no load (and no
    branch target) after it: no load into LDS may outlive the workgroup that
    owns the LDS.  Stores may still be in flight."""
    for name, (body, _) in kernels(text).items():
        raw = [l for l in body]
        for i, l in enumerate(raw):
            if l != "s_endpgm":
                continue
            j = i - 1
            while raw[j] != "s_waitcnt vmcnt(0)":
                assert not raw[j].startswith("buffer_load"), (name, raw[j])
                j -= 1
                assert j > 0, name


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


# ---- the backward's DMA address stream, executed on the CPU ----------------

class Salu:
    """Executes the scalar instructions of generated code (the subset the
    backward's set-up and DMA use); vector instructions are skipped except
    v_readfirstlane (which gives the wave's first lane id).  Records the
    descriptor and M0 of every buffer load into LDS."""

    def __init__(self, kernarg, wave):
        self.s = [0] * 128
        self.m0 = 0
        self.scc = 0
        self.kernarg = kernarg
        self.wave = wave
        self.loads = []

    def val(self, x):
        if x.startswith("s") and x[1:].isdigit():
            return self.s[int(x[1:])]
        if x == "m0":
            return self.m0
        return int(x, 0) & 0xffffffff

    def set(self, d, v):
        v &= 0xffffffff
        if d == "m0":
            self.m0 = v
        else:
            self.s[int(d[1:])] = v

    def run(self, lines):
        labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
        i = 0
        while i < len(lines):
            l = lines[i]
            i += 1
            if not l or l.endswith(":") or l.startswith((";", ".")):
                continue
            op, _, rest = l.partition(" ")
            a = [x.strip() for x in rest.split(",")] if rest else []
            sgn = lambda v: v - (1 << 32) if v & (1 << 31) else v
            if op == "s_load_dwordx16":
                lo = int(a[0][2:].split(":")[0])
                off = int(a[2], 0) // 4
                for k in range(16):
                    self.s[lo + k] = self.kernarg[off + k]
            elif op == "v_readfirstlane_b32":
                self.set(a[0], 64 * self.wave)
            elif op in ("s_mov_b32",):
                self.set(a[0], self.val(a[1]))
            elif op == "s_add_u32":
                r = self.val(a[1]) + self.val(a[2]); self.scc = r >> 32; self.set(a[0], r)
            elif op == "s_addc_u32":
                r = self.val(a[1]) + self.val(a[2]) + self.scc; self.scc = r >> 32; self.set(a[0], r)
            elif op == "s_sub_u32":
                r = self.val(a[1]) - self.val(a[2]); self.scc = int(r < 0); self.set(a[0], r)
            elif op == "s_add_i32":
                self.set(a[0], sgn(self.val(a[1])) + sgn(self.val(a[2])))
            elif op == "s_sub_i32":
                self.set(a[0], sgn(self.val(a[1])) - sgn(self.val(a[2])))
            elif op == "s_mul_i32":
                self.set(a[0], sgn(self.val(a[1])) * sgn(self.val(a[2])))
            elif op == "s_mul_hi_u32":
                self.set(a[0], (self.val(a[1]) * self.val(a[2])) >> 32)
            elif op in ("s_lshl_b32", "s_lshr_b32", "s_ashr_i32", "s_and_b32", "s_xor_b32", "s_or_b32"):
                x, y = self.val(a[1]), self.val(a[2])
                r = {"s_lshl_b32": x << (y & 31), "s_lshr_b32": x >> (y & 31), "s_ashr_i32": sgn(x) >> (y & 31),
                     "s_and_b32": x & y, "s_xor_b32": x ^ y, "s_or_b32": x | y}[op]
                self.scc = int((r & 0xffffffff) != 0); self.set(a[0], r)
            elif op in ("s_min_u32", "s_max_u32"):
                self.set(a[0], (min if op == "s_min_u32" else max)(self.val(a[1]), self.val(a[2])))
            elif op in ("s_min_i32", "s_max_i32"):
                self.set(a[0], (min if op == "s_min_i32" else max)(sgn(self.val(a[1])), sgn(self.val(a[2]))))
            elif op.startswith("s_cmp_"):
                kind, ty = op[6:].split("_")
                x, y = self.val(a[0]), self.val(a[1])
                if ty == "i32":
                    x, y = sgn(x), sgn(y)
                self.scc = int({"eq": x == y, "lg": x != y, "lt": x < y, "le": x <= y, "gt": x > y, "ge": x >= y}[kind])
            elif op == "s_cselect_b32":
                self.set(a[0], self.val(a[1]) if self.scc else self.val(a[2]))
            elif op == "s_cbranch_scc1":
                if self.scc:
                    i = labels[a[0]]
            elif op == "s_cbranch_scc0":
                if not self.scc:
                    i = labels[a[0]]
            elif op == "s_branch":
                i = labels[a[0]]
            elif op.startswith("buffer_load") and l.endswith(" lds"):
                d = int(a[1][2:].split(":")[0])
                base = self.s[d] | ((self.s[d + 1] & 0xffff) << 32)
                self.loads.append((base, self.s[d + 2], self.m0, op))
            elif op.startswith(("s_waitcnt", "s_nop", "s_barrier")) or op.startswith(("v_", "buffer_", "ds_")):
                pass
            else:
                raise AssertionError(f"unhandled scalar instruction: {l}")


def _dma_stream(kind, D, shape, wave, steps):
    """Run the kernel's set-up and `steps` DMA issues on the CPU; returns the
    recorded loads and the generator."""
    B, Sq, Skv, Hq, Hkv, causal, blk, head, b = shape
    g = GenBwd(kind, "bf16", D)
    g.alloc()
    g.setup()
    if kind == "dkv":
        g.lane_consts()
    g.dma_init()
    for _ in range(steps):
        g.emit_dma()
    lines = [l.strip() for l in g.em.text().splitlines()]
    # kernel arguments: pointers at distinct, far-apart bases
    P = {n: (i + 1) << 40 for i, n in enumerate(("q", "k", "v", "do", "l2", "dl", "dq", "dk", "dv"))}
    karg = []
    for n in ("q", "k", "v", "do", "l2", "dl", "dq", "dk", "dv"):
        karg += [P[n] & 0xffffffff, P[n] >> 32]
    nqb128 = (Sq + 127) // 128
    g_ = Hq // Hkv
    magic = (1 << 20) // g_ + 1
    karg += [B, Sq, Skv, Hq, Hkv, causal, 0x3f000000, 0x3f000000, nqb128, magic, g_, 0, 0, 0, 0]
    karg += [0] * (32 - len(karg))
    m = Salu(karg, wave)
    m.s[2], m.s[3], m.s[4] = head, b, blk              # workgroup ids (heads, batch, blocks)
    m.run(lines)
    return m.loads, g, P


@pytest.mark.parametrize("shape", [
    # B, Sq, Skv, Hq, Hkv, causal, block, head, batch
    (2, 517, 517, 8, 2, 1, 2, 1, 1),     # GQA 4, ragged, causal, blocks past the diagonal
    (1, 300, 700, 16, 1, 1, 0, 0, 0),    # sixteen q-heads per kv-head, bottom-right offset
    (3, 130, 77, 2, 2, 0, 0, 1, 2),      # non-causal, Skv < 128
    (1, 4096, 4096, 32, 32, 1, 5, 31, 0),
    # a batch slice of q just under 2 GiB at D = 128: the step from a q-head's
    # last query block back to the next q-head's first is -2.14e9 bytes, near
    # the signed 32-bit limit, and batch 1 starts 2.1e9 bytes in
    (2, 65472, 65472, 128, 64, 0, 500, 63, 1),
])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("wave", [0, 1, 3])
def test_dkv_dma_stream(shape, D, wave):
    """dK/dV: step d loads 64 rows of Q and dO of (q-head hk*g + j, query block
    qb), j outer and qb inner from the first block with a row that sees the
    workgroup's keys; rows past Sq and steps past the last are out of range
    (0 bytes); waves 0 / 1 load l2 / delta of those rows."""
    B, Sq, Skv, Hq, Hkv, causal, kb, hk, b = shape
    g_ = Hq // Hkv
    off = Skv - Sq
    qb0 = max(0, kb * 128 - off) // 64 if causal else 0
    nqb = (Sq + 63) // 64
    n = max(nqb - qb0, 0) * g_
    steps = n + 3
    loads, gen, P = _dma_stream("dkv", D, shape, wave, steps)
    rowb = Hq * D * 2
    dpw, tile = gen.DPW, gen.TILE
    per = 2 * dpw + (1 if wave < 2 else 0)
    assert len(loads) == steps * per
    seq = [(j, qb) for j in range(g_) for qb in range(qb0, nqb)]
    for d in range(steps):
        ld = loads[d * per:(d + 1) * per]
        if d < n:
            j, qb = seq[d]
            rows = min(Sq - 64 * qb, 64)
            qbase = ((b * Sq + 64 * qb) * Hq + hk * g_ + j) * D * 2
            want = [(P["q"] + qbase, rows * rowb)] * dpw + [(P["do"] + qbase, rows * rowb)] * dpw
            lrow = ((b * Hq + hk * g_ + j) * Sq + 64 * qb) * 4
            if wave < 2:
                want.append(((P["l2"] if wave == 0 else P["dl"]) + lrow, rows * 4))
        else:
            want = None
        stage = d % 4
        for i, (base, rec, m0, op) in enumerate(ld):
            if want is None:
                assert rec == 0, (d, i)
            else:
                assert (base, rec) == want[i], (d, i, hex(base), rec, want[i])
            if i < 2 * dpw:
                region = 0 if i < dpw else gen.REG_B
                assert m0 == region + stage * tile + (wave * dpw + i % dpw) * 1024, (d, i, m0)
            else:
                assert m0 == gen.REG_L + wave * 4 * 256 + stage * 256, (d, i, m0)


@pytest.mark.parametrize("shape", [
    (2, 517, 517, 8, 2, 1, 0, 5, 1),     # the last query block (counted from the last): block 0 of x
    (1, 300, 700, 16, 1, 1, 1, 15, 0),
    (3, 130, 77, 2, 2, 0, 0, 1, 2),
    (1, 4096, 4096, 32, 8, 1, 3, 17, 0),
    # a batch slice of k just under 2 GiB at D = 128 (the longest block: 1023 tiles)
    (2, 65472, 65472, 128, 128, 1, 0, 127, 1),
])
@pytest.mark.parametrize("D", [128, 64])
def test_dq_dma_stream(shape, D):
    """dQ: step d loads key tile d (64 rows of K and V of kv-head hq / g) up to
    the last key a row of the workgroup's block sees; keys past Skv and steps
    past the last are out of range."""
    B, Sq, Skv, Hq, Hkv, causal, x, hq, b = shape
    g_ = Hq // Hkv
    hk = hq // g_
    nqb128 = (Sq + 127) // 128
    r0 = (nqb128 - 1 - x) * 128
    kend = min(Skv, min(Sq, r0 + 128) + Skv - Sq) if causal else Skv
    n = (max(kend, 0) + 63) // 64
    steps = n + 3
    loads, gen, P = _dma_stream("dq", D, shape, 1, steps)
    rowb = Hkv * D * 2
    dpw, tile = gen.DPW, gen.TILE
    assert len(loads) == steps * 2 * dpw
    for d in range(steps):
        for i, (base, rec, m0, op) in enumerate(loads[d * 2 * dpw:(d + 1) * 2 * dpw]):
            if d < n:
                kbase = ((b * Skv + 64 * d) * Hkv + hk) * D * 2
                want = (P["k"] if i < dpw else P["v"]) + kbase
                assert (base, rec) == (want, min(Skv - 64 * d, 64) * rowb), (d, i)
            else:
                assert rec == 0
            region = 0 if i < dpw else gen.REG_B
            assert m0 == region + (d % 4) * tile + (1 * dpw + i % dpw) * 1024
