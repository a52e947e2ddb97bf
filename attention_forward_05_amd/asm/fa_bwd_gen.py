"""Generator of the gfx950 (MI355X) attention backward kernels: dK/dV and dQ.

The backward of the JAX Pallas FlashAttention3 page (`kernel_dkv`,
`kernel_dq`), with this library's scale and its LSE in log2 units
(l2 = LSE * log2(e), written beside delta by the HIP delta kernel):

    P  = 2^(c*S - l2)      (c = scale * log2(e); S = q.k)
    dS = P * (dP - delta)  (dP = dO.v)
    dV = P^T.dO,  dK = scale * dS^T.Q   (summed over the q-heads of a kv-head)
    dQ = scale * dS.K

P and dS are rounded to the input dtype before the products that read them;
every product accumulates in fp32.

Both kernels have one wave per SIMD (four per workgroup) and the same
organisation.  A wave keeps its 32 columns' operands in the accumulator
registers for the whole kernel (dK/dV: its 32 keys' K and V rows; dQ: its
32 query rows' Q and dO rows) next to its fp32 gradient accumulators, and
streams 64-row tiles of the other side (dK/dV: Q and dO blocks of one
q-head, with their l2 and delta; dQ: K and V tiles) HBM -> LDS by
buffer_load ... lds into four LDS stages, two tiles ahead.  Each 32-row
half g of a tile takes

    X(g): S and dP, the rows of the tile against the wave's columns
          (dK/dV: C[row][key]; dQ: C[key][row]), 16 MFMAs
    Y(g): P and dS from S and dP (vector ALU, exponentials), rounded
    Z(g): the gradient products with the tile read transposed
          (dK/dV: dV += dO^T.P, dK += Q^T.dS, 16 MFMAs;
           dQ: dQ += K^T.dS, 8 MFMAs)

and the MFMA blocks run in the order X(g), Z(g-1), X(g+1), Z(g), ...
with Y(g) spread over the two blocks between X(g) and Z(g), so that the
vector work of one half runs next to the MFMAs of its neighbours.  A
half whose elements the causal mask leaves all visible runs without the
mask.  Operand reads from LDS run a few MFMAs ahead through a ring of
registers, also across the step loop's back-edge.
"""
from __future__ import annotations

from .regs import Alloc, Emitter, Op

NST = 4             # LDS stages (tiles) in flight
KERNARG_BYTES = 128


def kernel_name(kind: str, dtype: str, D: int) -> str:
    return f"fa_bwd_{kind}_{dtype}_d{D}_gfx950"


class Item:
    """One MFMA and the LDS reads of its A operand (into a ring buffer)."""

    def __init__(self, reads, mfma):
        self.reads, self.mfma = reads, mfma


class Block4:
    """Four consecutive registers of a larger block."""

    def __init__(self, blk, off):
        self.blk, self.off = blk, off

    def r(self, i=0, n=1):
        return self.blk.r(self.off + i, n)


class GenBwd:

    def __init__(self, kind: str, dtype: str, D: int):
        assert kind in ("dkv", "dq") and dtype in ("bf16", "f16") and D in (64, 128)
        self.kind, self.dtype, self.D = kind, dtype, D
        self.dkv = kind == "dkv"
        self.ROW = 2 * D                        # bytes of one row
        self.TILE = 64 * self.ROW               # bytes of one 64-row tile
        self.NQ = D // 16                       # k-steps of S and dP
        self.ND = D // 32                       # 32-dim blocks of the gradients
        self.CPR = self.ROW // 16               # 16-byte chunks per row
        self.RPI = 1024 // self.ROW             # rows per DMA instruction
        self.DPW = self.TILE // 1024 // 4       # DMA instructions per wave per tile
        self.REG_B = NST * self.TILE            # LDS: second tensor's stages
        self.REG_L = 2 * NST * self.TILE        # LDS: l2 stages, then delta stages (dK/dV)
        self.LDS = self.REG_L + (2 * NST * 256 if self.dkv else 0)
        # operand buffers (accumulator registers) and the MFMAs whose reads are
        # issued ahead; at most 15 LDS reads are in flight (two per Z MFMA)
        self.RING = 16 if D == 128 else 8
        self.LOOK = 7 if D == 128 else 5
        # MFMAs of a step's first block whose reads the previous step issues
        self.PRE = min(self.LOOK, 2 * self.ND * (2 if self.dkv else 1))
        self.mfma_op = f"v_mfma_f32_32x32x16_{dtype}"
        self.cvt_op = "v_cvt_pk_bf16_f32" if dtype == "bf16" else "v_cvt_pk_f16_f32"
        self.name = kernel_name(kind, dtype, D)
        self.em = Emitter()
        self._lab = 0
        # workgroup ids: the grid is (heads, batch, blocks), so that the
        # blocks with the most work (dK/dV: the first keys; dQ: the last
        # rows) are dispatched first over every head
        self.g_head, self.g_b, self.g_blk = "s2", "s3", "s4"

    def lab(self, tag):
        self._lab += 1
        return f".Lbwd_{self.kind}_{self.dtype}{self.D}_{tag}_{self._lab}"

    # ------------------------------------------------------------------------
    def alloc(self):
        V = Alloc("v", 0, 256)
        A = Alloc("a", 0, 256)
        S = Alloc("s", 40, 102)
        r = self.__dict__
        V.take("lane", 1)                          # v0: the lane id
        r["v_S"] = [V.take(f"S{p}", 16, 4) for p in range(2)]     # S, then P in place
        r["v_P"] = [V.take(f"dP{p}", 16, 4) for p in range(2)]    # dP, then dS in place
        r["v_pk"] = [[V.take(f"pk{p}{t}", 4, 4) for t in range(2)] for p in range(2)]  # P rounded
        r["v_sk"] = [[V.take(f"sk{p}{t}", 4, 4) for t in range(2)] for p in range(2)]  # dS rounded
        if self.dkv:
            r["v_L"] = [V.take(f"L{p}", 16, 4) for p in range(2)]     # l2 of the half's rows
            r["v_Dl"] = [V.take(f"Dl{p}", 16, 4) for p in range(2)]   # delta of the half's rows
        r["v_xa"] = V.take("xa", self.NQ)        # row reads of the first tensor (k-step t)
        r["v_xb"] = V.take("xb", self.NQ)        # row reads of the second tensor
        r["v_za"] = V.take("za", 2 * self.ND)    # transposing reads, first tensor (db, lo/hi)
        if self.dkv:
            r["v_zb"] = V.take("zb", 2 * self.ND)  # transposing reads, second tensor
            r["v_la"] = V.take("la", 1)            # l2 / delta reads
        r["v_dma"] = V.take("dma", self.DPW)
        r["v_dml"] = V.take("dml", 1)
        r["v_col"] = V.take("col", 1)            # dK/dV: key - 4h; dQ: last visible key - 4h
        r["v_tq"] = V.take("tq", 1)
        r["v_ninf"] = V.take("ninf", 1)
        if not self.dkv:
            r["v_l2"] = V.take("l2", 1)
            r["v_dl"] = V.take("dl", 1)
        r["v_so"] = V.take("so", 1)             # the lane's column in the gradient stores
        r["v_t"] = V.take("t", 8, 4)
        self.nvgpr = (V.next + 3) // 4 * 4
        # accumulators and the resident operands
        r["a_acc1"] = [A.take(f"g1{d}", 16, 4) for d in range(self.ND)]   # dK or dQ
        if self.dkv:
            r["a_acc2"] = [A.take(f"g2{d}", 16, 4) for d in range(self.ND)]   # dV
        r["a_f1"] = [A.take(f"f1{t}", 4, 4) for t in range(self.NQ)]   # K or Q rows
        r["a_f2"] = [A.take(f"f2{t}", 4, 4) for t in range(self.NQ)]   # V or dO rows
        r["a_R"] = [A.take(f"R{i}", 4, 4) for i in range(self.RING)]     # operand ring
        self.nagpr = (A.next + 3) // 4 * 4
        t = S.take
        r["s_w"] = t("w", 1)
        r["s_off"] = t("off", 1)
        r["s_n"] = t("nsteps", 1)
        r["s_t"] = t("step", 1)
        r["s_rowb"] = t("rowb", 1)               # row stride of the streamed tensors
        r["s_x"] = [t(f"x{i}", 1) for i in range(8)]
        r["s_ra"] = t("ra", 4, 4)                # DMA descriptors: first tensor
        r["s_rb"] = t("rb", 4, 4)                # second tensor
        r["s_rl"] = t("rl", 4, 4)                # l2 or delta (dK/dV, waves 0 and 1)
        r["s_ro1"] = t("ro1", 4, 4)              # stores (dK / dQ)
        r["s_ro2"] = t("ro2", 4, 4)              # stores (dV)
        r["s_b0"] = t("base0", 2, 2)             # first tensor's base for the current b(, hk)
        r["s_b1"] = t("base1", 2, 2)
        r["s_bl"] = t("basel", 2, 2)
        r["s_ds"] = t("dstep", 1)                # DMA stream: step
        r["s_dq"] = t("dqb", 1)                  # its query block (dK/dV)
        r["s_full"] = t("full", 1)               # bytes of 64 rows of the streamed tensors
        r["s_wd"], r["s_wdh"] = t("wrapd", 1), t("wrapdh", 1)  # base step to the next q-head (64-bit)
        r["s_wdl"] = t("wrapdl", 1)              # the same for l2 / delta
        r["s_wb"], r["s_wl"] = t("wbase", 1), t("wlbase", 1)   # the wave's LDS DMA offsets
        r["s_cq"] = t("cqb", 1)                  # the current step's query block (dK/dV)
        r["s_qb0"], r["s_nqb"] = t("qb0", 1), t("nqb", 1)
        r["s_lim"] = t("lim", 1)                 # dK/dV: the wave's first key; dQ: last key seen by all its rows
        r["s_hk"] = t("hk", 1)
        r["s_q0"], r["s_q1"] = t("q0", 1), t("q1", 1)   # mask offsets of the step's two halves
        self.nsgpr = S.next

    # ------------------------------------------------------------------------
    def emit_swz(self, dst, r, tmp):
        """The LDS chunk swizzle of a row r (the HIP tile kernels' layout):
        D = 128: (r & 15) ^ 4(r & 3); D = 64: ((r >> 1) & 7) ^ 4((r >> 1) & 1)."""
        em = self.em
        if self.D == 128:
            em.valu(f"v_and_b32 {tmp}, 3, {r}", dst=[tmp], src=[r])
            em.valu(f"v_lshlrev_b32 {tmp}, 2, {tmp}", dst=[tmp], src=[tmp])
            em.valu(f"v_and_b32 {dst}, 15, {r}", dst=[dst], src=[r])
        else:
            em.valu(f"v_bfe_u32 {tmp}, {r}, 1, 1", dst=[tmp], src=[r])
            em.valu(f"v_lshlrev_b32 {tmp}, 2, {tmp}", dst=[tmp], src=[tmp])
            em.valu(f"v_bfe_u32 {dst}, {r}, 1, 3", dst=[dst], src=[r])
        em.valu(f"v_xor_b32 {dst}, {dst}, {tmp}", dst=[dst], src=[dst, tmp])

    def mul64(self, lo, hi, a, b):
        self.em.salu(f"s_mul_hi_u32 {hi}, {a}, {b}")
        self.em.salu(f"s_mul_i32 {lo}, {a}, {b}")

    def set_desc(self, rs, blo, bhi, records):
        em = self.em
        em.salu(f"s_mov_b32 {rs.r(0)}, {blo}")
        em.salu(f"s_and_b32 {rs.r(1)}, {bhi}, 0xffff")
        em.salu(f"s_mov_b32 {rs.r(2)}, {records}")
        em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")

    # ------------------------------------------------------------------------
    def setup(self):
        """Arguments, the workgroup's ids and step count, bases and the lane's
        resident operands (loads left in flight)."""
        em = self.em
        em.salu("s_load_dwordx16 s[8:23], s[0:1], 0x0")
        em.salu("s_load_dwordx16 s[24:39], s[0:1], 0x40")
        em.valu(f"v_readfirstlane_b32 {self.s_w}, v0", src=["v0"])
        em.salu(f"s_lshr_b32 {self.s_w}, {self.s_w}, 6")
        em.valu("v_and_b32 v0, 63, v0", dst=["v0"], src=["v0"])
        em.salu("s_waitcnt lgkmcnt(0)")
        # s[8:9] q, [10:11] k, [12:13] v, [14:15] dO, [16:17] l2, [18:19] delta,
        # [20:21] dQ, [22:23] dK, [24:25] dV, s26 B, s27 Sq, s28 Skv, s29 Hq,
        # s30 Hkv, s31 causal, s32 c, s33 scale, s34 query blocks (dQ),
        # s35 group magic, s36 group size
        em.salu(f"s_sub_i32 {self.s_off}, s28, s27")
        em.valu(f"v_mov_b32 {self.v_ninf}, 0xff800000", dst=[str(self.v_ninf)])
        if self.dkv:
            self.setup_dkv()
        else:
            self.setup_dq()

    def setup_dkv(self):
        """Workgroup (key block kb, kv-head hk, batch b): the keys 128*kb ..;
        steps over (q-head of the group, 64-row query block), query blocks
        innermost, from the first block with a row that sees a key."""
        em, x, t = self.em, self.s_x, self.v_t
        D2 = 2 * self.D
        em.salu(f"s_mul_i32 {self.s_rowb}, s29, {D2}")                # Q / dO row stride
        em.salu(f"s_lshl_b32 {x[0]}, {self.g_blk}, 7")                          # k0
        em.salu(f"s_sub_i32 {x[1]}, {x[0]}, {self.s_off}")
        em.salu(f"s_max_i32 {x[1]}, {x[1]}, 0")
        em.salu(f"s_lshr_b32 {x[1]}, {x[1]}, 6")
        em.salu("s_cmp_eq_u32 s31, 0")
        em.salu(f"s_cselect_b32 {self.s_qb0}, 0, {x[1]}")
        em.salu(f"s_add_u32 {self.s_nqb}, s27, 63")
        em.salu(f"s_lshr_b32 {self.s_nqb}, {self.s_nqb}, 6")
        em.salu(f"s_sub_i32 {x[2]}, {self.s_nqb}, {self.s_qb0}")
        em.salu(f"s_max_i32 {x[2]}, {x[2]}, 0")
        em.salu(f"s_mul_i32 {self.s_n}, {x[2]}, s36")
        em.salu(f"s_lshl_b32 {x[3]}, {self.s_w}, 5")
        em.salu(f"s_add_u32 {self.s_lim}, {x[0]}, {x[3]}")           # the wave's first key
        em.salu(f"s_mul_i32 {x[5]}, {self.g_head}, s36")                         # hq0 = hk * g
        # l2 (wave 0) or delta (wave 1) rows of (b, hq0): ((b*Hq + hq0) * Sq) * 4
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s29")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {x[5]}")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s27")
        self.mul64(x[6], x[7], x[4], 4)
        em.salu(f"s_cmp_eq_u32 {self.s_w}, 0")
        em.salu(f"s_cselect_b32 {x[0]}, s16, s18")
        em.salu(f"s_cselect_b32 {x[1]}, s17, s19")
        em.salu(f"s_add_u32 {self.s_bl.r(0)}, {x[0]}, {x[6]}")
        em.salu(f"s_addc_u32 {self.s_bl.r(1)}, {x[1]}, {x[7]}")
        # Q / dO of (b, hq0): ((b*Sq)*Hq + hq0) * 2D
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s27")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s29")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {x[5]}")
        self.mul64(x[6], x[7], x[4], D2)
        for base, ptr in ((self.s_b0, 8), (self.s_b1, 14)):
            em.salu(f"s_add_u32 {base.r(0)}, s{ptr}, {x[6]}")
            em.salu(f"s_addc_u32 {base.r(1)}, s{ptr + 1}, {x[7]}")
        # K / V / dK / dV of (b, hk): ((b*Skv)*Hkv + hk) * 2D, ranges up to
        # the tensor's end (a key past Skv is out of range)
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s28")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s30")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.g_head}")
        self.mul64(x[6], x[7], x[4], D2)
        em.salu(f"s_mul_i32 {x[5]}, s28, s30")
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, {self.g_head}")
        em.salu(f"s_mul_i32 {x[5]}, {x[5]}, {D2}")
        for rs, ptr in ((self.s_ra, 10), (self.s_rb, 12), (self.s_ro1, 22), (self.s_ro2, 24)):
            em.salu(f"s_add_u32 {x[0]}, s{ptr}, {x[6]}")
            em.salu(f"s_addc_u32 {x[1]}, s{ptr + 1}, {x[7]}")
            self.set_desc(rs, x[0], x[1], x[5])
        # the lane's key (its column): K / V rows (a key past the end reads
        # the last key: finite values in a column that is not stored), the
        # store offset, and key - off - 4h for the mask
        em.salu(f"s_mul_i32 {x[2]}, s30, {D2}")                       # K / V row stride
        em.salu(f"s_sub_u32 {x[3]}, s28, 1")
        em.valu(f"v_and_b32 {t.r(0)}, 31, v0", dst=[t.r(0)], src=["v0"])
        em.valu(f"v_add_u32 {t.r(0)}, {self.s_lim}, {t.r(0)}", dst=[t.r(0)], src=[t.r(0)])
        em.valu(f"v_lshrrev_b32 {t.r(1)}, 5, v0", dst=[t.r(1)], src=["v0"])
        em.valu(f"v_min_u32 {t.r(2)}, {x[3]}, {t.r(0)}", dst=[t.r(2)], src=[t.r(0)])
        em.valu(f"v_mul_lo_u32 {t.r(2)}, {t.r(2)}, {x[2]}", dst=[t.r(2)], src=[t.r(2)])
        em.valu(f"v_lshl_add_u32 {t.r(2)}, {t.r(1)}, 4, {t.r(2)}", dst=[t.r(2)], src=[t.r(1), t.r(2)])
        em.valu(f"v_mul_lo_u32 {t.r(3)}, {t.r(0)}, {x[2]}", dst=[t.r(3)], src=[t.r(0)])
        em.valu(f"v_lshl_add_u32 {self.v_so}, {t.r(1)}, 3, {t.r(3)}", dst=[str(self.v_so)], src=[t.r(1), t.r(3)])
        em.valu(f"v_subrev_u32 {t.r(3)}, {self.s_off}, {t.r(0)}", dst=[t.r(3)], src=[t.r(0)])
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 2, {t.r(1)}", dst=[t.r(4)], src=[t.r(1)])
        em.valu(f"v_sub_u32 {self.v_col}, {t.r(3)}, {t.r(4)}", dst=[str(self.v_col)], src=[t.r(3), t.r(4)])
        for frags, rs in ((self.a_f1, self.s_ra), (self.a_f2, self.s_rb)):
            for tt in range(self.NQ):
                em.vmem_load_to(f"buffer_load_dwordx4 {frags[tt]}, {t.r(2)}, {rs}, 0 offen "
                                f"offset:{32 * tt}", str(frags[tt]), src=[t.r(2)])

    def setup_dq(self):
        """Workgroup (query block counted from the last, q-head hq, batch b):
        the rows 128*qb ..; steps over the 64-key tiles they see."""
        em, x, t = self.em, self.s_x, self.v_t
        D2 = 2 * self.D
        em.salu(f"s_mul_i32 {self.s_rowb}, s30, {D2}")                # K / V row stride
        em.salu(f"s_mul_i32 {self.s_hk}, {self.g_head}, s35")
        em.salu(f"s_lshr_b32 {self.s_hk}, {self.s_hk}, 20")           # hk = (hq * magic) >> 20
        em.salu(f"s_sub_u32 {x[0]}, s34, 1")
        em.salu(f"s_sub_u32 {x[0]}, {x[0]}, {self.g_blk}")
        em.salu(f"s_lshl_b32 {x[0]}, {x[0]}, 7")                      # the block's first row
        # causal: a row i sees the keys k <= i + off; offe = off, else Skv
        # (every key)
        em.salu("s_cmp_eq_u32 s31, 0")
        em.salu(f"s_cselect_b32 {x[4]}, s28, {self.s_off}")
        # keys seen by the block: min(Skv, min(Sq, r0 + 128) + offe), at least 0
        em.salu(f"s_add_u32 {x[1]}, {x[0]}, 128")
        em.salu(f"s_min_u32 {x[1]}, {x[1]}, s27")
        em.salu(f"s_add_i32 {x[1]}, {x[1]}, {x[4]}")
        em.salu(f"s_min_i32 {x[1]}, {x[1]}, s28")
        em.salu(f"s_max_i32 {x[1]}, {x[1]}, 0")
        em.salu(f"s_add_u32 {x[1]}, {x[1]}, 63")
        em.salu(f"s_lshr_b32 {self.s_n}, {x[1]}, 6")
        # every row of the wave sees the keys k <= lim = min(r + offe, Skv - 1)
        em.salu(f"s_lshl_b32 {x[2]}, {self.s_w}, 5")
        em.salu(f"s_add_u32 {x[2]}, {x[0]}, {x[2]}")                  # the wave's first row
        em.salu(f"s_sub_u32 {x[3]}, s28, 1")
        em.salu(f"s_add_i32 {self.s_lim}, {x[2]}, {x[4]}")
        em.salu(f"s_min_i32 {self.s_lim}, {self.s_lim}, {x[3]}")
        # per lane: its row qi (the column), its last visible key - 4h
        em.valu(f"v_and_b32 {t.r(0)}, 31, v0", dst=[t.r(0)], src=["v0"])
        em.valu(f"v_add_u32 {t.r(0)}, {x[2]}, {t.r(0)}", dst=[t.r(0)], src=[t.r(0)])
        em.valu(f"v_lshrrev_b32 {t.r(1)}, 5, v0", dst=[t.r(1)], src=["v0"])
        em.valu(f"v_add_u32 {t.r(2)}, {x[4]}, {t.r(0)}", dst=[t.r(2)], src=[t.r(0)])
        em.valu(f"v_min_i32 {t.r(2)}, {x[3]}, {t.r(2)}", dst=[t.r(2)], src=[t.r(2)])
        em.valu(f"v_lshlrev_b32 {t.r(3)}, 2, {t.r(1)}", dst=[t.r(3)], src=[t.r(1)])
        em.valu(f"v_sub_u32 {self.v_col}, {t.r(2)}, {t.r(3)}", dst=[str(self.v_col)], src=[t.r(2), t.r(3)])
        # l2 and delta of (b, hq, qi); a row past Sq reads 0 (its Q and dO
        # are 0 too, so its products are 0)
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s29")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.g_head}")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s27")
        self.mul64(x[6], x[7], x[4], 4)
        em.salu(f"s_lshl_b32 {x[5]}, s27, 2")
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 2, {t.r(0)}", dst=[t.r(4)], src=[t.r(0)])
        for ptr, dst, rs in ((16, self.v_l2, self.s_ra), (18, self.v_dl, self.s_rb)):
            em.salu(f"s_add_u32 {x[0]}, s{ptr}, {x[6]}")
            em.salu(f"s_addc_u32 {x[1]}, s{ptr + 1}, {x[7]}")
            self.set_desc(rs, x[0], x[1], x[5])
            em.vmem_load_to(f"buffer_load_dword {dst}, {t.r(4)}, {rs}, 0 offen", str(dst), src=[t.r(4)])
        # Q / dO rows of (b, qi, hq): base ((b*Sq)*Hq + hq) * 2D, lane qi*rowq + 16h
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s27")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s29")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.g_head}")
        self.mul64(x[6], x[7], x[4], D2)
        em.salu(f"s_mul_i32 {x[2]}, s29, {D2}")                       # Q row stride
        em.salu(f"s_mul_i32 {x[5]}, s27, s29")
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, {self.g_head}")
        em.salu(f"s_mul_i32 {x[5]}, {x[5]}, {D2}")                    # up to the end of q
        em.valu(f"v_mul_lo_u32 {t.r(5)}, {t.r(0)}, {x[2]}", dst=[t.r(5)], src=[t.r(0)])
        em.valu(f"v_lshl_add_u32 {t.r(6)}, {t.r(1)}, 4, {t.r(5)}", dst=[t.r(6)], src=[t.r(1), t.r(5)])
        em.valu(f"v_lshl_add_u32 {self.v_so}, {t.r(1)}, 3, {t.r(5)}", dst=[str(self.v_so)], src=[t.r(1), t.r(5)])
        for frags, ptr, rs in ((self.a_f1, 8, self.s_rl), (self.a_f2, 14, self.s_ro2)):
            em.salu(f"s_add_u32 {x[0]}, s{ptr}, {x[6]}")
            em.salu(f"s_addc_u32 {x[1]}, s{ptr + 1}, {x[7]}")
            self.set_desc(rs, x[0], x[1], x[5])
            for tt in range(self.NQ):
                em.vmem_load_to(f"buffer_load_dwordx4 {frags[tt]}, {t.r(6)}, {rs}, 0 offen "
                                f"offset:{32 * tt}", str(frags[tt]), src=[t.r(6)])
        em.salu(f"s_add_u32 {x[0]}, s20, {x[6]}")
        em.salu(f"s_addc_u32 {x[1]}, s21, {x[7]}")
        self.set_desc(self.s_ro1, x[0], x[1], x[5])                   # dQ stores
        # K / V of (b, hk)
        em.salu(f"s_mul_i32 {x[4]}, {self.g_b}, s28")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s30")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_hk}")
        self.mul64(x[6], x[7], x[4], D2)
        for base, ptr in ((self.s_b0, 10), (self.s_b1, 12)):
            em.salu(f"s_add_u32 {base.r(0)}, s{ptr}, {x[6]}")
            em.salu(f"s_addc_u32 {base.r(1)}, s{ptr + 1}, {x[7]}")

    # ------------------------------------------------------------------------
    def lane_consts(self):
        """LDS addresses of the operand reads and the DMA source offsets."""
        em, t, x = self.em, self.v_t, self.s_x
        lane = "v0"
        l32, h = t.r(0), t.r(1)
        em.valu(f"v_and_b32 {l32}, 31, {lane}", dst=[l32], src=[lane])
        em.valu(f"v_lshrrev_b32 {h}, 5, {lane}", dst=[h], src=[lane])
        # row reads, k-step t: row l32, chunk (2t + h) ^ swz(l32)
        #   = l32*ROW + ((h ^ swz(l32)) << 4) ^ (t << 5)
        self.emit_swz(t.r(2), l32, t.r(3))
        em.valu(f"v_xor_b32 {t.r(2)}, {t.r(2)}, {h}", dst=[t.r(2)], src=[t.r(2), h])
        em.valu(f"v_mul_u32_u24 {t.r(3)}, {self.ROW}, {l32}", dst=[t.r(3)], src=[l32])
        em.valu(f"v_lshl_add_u32 {t.r(4)}, {t.r(2)}, 4, {t.r(3)}", dst=[t.r(4)], src=[t.r(2), t.r(3)])
        for tt in range(self.NQ):
            xa, xb = self.v_xa.r(tt), self.v_xb.r(tt)
            em.valu(f"v_xor_b32 {xa}, {tt << 5}, {t.r(4)}", dst=[xa], src=[t.r(4)])
            em.valu(f"v_add_u32 {xb}, {self.REG_B}, {xa}", dst=[xb], src=[xa])
        # transposing reads (A operand of dims 32db.., rows 16ts.. of a half):
        # row r_e = 4h + ((lane & 15) >> 2) + 8e, chunk (4db + c0) ^ swz(r_e)
        # with c0 = 2((lane >> 4) & 1) + ((lane >> 1) & 1), byte 8(lane & 1);
        # 4db enters as ^ (db << 6).  Set to the stage before the first.
        em.valu(f"v_bfe_u32 {t.r(2)}, {lane}, 2, 2", dst=[t.r(2)], src=[lane])
        em.valu(f"v_lshl_add_u32 {t.r(2)}, {h}, 2, {t.r(2)}", dst=[t.r(2)], src=[h, t.r(2)])
        em.valu(f"v_bfe_u32 {t.r(3)}, {lane}, 4, 1", dst=[t.r(3)], src=[lane])
        em.valu(f"v_bfe_u32 {t.r(4)}, {lane}, 1, 1", dst=[t.r(4)], src=[lane])
        em.valu(f"v_lshl_add_u32 {t.r(3)}, {t.r(3)}, 1, {t.r(4)}", dst=[t.r(3)], src=[t.r(3), t.r(4)])
        em.valu(f"v_and_b32 {t.r(4)}, 1, {lane}", dst=[t.r(4)], src=[lane])
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 3, {t.r(4)}", dst=[t.r(4)], src=[t.r(4)])
        for e in range(2):
            r_, sw, a_ = t.r(5), t.r(6), t.r(7)
            em.valu(f"v_add_u32 {r_}, {8 * e}, {t.r(2)}", dst=[r_], src=[t.r(2)])
            self.emit_swz(sw, r_, a_)
            em.valu(f"v_xor_b32 {sw}, {sw}, {t.r(3)}", dst=[sw], src=[sw, t.r(3)])
            em.valu(f"v_mul_u32_u24 {a_}, {self.ROW}, {r_}", dst=[a_], src=[r_])
            em.valu(f"v_lshl_add_u32 {a_}, {sw}, 4, {a_}", dst=[a_], src=[sw, a_])
            em.valu(f"v_add_u32 {a_}, {a_}, {t.r(4)}", dst=[a_], src=[a_, t.r(4)])
            em.valu(f"v_add_u32 {a_}, {(NST - 1) * self.TILE}, {a_}", dst=[a_], src=[a_])
            for db in range(self.ND):
                z = self.v_za.r(2 * db + e)
                em.valu(f"v_xor_b32 {z}, {db << 6}, {a_}", dst=[z], src=[a_])
                if self.dkv:
                    zb = self.v_zb.r(2 * db + e)
                    em.valu(f"v_add_u32 {zb}, {self.REG_B}, {z}", dst=[zb], src=[z])
        if self.dkv:
            em.salu(f"s_mov_b32 {x[0]}, {self.REG_L}")
            em.valu(f"v_lshl_add_u32 {self.v_la}, {h}, 4, {x[0]}", dst=[str(self.v_la)], src=[h])
        # DMA: instruction i of wave w fills 1 KB of a tile: rows
        # r = (w*DPW + i)*RPI + lane / CPR; LDS chunk p = lane % CPR holds the
        # row's chunk p ^ swz(r)
        lg = self.CPR.bit_length() - 1
        em.valu(f"v_lshrrev_b32 {t.r(2)}, {lg}, {lane}", dst=[t.r(2)], src=[lane])
        em.valu(f"v_and_b32 {t.r(3)}, {self.CPR - 1}, {lane}", dst=[t.r(3)], src=[lane])
        em.salu(f"s_mul_i32 {x[0]}, {self.s_w}, {self.DPW * self.RPI}")
        em.valu(f"v_add_u32 {t.r(2)}, {x[0]}, {t.r(2)}", dst=[t.r(2)], src=[t.r(2)])
        for i in range(self.DPW):
            r_, sw, a_ = t.r(4), t.r(5), t.r(6)
            em.valu(f"v_add_u32 {r_}, {self.RPI * i}, {t.r(2)}", dst=[r_], src=[t.r(2)])
            self.emit_swz(sw, r_, a_)
            em.valu(f"v_xor_b32 {sw}, {sw}, {t.r(3)}", dst=[sw], src=[sw, t.r(3)])
            em.valu(f"v_mul_lo_u32 {a_}, {r_}, {self.s_rowb}", dst=[a_], src=[r_])
            d = self.v_dma.r(i)
            em.valu(f"v_lshl_add_u32 {d}, {sw}, 4, {a_}", dst=[d], src=[sw, a_])
        em.valu(f"v_lshlrev_b32 {self.v_dml}, 2, {lane}", dst=[str(self.v_dml)], src=[lane])

    def zero_init(self):
        """Zero gradient accumulators; the rounded P / dS of the half before
        the first and the LDS stage it reads, so that the first step runs
        the same code as the others (its first Z block adds zeros)."""
        em, t, x = self.em, self.v_t, self.s_x
        for blk in self.a_acc1 + (self.a_acc2 if self.dkv else []):
            for i in range(16):
                em.valu(f"v_accvgpr_write_b32 {blk.r(i)}, 0", dst=[blk.r(i)])
        for b in self.v_pk[1] + self.v_sk[1]:
            for i in range(4):
                em.valu(f"v_mov_b32 {b.r(i)}, 0", dst=[b.r(i)])
        for i in range(4):
            em.valu(f"v_mov_b32 {t.r(i)}, 0", dst=[t.r(i)])
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 4, v0", dst=[t.r(4)], src=["v0"])
        em.salu(f"s_lshl_b32 {x[0]}, {self.s_w}, 10")
        em.valu(f"v_add_u32 {t.r(4)}, {x[0]}, {t.r(4)}", dst=[t.r(4)], src=[t.r(4)])
        for reg in ([0, self.REG_B] if self.dkv else [0]):
            em.valu(f"v_add_u32 {t.r(5)}, {reg + (NST - 1) * self.TILE}, {t.r(4)}", dst=[t.r(5)], src=[t.r(4)])
            for k in range(self.TILE // 4096):
                em._raw(f"ds_write_b128 {t.r(5)}, {t.r(0, 4)} offset:{4096 * k}")
        em.salu("s_waitcnt lgkmcnt(0)")

    # ------------------------------------------------------------------------
    def dma_init(self):
        """The stream's running state for step 0: descriptors at its first
        block (dK/dV: q-head hk*g, query block qb0; dQ: key tile 0), the
        per-step and next-q-head base steps, and the wave's LDS offsets."""
        em, x = self.em, self.s_x
        em.salu(f"s_lshl_b32 {self.s_full}, {self.s_rowb}, 6")
        em.salu(f"s_mov_b32 {self.s_ds}, 0")
        if self.dkv:
            em.salu(f"s_mov_b32 {self.s_dq}, {self.s_qb0}")
            em.salu(f"s_mul_i32 {x[0]}, {self.s_qb0}, {self.s_full}")       # rows 64*qb0 on
            em.salu(f"s_lshl_b32 {x[1]}, {self.s_qb0}, 8")
            # next q-head: + 2D, back by the blocks after qb0 (signed)
            em.salu(f"s_sub_u32 {x[2]}, {self.s_nqb}, {self.s_qb0}")
            em.salu(f"s_sub_u32 {x[2]}, {x[2]}, 1")
            em.salu(f"s_mul_i32 {x[3]}, {x[2]}, {self.s_full}")
            em.salu(f"s_sub_u32 {self.s_wd}, {2 * self.D}, {x[3]}")
            em.salu(f"s_ashr_i32 {self.s_wdh}, {self.s_wd}, 31")
            em.salu(f"s_lshl_b32 {x[3]}, {x[2]}, 8")
            em.salu(f"s_lshl_b32 {self.s_wdl}, s27, 2")
            em.salu(f"s_sub_u32 {self.s_wdl}, {self.s_wdl}, {x[3]}")
        else:
            em.salu(f"s_mov_b32 {x[0]}, 0")
            em.salu(f"s_mov_b32 {x[1]}, 0")
        for rs, base in ((self.s_ra, self.s_b0), (self.s_rb, self.s_b1)):
            em.salu(f"s_add_u32 {x[4]}, {base.r(0)}, {x[0]}")
            em.salu(f"s_addc_u32 {x[5]}, {base.r(1)}, 0")
            self.set_desc(rs, x[4], x[5], 0)
        if self.dkv:
            em.salu(f"s_add_u32 {x[4]}, {self.s_bl.r(0)}, {x[1]}")
            em.salu(f"s_addc_u32 {x[5]}, {self.s_bl.r(1)}, 0")
            self.set_desc(self.s_rl, x[4], x[5], 0)
            em.salu(f"s_mul_i32 {self.s_wl}, {self.s_w}, {NST * 256}")
            em.salu(f"s_add_u32 {self.s_wl}, {self.s_wl}, {self.REG_L}")
        em.salu(f"s_mul_i32 {self.s_wb}, {self.s_w}, {self.DPW * 1024}")

    def emit_dma(self):
        """The wave's loads of stream step s_ds into LDS stage s_ds % NST,
        then the stream advances.  Past the last step the ranges are 0
        bytes: the loads write zeros into a stage no one reads, and every
        step issues the same number of loads.  The last block of a q-head
        (of the keys) has a range of its rows only."""
        em, x = self.em, self.s_x
        TB = self.TILE.bit_length() - 1
        em.salu(f"s_lshl_b32 {x[0]}, {self.s_dq if self.dkv else self.s_ds}, 6")   # first row (key)
        em.salu(f"s_sub_u32 {x[1]}, {'s27' if self.dkv else 's28'}, {x[0]}")
        em.salu(f"s_min_u32 {x[1]}, {x[1]}, 64")
        em.salu(f"s_cmp_lt_u32 {self.s_ds}, {self.s_n}")
        em.salu(f"s_cselect_b32 {x[1]}, {x[1]}, 0")                   # rows
        em.salu(f"s_mul_i32 {self.s_ra.r(2)}, {x[1]}, {self.s_rowb}")
        em.salu(f"s_mov_b32 {self.s_rb.r(2)}, {self.s_ra.r(2)}")
        em.salu(f"s_and_b32 {x[6]}, {self.s_ds}, {NST - 1}")
        em.salu(f"s_lshl_b32 {x[7]}, {x[6]}, {TB}")
        em.salu(f"s_add_u32 {x[7]}, {x[7]}, {self.s_wb}")
        for region, rs in ((0, self.s_ra), (self.REG_B, self.s_rb)):
            for i in range(self.DPW):
                em.salu(f"s_add_u32 m0, {x[7]}, {region + 1024 * i}")
                em.salu("s_nop 0")
                em.vmem(f"buffer_load_dwordx4 {self.v_dma.r(i)}, {rs}, 0 offen lds", src=[self.v_dma.r(i)])
        if self.dkv:
            # 64 rows of l2 (wave 0) or delta (wave 1)
            l_skip = self.lab("nol")
            em.salu(f"s_cmp_ge_u32 {self.s_w}, 2")
            em.salu(f"s_cbranch_scc1 {l_skip}")
            em.salu(f"s_lshl_b32 {self.s_rl.r(2)}, {x[1]}, 2")
            em.salu(f"s_lshl_b32 {x[6]}, {x[6]}, 8")
            em.salu(f"s_add_u32 m0, {x[6]}, {self.s_wl}")
            em.salu("s_nop 0")
            em.vmem(f"buffer_load_dword {self.v_dml}, {self.s_rl}, 0 offen lds", src=[str(self.v_dml)])
            em.label(l_skip)
        em.salu(f"s_add_u32 {self.s_ds}, {self.s_ds}, 1")
        if self.dkv:
            # the next block, or the next q-head's first block
            em.salu(f"s_add_u32 {self.s_dq}, {self.s_dq}, 1")
            em.salu(f"s_cmp_eq_u32 {self.s_dq}, {self.s_nqb}")
            em.salu(f"s_cselect_b32 {self.s_dq}, {self.s_qb0}, {self.s_dq}")
            em.salu(f"s_cselect_b32 {x[2]}, {self.s_wd}, {self.s_full}")
            em.salu(f"s_cselect_b32 {x[3]}, {self.s_wdh}, 0")
            em.salu(f"s_cselect_b32 {x[4]}, {self.s_wdl}, 256")
            for rs in (self.s_ra, self.s_rb):
                em.salu(f"s_add_u32 {rs.r(0)}, {rs.r(0)}, {x[2]}")
                em.salu(f"s_addc_u32 {rs.r(1)}, {rs.r(1)}, {x[3]}")
            em.salu(f"s_add_u32 {self.s_rl.r(0)}, {self.s_rl.r(0)}, {x[4]}")
            em.salu(f"s_addc_u32 {self.s_rl.r(1)}, {self.s_rl.r(1)}, 0")
        else:
            for rs in (self.s_ra, self.s_rb):
                em.salu(f"s_add_u32 {rs.r(0)}, {rs.r(0)}, {self.s_full}")
                em.salu(f"s_addc_u32 {rs.r(1)}, {rs.r(1)}, 0")

    # ------------------------------------------------------------------------
    def x_items(self, hb):
        """X of half hb (tile rows 32hb..): S and dP, k-steps interleaved.  For
        dK/dV the half's l2 and delta reads ride along (after the operand
        reads of the odd items)."""
        em = self.em
        items = []
        for tt in range(self.NQ):
            for which in (0, 1):
                addr = (self.v_xa if which == 0 else self.v_xb).r(tt)
                frag = (self.a_f1 if which == 0 else self.a_f2)[tt]
                dst = str((self.v_S if which == 0 else self.v_P)[hb])

                def reads(buf, addr=addr):
                    R = self.a_R[buf]
                    em.ds_read(f"ds_read_b128 {R}, {addr} offset:{32 * hb * self.ROW}", str(R), addr)

                def mfma(buf, dst=dst, frag=frag, first=(tt == 0)):
                    em.mfma(self.mfma_op, dst, str(self.a_R[buf]), str(frag), "0" if first else dst)
                items.append(Item(reads, mfma))
        if self.dkv:
            extra = []
            for j in range(4):
                for which in (0, 1):
                    reg = (self.v_L if which == 0 else self.v_Dl)[hb].r(4 * j, 4)
                    off = (NST * 256 if which else 0) + 128 * hb + 32 * j
                    extra.append((reg, off))
            for k, (reg, off) in enumerate(extra):
                it = items[(2 * k + 1) * len(items) // 16]
                base = it.reads

                def reads(buf, base=base, reg=reg, off=off):
                    base(buf)
                    em.ds_read(f"ds_read_b128 {reg}, {self.v_la} offset:{off}", reg, str(self.v_la))
                it.reads = reads
        return items

    def z_items(self, hb):
        """Z of half hb: the gradient products with the half's rows of the
        tile read transposed (A) and the rounded P / dS (B)."""
        em = self.em
        items = []
        for ts in range(2):
            for db in range(self.ND):
                if self.dkv:
                    pairs = [(self.v_zb, self.a_acc2[db], self.v_pk[hb][ts]),    # dV += dO^T.P
                             (self.v_za, self.a_acc1[db], self.v_sk[hb][ts])]    # dK += Q^T.dS
                else:
                    pairs = [(self.v_za, self.a_acc1[db], self.v_sk[hb][ts])]    # dQ += K^T.dS
                for zr, acc, bop in pairs:
                    off = (32 * hb + 16 * ts) * self.ROW

                    def reads(buf, zr=zr, db=db, off=off):
                        R = self.a_R[buf]
                        for e in range(2):
                            em.ds_read(f"ds_read_b64_tr_b16 {R.r(2 * e, 2)}, {zr.r(2 * db + e)} offset:{off}",
                                       R.r(2 * e, 2), zr.r(2 * db + e))

                    def mfma(buf, acc=acc, bop=bop):
                        em.mfma(self.mfma_op, str(acc), str(self.a_R[buf]), str(bop), str(acc))
                    items.append(Item(reads, mfma))
        return items

    def y_ops(self, hb, part, masked, s_sub):
        """Y of half hb, registers 8*part .. 8*part+7: P = 2^(c*S - l2) (masked
        to 0 where a key is hidden), dS = P * (dP - delta), both rounded into
        the B operands of Z (k-step `part`)."""
        em = self.em
        S, P = self.v_S[hb], self.v_P[hb]
        tq, col, ninf = str(self.v_tq), str(self.v_col), str(self.v_ninf)
        ops = []
        if masked and part == 0:
            ops.append(Op(lambda: em.valu(f"v_subrev_u32 {tq}, {s_sub}, {col}", dst=[tq], src=[col])))
        idx = range(8 * part, 8 * part + 8)
        for i in idx:
            s_ = S.r(i)
            l2 = self.v_L[hb].r(i) if self.dkv else str(self.v_l2)
            ops.append(Op(lambda s_=s_, l2=l2: em.valu(f"v_fma_f32 {s_}, {s_}, s32, -{l2}", dst=[s_], src=[s_, l2])))
            if masked:
                # dK/dV: row 8j + e of the half sees the key when 8j + e >= tq;
                # dQ: key 8j + e of the block is seen when 8j + e <= tq
                cmp = "v_cmp_ge_i32" if self.dkv else "v_cmp_le_i32"
                k = 8 * (i // 4) + i % 4

                def msk(s_=s_, k=k):
                    em.valu(f"{cmp} vcc, {k}, {tq}", src=[tq])
                    em.valu(f"v_cndmask_b32 {s_}, {ninf}, {s_}, vcc", dst=[s_], src=[ninf, s_])
                ops.append(Op(msk, 2))
        for i in idx:
            s_ = S.r(i)
            ops.append(Op(lambda s_=s_: em.valu(f"v_exp_f32 {s_}, {s_}", dst=[s_], src=[s_], trans=True), 4))
        for i in idx:
            p_ = P.r(i)
            d_ = self.v_Dl[hb].r(i) if self.dkv else str(self.v_dl)
            ops.append(Op(lambda p_=p_, d_=d_: em.valu(f"v_sub_f32 {p_}, {p_}, {d_}", dst=[p_], src=[p_, d_])))
        for i in idx:
            s_, p_ = S.r(i), P.r(i)
            ops.append(Op(lambda s_=s_, p_=p_: em.valu(f"v_mul_f32 {p_}, {s_}, {p_}", dst=[p_], src=[s_, p_])))
        for m in range(4):
            a_, b_ = 8 * part + 2 * m, 8 * part + 2 * m + 1
            outs = [(self.v_sk[hb][part].r(m), P)]
            if self.dkv:
                outs.insert(0, (self.v_pk[hb][part].r(m), S))
            for dst, src in outs:
                ops.append(Op(lambda dst=dst, src=src, a_=a_, b_=b_: em.valu(
                    f"{self.cvt_op} {dst}, {src.r(a_)}, {src.r(b_)}", dst=[dst], src=[src.r(a_), src.r(b_)])))
        return ops

    # ------------------------------------------------------------------------
    def run_blocks(self, blocks, nxt, pre):
        """Emit MFMA blocks (items, vector ops, fence): each item's operand
        reads go LOOK MFMAs ahead (not ahead of a later block's fence), the
        vector ops are spread over the block's MFMAs by cost.  The reads of
        the first `pre` items were issued before; those of the first items of
        `nxt` are issued at the end."""
        em = self.em
        seq, bidx = [], []
        for bi, (items, _ops, _f) in enumerate(blocks):
            seq += items
            bidx += [bi] * len(items)
        seq += nxt
        bidx += [len(blocks)] * len(nxt)
        fenced = [f is not None for (_i, _o, f) in blocks] + [False]
        st = {"n": pre}

        def issue(limit, cur):
            while st["n"] < min(limit, len(seq)):
                k = st["n"]
                if any(fenced[b] for b in range(cur + 1, bidx[k] + 1)):
                    return
                seq[k].reads(k % self.RING)
                issued.add(k)
                st["n"] += 1

        issued = set(range(pre))
        k = 0
        for bi, (items, ops, fence) in enumerate(blocks):
            if fence is not None:
                assert st["n"] == k, "reads issued across a fence"
                fence()
            issue(k + self.LOOK, bi)
            total = sum(o.cost for o in ops)
            done, oi = 0.0, 0
            M = len(items)
            for m in range(M):
                assert k in issued, "an MFMA's operand reads were never issued"
                seq[k].mfma(k % self.RING)
                k += 1
                issue(k + self.LOOK, bi)
                target = total * (m + 1) / M
                while oi < len(ops) and done + ops[oi].cost * 0.5 <= target:
                    ops[oi]()
                    done += ops[oi].cost
                    oi += 1
            while oi < len(ops):
                ops[oi]()
                oi += 1
        assert st["n"] == min(len(seq), k + self.LOOK)
        return seq

    def loop_edge(self):
        """State at the step loop's head: every MFMA / VALU result settled,
        the operand reads of the next step's first MFMAs (and, dK/dV, the l2 /
        delta reads of its first half) in flight."""
        em = self.em
        em._nop(12)
        em.mfma_w.clear()
        em.valu_w.clear()
        em.trans_w.clear()

    def step_body(self, m0, m1):
        """One step (a 64-row tile, halves 2t and 2t+1): Z(2t-1) | X(2t+1) |
        Z(2t) | barrier, next DMA | X(2t+2), with Y(2t) in the first two
        blocks and Y(2t+1) in the last two."""
        em, x = self.em, self.s_x
        TB = self.TILE.bit_length() - 1
        # the transposing reads move from stage t-1 to stage t before Z(2t)
        em.salu(f"s_sub_u32 {x[6]}, {self.s_t}, 1")
        em.salu(f"s_xor_b32 {x[7]}, {x[6]}, {self.s_t}")
        em.salu(f"s_and_b32 {x[7]}, {x[7]}, {NST - 1}")
        em.salu(f"s_lshl_b32 {x[7]}, {x[7]}, {TB}")
        zregs = [self.v_za.r(i) for i in range(2 * self.ND)]
        if self.dkv:
            zregs += [self.v_zb.r(i) for i in range(2 * self.ND)]
        upd = [Op(lambda z=z: em.valu(f"v_xor_b32 {z}, {x[7]}, {z}", dst=[z], src=[z])) for z in zregs]

        def barrier():
            em.salu(f"s_waitcnt vmcnt({2 * self.DPW})")       # the next tile in LDS
            em.salu("s_barrier")
            self.emit_dma()
            # the row reads move to stage t+1
            em.salu(f"s_add_u32 {x[6]}, {self.s_t}, 1")
            em.salu(f"s_xor_b32 {x[7]}, {x[6]}, {self.s_t}")
            em.salu(f"s_and_b32 {x[7]}, {x[7]}, {NST - 1}")
            em.salu(f"s_lshl_b32 {x[6]}, {x[7]}, {TB}")
            em.salu(f"s_lshl_b32 {x[7]}, {x[7]}, 8")
            for tt in range(self.NQ):
                for r in (self.v_xa.r(tt), self.v_xb.r(tt)):
                    em.valu(f"v_xor_b32 {r}, {x[6]}, {r}", dst=[r], src=[r])
            if self.dkv:
                la = str(self.v_la)
                em.valu(f"v_xor_b32 {la}, {x[7]}, {la}", dst=[la], src=[la])

        blocks = [
            (self.z_items(1), self.y_ops(0, 0, m0, self.s_q0), None),
            (self.x_items(1), upd + self.y_ops(0, 1, m0, self.s_q0), None),
            (self.z_items(0), self.y_ops(1, 0, m1, self.s_q1), None),
            (self.x_items(0), self.y_ops(1, 1, m1, self.s_q1), barrier),
        ]
        self.run_blocks(blocks, self.z_items(1)[:self.PRE], self.PRE)

    def epilogue(self):
        """The gradients, scaled (dK, dQ) and rounded, to their rows: lane
        column, dims 32db + 8j + 4h .. +3 (8 bytes)."""
        em = self.em
        outs = [(self.a_acc1, self.s_ro1, True)]
        if self.dkv:
            outs.append((self.a_acc2, self.s_ro2, False))
        # temporaries: the S / dP registers, four at a time
        tmps = [(blk, 4 * q) for blk in self.v_S + self.v_P for q in range(4)]
        n = 0
        for db in range(self.ND):
            for j in range(4):
                for acc, rs, scaled in outs:
                    blk, o = tmps[n % len(tmps)]
                    R = Block4(blk, o)
                    n += 1
                    for e in range(4):
                        em.valu(f"v_accvgpr_read_b32 {R.r(e)}, {acc[db].r(4 * j + e)}", dst=[R.r(e)],
                                src=[acc[db].r(4 * j + e)])
                        if scaled:
                            em.valu(f"v_mul_f32 {R.r(e)}, s33, {R.r(e)}", dst=[R.r(e)], src=[R.r(e)])
                    for c in range(2):
                        em.valu(f"{self.cvt_op} {R.r(c)}, {R.r(2 * c)}, {R.r(2 * c + 1)}", dst=[R.r(c)],
                                src=[R.r(2 * c), R.r(2 * c + 1)])
                    em.vmem(f"buffer_store_dwordx2 {R.r(0, 2)}, {self.v_so}, {rs}, 0 offen "
                            f"offset:{64 * db + 16 * j}", src=[R.r(0, 2), str(self.v_so)])

    def body(self):
        self.alloc()
        em, x = self.em, self.s_x
        self.setup()
        self.lane_consts()
        self.zero_init()
        em.drain()
        l_store, l_head, l_exit = self.lab("store"), self.lab("head"), self.lab("exit")
        em.salu(f"s_cmp_eq_u32 {self.s_n}, 0")
        em.salu(f"s_cbranch_scc1 {l_store}")
        em.salu(f"s_mov_b32 {self.s_t}, 0")
        if self.dkv:
            em.salu(f"s_mov_b32 {self.s_cq}, {self.s_qb0}")
        self.dma_init()
        self.emit_dma()
        self.emit_dma()
        em.salu(f"s_waitcnt vmcnt({2 * self.DPW})")          # resident operands, tile 0
        em.salu("s_barrier")
        self.emit_dma()
        self.run_blocks([(self.x_items(0), [], None)], self.z_items(1)[:self.PRE], 0)
        self.loop_edge()
        snap = em.snapshot()
        pend = [set(p) for p in em.lds_pending]
        em.label(l_head)
        names = {k: self.lab(k) for k in ("ff", "mf", "mm")}
        if self.dkv:
            # half 0 (rows i0 .. i0+31) sees every key of the wave when
            # kw0 + 31 <= i0 + off; then half 1 does too
            em.salu("s_cmp_eq_u32 s31, 0")
            em.salu(f"s_cbranch_scc1 {names['ff']}")
            em.salu(f"s_lshl_b32 {x[0]}, {self.s_cq}, 6")
            em.salu(f"s_add_i32 {x[0]}, {x[0]}, {self.s_off}")
            em.salu(f"s_add_u32 {x[1]}, {self.s_lim}, 31")
            em.salu(f"s_cmp_le_i32 {x[1]}, {x[0]}")
            em.salu(f"s_cbranch_scc1 {names['ff']}")
            em.salu(f"s_add_i32 {x[0]}, {x[0]}, 32")
            em.salu(f"s_cmp_le_i32 {x[1]}, {x[0]}")
            em.salu(f"s_cbranch_scc1 {names['mf']}")
        else:
            # block 2t (keys 64t .. 64t+31) is seen in full when 64t + 31 <= lim
            em.salu(f"s_lshl_b32 {x[0]}, {self.s_t}, 6")
            em.salu(f"s_add_u32 {x[1]}, {x[0]}, 63")
            em.salu(f"s_cmp_le_i32 {x[1]}, {self.s_lim}")
            em.salu(f"s_cbranch_scc1 {names['ff']}")
            em.salu(f"s_add_u32 {x[1]}, {x[0]}, 31")
            em.salu(f"s_cmp_le_i32 {x[1]}, {self.s_lim}")
            em.salu(f"s_cbranch_scc1 {names['mf']}")
        em.salu(f"s_branch {names['mm']}")
        # dK/dV: (half 0, half 1) masked = (no, no), (yes, no), (yes, yes);
        # dQ: (no, no), (no, yes), (yes, yes)
        variants = {"ff": (False, False), "mf": (True, False) if self.dkv else (False, True),
                    "mm": (True, True)}
        for key, (m0, m1) in variants.items():
            em.restore(snap)
            em.label(names[key])
            if self.dkv:
                em.salu(f"s_lshl_b32 {self.s_q0}, {self.s_cq}, 6")
            else:
                em.salu(f"s_lshl_b32 {self.s_q0}, {self.s_t}, 6")
            em.salu(f"s_add_u32 {self.s_q1}, {self.s_q0}, 32")
            self.step_body(m0, m1)
            if self.dkv:
                em.salu(f"s_add_u32 {self.s_cq}, {self.s_cq}, 1")
                em.salu(f"s_cmp_eq_u32 {self.s_cq}, {self.s_nqb}")
                em.salu(f"s_cselect_b32 {self.s_cq}, {self.s_qb0}, {self.s_cq}")
            em.salu(f"s_add_u32 {self.s_t}, {self.s_t}, 1")
            self.loop_edge()
            assert [set(p) for p in em.lds_pending] == pend, "loop-head reads differ"
            em.salu(f"s_cmp_lt_u32 {self.s_t}, {self.s_n}")
            em.salu(f"s_cbranch_scc1 {l_head}")
            em.salu(f"s_branch {l_exit}")
        em.restore(snap)
        em.label(l_exit)
        self.run_blocks([(self.z_items(1), [], None)], [], self.PRE)
        em.drain()
        em.label(l_store)
        # every load (LDS DMA included) is done before the wave's last
        # instructions; the stores need not be waited for
        em.salu("s_waitcnt vmcnt(0)")
        self.epilogue()
        em.salu("s_endpgm")

    def assemble_text(self):
        self.body()
        name = self.name
        nv, na = self.nvgpr, self.nagpr
        total = nv + na
        out = ['\t.text', f"\t.globl {name}", "\t.p2align 8", f"\t.type {name},@function", f"{name}:",
               self.em.text(), f"\t.size {name}, .-{name}", "\t.rodata", "\t.p2align 6",
               f"\t.amdhsa_kernel {name}"]
        for k, v in [
            ("group_segment_fixed_size", self.LDS), ("private_segment_fixed_size", 0),
            ("kernarg_size", KERNARG_BYTES), ("user_sgpr_count", 2),
            ("user_sgpr_dispatch_ptr", 0), ("user_sgpr_queue_ptr", 0),
            ("user_sgpr_kernarg_segment_ptr", 1), ("user_sgpr_dispatch_id", 0),
            ("user_sgpr_kernarg_preload_length", 0), ("user_sgpr_kernarg_preload_offset", 0),
            ("user_sgpr_private_segment_size", 0), ("uses_dynamic_stack", 0),
            ("enable_private_segment", 0), ("system_sgpr_workgroup_id_x", 1),
            ("system_sgpr_workgroup_id_y", 1), ("system_sgpr_workgroup_id_z", 1),
            ("system_sgpr_workgroup_info", 0), ("system_vgpr_workitem_id", 0),
            ("next_free_vgpr", total), ("next_free_sgpr", self.nsgpr), ("accum_offset", nv),
            ("reserve_vcc", 1), ("float_round_mode_32", 0), ("float_round_mode_16_64", 0),
            ("float_denorm_mode_32", 3), ("float_denorm_mode_16_64", 3), ("dx10_clamp", 1),
            ("ieee_mode", 1), ("fp16_overflow", 0), ("tg_split", 0),
        ]:
            out.append(f"\t\t.amdhsa_{k} {v}")
        out.append("\t.end_amdhsa_kernel")
        ptrs = [(8 * i, "read_only") for i in range(6)] + [(48 + 8 * i, "write_only") for i in range(3)]
        return "\n".join(out) + "\n", dict(name=name, nv=nv, na=na, total=total, lds=self.LDS,
                                          ns=self.nsgpr + 2, wg=256, ptrs=ptrs,
                                          kernarg=KERNARG_BYTES)


VARIANTS = [(kind, dt, D) for kind in ("dkv", "dq") for dt in ("bf16", "f16") for D in (128, 64)]
