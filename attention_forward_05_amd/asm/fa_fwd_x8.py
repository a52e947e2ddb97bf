"""Generator of the eight-wave gfx950 (MI355X) attention forward kernel, D = 128.

Same operation as the four-wave kernel (fa_fwd_gen.py): the tiled
online-softmax forward pass of the JAX Pallas FlashAttention3 page
(`kv_loop`: running max m, running sum l, rescaled accumulator) in the exp2
form of the Croqtile `flash_atten` page, with a lazy reference max:

    P = 2^(c*S - mc),  l += rowsum(P),  O += P.V          (mc = c*m)

and, only when some p of a sub-tile would exceed the trigger, a slow path
that moves m to the row max, rescales O and l by 2^(mc_old - mc_new) and
redoes the sub-tile.  At the end O / l and LSE = ln2*(mc + log2 l).

Organisation (per workgroup: 512 query rows of one (batch, q-head) against
the visible keys of its kv-head, in tiles of 64 keys):

* Eight waves, two per SIMD (waves w and w+4 share one).  Wave w owns the
  32-row query blocks w and 15-w of the 512-row tile (a causal diagonal then
  costs every wave about the same), 64 rows in all: O^T (128 VGPRs) and Q
  (64 AGPRs) stay in registers, 64 more VGPRs hold S/P (32), a ring of three
  MFMA operand buffers (12) and the rest: 256 registers, two waves per SIMD.
* Each wave alternates an MFMA phase (P.V of sub-tile j-1 then S^T = K.Q^T
  of sub-tile j: 32 MFMAs, operands streamed from LDS through the ring) and
  a softmax phase (exponentials, row sums, conversion of P, in place).
  Waves 4-7 run one phase behind waves 0-3, with one s_barrier per phase,
  so on every SIMD one wave's MFMAs overlap the other wave's softmax.
* K and V tiles go HBM -> LDS by buffer_load ... lds, three tiles ahead,
  through four K slots and four V slots (128 KB); each wave moves 8 rows of
  each tile.  Tile u is needed from global phase 4u and freed after phase
  4u+5; its loads are issued in phase 4u-9 (4u-8 for waves 4-7).
* S and P share registers: P (the input dtype) is converted over the first
  half of S, and the next S^T overwrites it only after the P.V MFMAs that
  read it have issued.  The slow path therefore recomputes S^T from the K
  tile, which is still resident.
* Persistent schedule as in the four-wave kernel: workgroup g takes items
  r*G + (g or G-1-g) of the longest-first (batch, q-head, q-tile) list.
"""
from __future__ import annotations

import math

from .regs import Alloc, Emitter
from .fa_fwd_gen import LN2, f32_hex

BM = 512          # query rows per workgroup
BN = 64           # keys per tile
WAVES = 8
SLOTS = 4         # K (and V) tiles held in LDS
AHEAD = 3         # tiles whose loads are in flight ahead of the tile in use
THRESH = 32768.0  # slow-path trigger: a lane's 16-key partial row sum above 2^15


def kernel_name(dtype: str, split: bool = False, D: int = 128) -> str:
    return f"fa_fwd_{dtype}_d{D}_x8{'s' if split else ''}_gfx950"


class Gen8:

    def __init__(self, dtype: str, split: bool = False, D: int = 128):
        assert dtype in ("bf16", "f16") and D in (64, 128)
        self.dtype = dtype
        self.D = D
        # split: every (batch, q-head, query tile) item is cut into 2^log2split
        # key ranges (kernel argument); each writes its normalised O (fp32)
        # and LSE to the partial buffers passed as o / lse, which a combine
        # kernel merges
        self.split = split
        self.name = kernel_name(dtype, split, D)
        self.mfma_op = "v_mfma_f32_32x32x16_bf16" if dtype == "bf16" else "v_mfma_f32_32x32x16_f16"
        self.cvt_op = "v_cvt_pk_bf16_f32" if dtype == "bf16" else "v_cvt_pk_f16_f32"
        D = self.D
        self.NS = D // 16             # k-steps of S^T
        self.NDB = D // 32            # 32-dim blocks of O^T
        self.ROW = D * 2              # bytes per K/V row in LDS
        self.TILE = BN * self.ROW     # bytes per K or V tile (16 KB)
        self.CH = D // 8              # 16-byte chunks per row
        self.RPD = 64 // self.CH      # rows per 64-lane DMA instruction
        self.DPW = (BN // WAVES) // self.RPD  # DMA instructions per wave per K (or V) tile
        self.LPT = 2 * self.DPW       # loads per wave per stream tile (K and V)
        self.KREG = 0
        self.VREG = SLOTS * self.TILE
        self.DUMP = 2 * SLOTS * self.TILE    # spare K and V tile for all-zero tiles
        self.LDS = self.DUMP + 2 * self.TILE
        assert self.DPW >= 1 and self.LDS <= 160 * 1024
        self.em = Emitter()
        self._lab = 0
        self.deferred = []

    def lab(self, tag):
        self._lab += 1
        d = "" if self.D == 128 else f"d{self.D}"
        return f".L{self.dtype}{d}x8{'s' if self.split else ''}_{tag}_{self._lab}"

    # ------------------------------------------------------------------------
    def alloc(self):
        V = Alloc("v", 0, 192)
        A = Alloc("a", 0, 64)
        S = Alloc("s", 28, 102)
        r = self.__dict__
        r["v_lane"] = V.take("lane", 1)        # v0: lane id (after kernel_setup)
        r["v_klane"] = V.take("klane", 1)      # K operand address of k-step 0, slot 0
        r["v_vlane"] = V.take("vlane", 1)      # V operand address of d-block 0, slot 0
        r["v_kb"] = V.take("kb", 1)            # K operand base of the tile in S^T
        r["v_S"] = [V.take(f"S{q}", 16, 4) for q in range(2)]
        r["v_R"] = [V.take(f"R{i}", 4, 4) for i in range(3)]
        r["v_vb"] = V.take("vb", 1)            # V operand base of the tile in P.V
        r["v_kdma"] = V.take("kdma", self.DPW)
        r["v_vdma"] = V.take("vdma", self.DPW)
        r["v_mc"] = V.take("mc", 2)            # c * m per query block (0 while m = -inf)
        r["v_l"] = V.take("l", 2)              # per-lane partial row sums
        r["v_rs"] = V.take("rs", 2)            # partial row sums of the current sub-tile
        r["v_t"] = V.take("tmp", 5)
        assert V.next <= 64, V.next
        V.next = 64
        # O^T accumulators in VGPRs (the epilogue and the slow path scale them
        # in place), Q in AGPRs (only ever an MFMA operand)
        r["v_O"] = [[V.take(f"O{q}{d}", 16, 4) for d in range(self.NDB)] for q in range(2)]
        self.nvgpr = V.next
        assert V.next == 64 + 32 * self.NDB
        r["a_Q"] = [[A.take(f"Q{q}{s}", 4, 4) for s in range(self.NS)] for q in range(2)]
        self.nagpr = A.next
        assert A.next == 8 * self.NS
        t = S.take
        # the current item
        r["s_hq"], r["s_qt"], r["s_b"], r["s_hk"] = t("hq", 1), t("qt", 1), t("b", 1), t("hk", 1)
        r["s_w"], r["s_off"], r["s_ntiles"] = t("w", 1), t("off", 1), t("nt", 1)
        r["s_rowlim"], r["s_rowb"], r["s_u"] = t("rowlim", 1), t("rowb", 1), t("u", 1)
        # per query block b: sub-tiles whose first key k0 <= fu_b are seen in
        # full by every row of the block; k0 > dl_b by none of them
        r["s_fu"] = [t("fu0", 1), t("fu1", 1)]
        r["s_dl"] = [t("dl0", 1), t("dl1", 1)]
        r["s_rb"] = [t("rb0", 1), t("rb1", 1)]
        r["s_ro"] = t("ro", 4, 4)
        r["s_rl"] = t("rl", 4, 4)
        r["s_rk"] = t("rk", 4, 4)
        r["s_rq"] = r["s_rk"]                  # Q loads are issued before a K descriptor is built
        r["s_rv"] = t("rv", 4, 4)
        r["s_g"], r["s_r"] = t("wg", 1), t("round", 1)
        r["s_kbase"] = t("kbase", 2, 2)
        r["s_vbase"] = t("vbase", 2, 2)
        r["s_k0"] = t("k0", 1)                 # first key of the current softmax sub-tile
        r["s_wrow"] = t("wrow", 1)
        r["s_ring"] = t("ring", 1)             # LDS slot of the item's tile 0
        # the next item: ids, K/V bases, row limit and tile count (0: none)
        r["s_nb"], r["s_nhq"], r["s_nqt"] = t("nb", 1), t("nhq", 1), t("nqt", 1)
        r["s_nkb"] = t("nkb", 2, 2)
        r["s_nvb"] = t("nvb", 2, 2)
        r["s_nrl"], r["s_nnt"] = t("nrl", 1), t("nnt", 1)
        r["s_x"] = [t(f"x{i}", 1) for i in range(6)]
        r["s_y"] = [t(f"y{i}", 1) for i in range(6)]
        r["s_m1"], r["s_m2"] = t("msk1", 2, 2), t("msk2", 2, 2)
        r["s_thr"] = t("thr", 1)
        if self.split:
            r["s_l2s"] = t("log2split", 1)     # log2 of the key ranges per item
            r["s_sp"], r["s_nsp"] = t("sp", 1), t("nsp", 1)   # key range of the item / the next
            r["s_kst"] = t("kstart", 1)        # first key of the item's range
        self.nsgpr = S.next

    # ------------------------------------------------------------------------
    # set-up
    # ------------------------------------------------------------------------
    def kernel_setup(self):
        em, D = self.em, self.D
        em.salu("s_load_dwordx16 s[8:23], s[0:1], 0x0")
        em.salu("s_load_dwordx4 s[24:27], s[0:1], 0x40")
        em.valu(f"v_readfirstlane_b32 {self.s_w}, v0", src=["v0"])
        em.salu(f"s_lshr_b32 {self.s_w}, {self.s_w}, 6")
        em.valu("v_and_b32 v0, 63, v0", dst=["v0"], src=["v0"])
        em.salu(f"s_mov_b32 {self.s_g}, s2")
        em.salu(f"s_mov_b32 {self.s_r}, 0")
        em.salu(f"s_mov_b32 {self.s_ring}, 0")
        if self.split:
            em.salu(f"s_load_dword {self.s_l2s}, s[0:1], 0x50")
        em.salu("s_waitcnt lgkmcnt(0)")
        em.salu(f"s_mov_b32 {self.s_thr}, {f32_hex(THRESH)}")
        em.salu(f"s_mul_i32 {self.s_rowb}, s22, {D * 2}")          # K/V row stride
        em.salu(f"s_mul_i32 {self.s_wrow}, {self.s_w}, {(BN // WAVES) * self.ROW}")

    # LDS swizzles (the LDS serves 256 bytes per pass: 16 lanes of a K row
    # read, 32 lanes of a transposing V read).  D = 128 (256-byte rows):
    # chunk c of K row r sits at c ^ (r & 15), of V row r at c ^ 4*(r & 3).
    # D = 64 (128-byte rows, two rows per pass of the banks): K at
    # c ^ ((r >> 1) & 7), V at c ^ 4*((r >> 1) & 1).  Row reads of 16
    # consecutive rows and transposing reads of 4 rows x 4 chunks then hit
    # 64 distinct banks.
    def emit_ksw(self, dst, row):
        if self.D == 128:
            self.em.valu(f"v_and_b32 {dst}, 15, {row}", dst=[dst], src=[row])
        else:
            self.em.valu(f"v_bfe_u32 {dst}, {row}, 1, 3", dst=[dst], src=[row])

    def emit_vsw(self, dst, row):
        if self.D == 128:
            self.em.valu(f"v_and_b32 {dst}, 3, {row}", dst=[dst], src=[row])
        else:
            self.em.valu(f"v_bfe_u32 {dst}, {row}, 1, 1", dst=[dst], src=[row])
        self.em.valu(f"v_lshlrev_b32 {dst}, 2, {dst}", dst=[dst], src=[dst])

    def tmps(self):
        """Scratch VGPRs for set-up code (the S registers are free then)."""
        return [self.v_S[i // 16].r(i % 16) for i in range(32)]

    def emit_div(self, num, den, q, rem, dv, z):
        """q = num / den, rem = num - q*den for num, den < 2^24 (VGPR num,
        SGPR den): float reciprocal estimate, then one correction each way."""
        em = self.em
        em.valu(f"v_mov_b32 {dv}, {den}", dst=[dv])
        em.valu(f"v_cvt_f32_u32 {q}, {num}", dst=[q], src=[num])
        em.valu(f"v_cvt_f32_u32 {rem}, {dv}", dst=[rem], src=[dv])
        em.valu(f"v_rcp_f32 {rem}, {rem}", dst=[rem], src=[rem], trans=True)
        em.valu(f"v_mul_f32 {q}, {q}, {rem}", dst=[q], src=[q, rem])
        em.valu(f"v_cvt_u32_f32 {q}, {q}", dst=[q], src=[q])
        em.valu(f"v_mul_lo_u32 {rem}, {q}, {dv}", dst=[rem], src=[q, dv])
        em.valu(f"v_sub_u32 {rem}, {num}, {rem}", dst=[rem], src=[num, rem])
        em.valu(f"v_cmp_gt_i32 vcc, 0, {rem}", src=[rem])
        em.valu(f"v_cndmask_b32 {z}, 0, -1, vcc", dst=[z])
        em.valu(f"v_add_u32 {q}, {q}, {z}", dst=[q], src=[q, z])
        em.valu(f"v_cndmask_b32 {z}, 0, {dv}, vcc", dst=[z], src=[dv])
        em.valu(f"v_add_u32 {rem}, {rem}, {z}", dst=[rem], src=[rem, z])
        em.valu(f"v_cmp_le_u32 vcc, {dv}, {rem}", src=[rem, dv])
        em.valu(f"v_cndmask_b32 {z}, 0, 1, vcc", dst=[z])
        em.valu(f"v_add_u32 {q}, {q}, {z}", dst=[q], src=[q, z])
        em.valu(f"v_cndmask_b32 {z}, 0, {dv}, vcc", dst=[z], src=[dv])
        em.valu(f"v_sub_u32 {rem}, {rem}, {z}", dst=[rem], src=[rem, z])

    def lane_consts(self):
        """Per-lane DMA source offsets and LDS operand addresses."""
        em, D = self.em, self.D
        t = self.tmps()
        lane = "v0"
        l32, h = t[0], t[1]
        em.valu(f"v_and_b32 {l32}, 31, {lane}", dst=[l32], src=[lane])
        em.valu(f"v_lshrrev_b32 {h}, 5, {lane}", dst=[h], src=[lane])
        # DMA: row r = 8w + RPD*i + lane/CH of the tile, LDS chunk p = lane % CH
        # holds row chunk p ^ swz(r) (K: r & 15, V: 4*(r & 3))
        CH = self.CH
        em.valu(f"v_lshrrev_b32 {t[2]}, {int(math.log2(CH))}, {lane}", dst=[t[2]], src=[lane])
        em.valu(f"v_and_b32 {t[3]}, {CH - 1}, {lane}", dst=[t[3]], src=[lane])
        em.salu(f"s_lshl_b32 {self.s_x[0]}, {self.s_w}, 3")
        em.valu(f"v_add_u32 {t[2]}, {self.s_x[0]}, {t[2]}", dst=[t[2]], src=[t[2]])
        for i in range(self.DPW):
            r_, off, sw = t[4], t[5], t[6]
            em.valu(f"v_add_u32 {r_}, {self.RPD * i}, {t[2]}", dst=[r_], src=[t[2]])
            em.valu(f"v_mul_lo_u32 {off}, {r_}, {self.s_rowb}", dst=[off], src=[r_])
            self.emit_ksw(sw, r_)
            em.valu(f"v_xor_b32 {sw}, {sw}, {t[3]}", dst=[sw], src=[sw, t[3]])
            em.valu(f"v_lshl_add_u32 {self.v_kdma.r(i)}, {sw}, 4, {off}", dst=[self.v_kdma.r(i)], src=[sw, off])
            self.emit_vsw(sw, r_)
            em.valu(f"v_xor_b32 {sw}, {sw}, {t[3]}", dst=[sw], src=[sw, t[3]])
            em.valu(f"v_lshl_add_u32 {self.v_vdma.r(i)}, {sw}, 4, {off}", dst=[self.v_vdma.r(i)], src=[sw, off])
        # K operand of k-step s: l32*ROW + 16*((2s + h) ^ ksw(l32)) = klane ^ (s << 5)
        self.emit_ksw(t[2], l32)
        em.valu(f"v_xor_b32 {t[2]}, {t[2]}, {h}", dst=[t[2]], src=[t[2], h])
        em.valu(f"v_mul_u32_u24 {t[3]}, {self.ROW}, {l32}", dst=[t[3]], src=[l32])
        em.valu(f"v_lshl_add_u32 {self.v_klane}, {t[2]}, 4, {t[3]}", dst=[str(self.v_klane)], src=[t[2], t[3]])
        # V operand of d-block db (transposing reads): tr_i = lane & 15,
        # tr_row = 4h + (tr_i >> 2), chunk (4db + 2*((lane >> 4) & 1) + ((lane >> 1) & 1))
        # ^ vsw(tr_row), byte 8*(lane & 1):  vlane ^ (db << 6)
        em.valu(f"v_bfe_u32 {t[2]}, {lane}, 2, 2", dst=[t[2]], src=[lane])
        em.valu(f"v_lshl_add_u32 {t[2]}, {h}, 2, {t[2]}", dst=[t[2]], src=[h, t[2]])       # tr_row
        self.emit_vsw(t[3], t[2])                                                          # sw
        em.valu(f"v_bfe_u32 {t[4]}, {lane}, 4, 1", dst=[t[4]], src=[lane])
        em.valu(f"v_bfe_u32 {t[5]}, {lane}, 1, 1", dst=[t[5]], src=[lane])
        em.valu(f"v_lshl_add_u32 {t[4]}, {t[4]}, 1, {t[5]}", dst=[t[4]], src=[t[4], t[5]])
        em.valu(f"v_xor_b32 {t[4]}, {t[4]}, {t[3]}", dst=[t[4]], src=[t[4], t[3]])
        em.valu(f"v_and_b32 {t[5]}, 1, {lane}", dst=[t[5]], src=[lane])
        em.valu(f"v_lshlrev_b32 {t[5]}, 3, {t[5]}", dst=[t[5]], src=[t[5]])
        em.salu(f"s_mov_b32 {self.s_x[0]}, {self.ROW}")
        em.valu(f"v_mad_u32_u24 {t[5]}, {t[2]}, {self.s_x[0]}, {t[5]}", dst=[t[5]], src=[t[2], t[5]])
        em.valu(f"v_lshl_add_u32 {t[5]}, {t[4]}, 4, {t[5]}", dst=[t[5]], src=[t[4], t[5]])
        em.valu(f"v_add_u32 {self.v_vlane}, {self.VREG}, {t[5]}", dst=[str(self.v_vlane)], src=[t[5]])

    # Items (batch, q-head, 512-row query tile) in decreasing key count;
    # workgroup g of G takes item r*G + (g or G-1-g, by the parity of round r).
    def decode(self, rsg, out, l_none):
        """(b, hq, qt) of the item of round `rsg` (sgpr) into the sgprs `out`;
        branches to l_none when there is no such item.  Uses the v_t temps."""
        em, x, t = self.em, self.s_x, self.v_t
        ob, ohq, oqt = out[:3]
        em.salu(f"s_lshr_b32 {x[1]}, s25, 16")                     # G
        em.salu(f"s_mul_i32 {x[2]}, {rsg}, {x[1]}")
        em.salu(f"s_sub_u32 {x[3]}, {x[1]}, 1")
        em.salu(f"s_sub_u32 {x[3]}, {x[3]}, {self.s_g}")
        em.salu(f"s_bitcmp1_b32 {rsg}, 0")
        em.salu(f"s_cselect_b32 {x[3]}, {x[3]}, {self.s_g}")
        em.salu(f"s_add_u32 {x[2]}, {x[2]}, {x[3]}")                # idx
        em.salu(f"s_mul_i32 {x[4]}, s18, s21")                      # (batch, head) pairs
        if self.split:
            em.salu(f"s_lshl_b32 {x[4]}, {x[4]}, {self.s_l2s}")     # ... times key ranges
        em.salu(f"s_and_b32 {x[5]}, s25, 0xffff")                   # query tiles
        em.salu(f"s_mul_i32 {x[1]}, {x[4]}, {x[5]}")
        em.salu(f"s_cmp_ge_u32 {x[2]}, {x[1]}")
        em.salu(f"s_cbranch_scc1 {l_none}")
        em.valu(f"v_mov_b32 {t.r(0)}, {x[2]}", dst=[t.r(0)])
        self.emit_div(t.r(0), x[4], t.r(1), t.r(2), t.r(3), t.r(4))        # level, within
        em.valu(f"v_readfirstlane_b32 {x[3]}, {t.r(1)}", src=[t.r(1)])
        if self.split:
            # within = key range * pairs + (batch, head) pair
            em.salu(f"s_mul_i32 {x[0]}, s18, s21")
            self.emit_div(t.r(2), x[0], t.r(3), t.r(4), t.r(0), t.r(1))    # key range, pair
            em.valu(f"v_readfirstlane_b32 {out[3]}, {t.r(3)}", src=[t.r(3)])
            em.valu(f"v_mov_b32 {t.r(2)}, {t.r(4)}", dst=[t.r(2)], src=[t.r(4)])
        self.emit_div(t.r(2), "s21", t.r(3), t.r(4), t.r(0), t.r(1))       # b, head slot
        em.valu(f"v_readfirstlane_b32 {ob}, {t.r(3)}", src=[t.r(3)])
        em.valu(f"v_readfirstlane_b32 {x[4]}, {t.r(4)}", src=[t.r(4)])
        # hq: contiguous head groups over the 8 XCDs.  Workgroup g runs on XCD
        # g % 8; in odd rounds it takes slot G-1-g's item, whose slot % 8 is
        # 7 - g % 8 (G and the pair count multiples of 8), so the group index
        # is flipped there and every round of a workgroup stays on one group
        # of heads (whose K/V its XCD's L2 holds)
        em.salu("s_cmp_eq_u32 s27, 0")
        em.salu(f"s_cselect_b32 {x[2]}, 0, 7")
        em.salu(f"s_and_b32 {ohq}, {x[4]}, {x[2]}")
        em.salu(f"s_bitcmp1_b32 {rsg}, 0")
        em.salu(f"s_cselect_b32 {x[1]}, {x[2]}, 0")
        em.salu(f"s_xor_b32 {ohq}, {ohq}, {x[1]}")
        em.salu(f"s_mul_i32 {ohq}, {ohq}, s27")
        em.salu("s_cmp_eq_u32 s27, 0")
        em.salu(f"s_cselect_b32 {x[2]}, 0, 3")
        em.salu(f"s_lshr_b32 {x[2]}, {x[4]}, {x[2]}")
        em.salu(f"s_add_u32 {ohq}, {ohq}, {x[2]}")
        # query tile: longest causal tiles first
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, 1")
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, {x[3]}")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {oqt}, {x[3]}, {x[5]}")

    def kv_range(self, qt, nt, rowlim, sp=None, kst=None):
        """Key tiles of query tile qt: kv_end = causal ? min(Skv, min(512 qt + 512,
        Sq) + Skv - Sq) : Skv; nt = ceil(kv_end / 64), rowlim = min(64 nt, Skv)."""
        em, x = self.em, self.s_x
        em.salu(f"s_lshl_b32 {x[0]}, {qt}, 9")
        em.salu(f"s_add_u32 {x[0]}, {x[0]}, {BM}")
        em.salu(f"s_min_i32 {x[0]}, {x[0]}, s19")
        em.salu(f"s_sub_i32 {x[1]}, s20, s19")
        em.salu(f"s_add_i32 {x[0]}, {x[0]}, {x[1]}")
        em.salu(f"s_min_i32 {x[0]}, {x[0]}, s20")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {x[0]}, s20, {x[0]}")
        em.salu(f"s_max_i32 {x[0]}, {x[0]}, 0")
        em.salu(f"s_add_u32 {x[0]}, {x[0]}, {BN - 1}")
        em.salu(f"s_lshr_b32 {nt}, {x[0]}, 6")
        if sp is None:
            em.salu(f"s_lshl_b32 {x[0]}, {nt}, 6")
            em.salu(f"s_min_u32 {rowlim}, {x[0]}, s20")
            return
        # key range sp of 2^log2split: tiles [sp n >> l, (sp+1) n >> l); the
        # row limit relative to the range's first key kst = 64 * first tile
        em.salu(f"s_mul_i32 {x[0]}, {sp}, {nt}")
        em.salu(f"s_lshr_b32 {x[0]}, {x[0]}, {self.s_l2s}")        # first tile
        em.salu(f"s_add_u32 {x[1]}, {sp}, 1")
        em.salu(f"s_mul_i32 {x[1]}, {x[1]}, {nt}")
        em.salu(f"s_lshr_b32 {x[1]}, {x[1]}, {self.s_l2s}")        # end tile
        em.salu(f"s_sub_u32 {nt}, {x[1]}, {x[0]}")
        em.salu(f"s_lshl_b32 {kst}, {x[0]}, 6")
        em.salu(f"s_lshl_b32 {x[1]}, {x[1]}, 6")
        em.salu(f"s_min_u32 {x[1]}, {x[1]}, s20")
        em.salu(f"s_sub_u32 {rowlim}, {x[1]}, {kst}")

    def kv_bases(self, b, hq, kb, vb, kst=None):
        """K and V byte bases of (b, kv-head of hq) (+ kst rows): kv-head =
        (hq * gmagic) >> 20."""
        em, x, D = self.em, self.s_x, self.D
        em.salu(f"s_mul_i32 {x[5]}, {hq}, s26")
        em.salu(f"s_lshr_b32 {x[5]}, {x[5]}, 20")
        em.salu(f"s_mul_i32 {x[0]}, {b}, s20")
        em.salu(f"s_mul_i32 {x[2]}, {x[0]}, {self.s_rowb}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[0]}, {self.s_rowb}")
        em.salu(f"s_mul_i32 {x[4]}, {x[5]}, {D * 2}")
        em.salu(f"s_add_u32 {x[2]}, {x[2]}, {x[4]}")
        em.salu(f"s_addc_u32 {x[3]}, {x[3]}, 0")
        if kst is not None:
            em.salu(f"s_mul_i32 {x[4]}, {kst}, {self.s_rowb}")
            em.salu(f"s_mul_hi_u32 {x[5]}, {kst}, {self.s_rowb}")
            em.salu(f"s_add_u32 {x[2]}, {x[2]}, {x[4]}")
            em.salu(f"s_addc_u32 {x[3]}, {x[3]}, {x[5]}")
        em.salu(f"s_add_u32 {kb.r(0)}, s10, {x[2]}")
        em.salu(f"s_addc_u32 {kb.r(1)}, s11, {x[3]}")
        em.salu(f"s_add_u32 {vb.r(0)}, s12, {x[2]}")
        em.salu(f"s_addc_u32 {vb.r(1)}, s13, {x[3]}")

    def derive(self):
        """The current item's rows, key range, block thresholds, K/V bases and
        O / LSE resources, from s_b, s_hq, s_qt."""
        em, x = self.em, self.s_x
        em.salu(f"s_lshl_b32 {x[0]}, {self.s_qt}, 9")               # q0
        em.salu(f"s_lshl_b32 {x[1]}, {self.s_w}, 5")
        em.salu(f"s_add_u32 {self.s_rb[0]}, {x[0]}, {x[1]}")
        em.salu(f"s_sub_u32 {self.s_rb[1]}, {x[0]}, {x[1]}")
        em.salu(f"s_add_u32 {self.s_rb[1]}, {self.s_rb[1]}, {32 * 15}")
        em.salu(f"s_sub_i32 {self.s_off}, s20, s19")              # Skv - Sq
        if self.split:
            self.kv_range(self.s_qt, self.s_ntiles, self.s_rowlim, self.s_sp, self.s_kst)
        else:
            self.kv_range(self.s_qt, self.s_ntiles, self.s_rowlim)
        # block thresholds: a row's last visible key is min(row + off, Skv-1)
        # (causal) or Skv-1; fu_b = that of the block's first row - 31,
        # dl_b = that of its last row
        em.salu(f"s_sub_i32 {x[1]}, s20, 1")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {x[2]}, s20, {self.s_off}")
        for qb in range(2):
            em.salu(f"s_add_i32 {x[0]}, {self.s_rb[qb]}, {x[2]}")
            em.salu(f"s_min_i32 {self.s_fu[qb]}, {x[0]}, {x[1]}")
            em.salu(f"s_sub_i32 {self.s_fu[qb]}, {self.s_fu[qb]}, 31")
            em.salu(f"s_add_i32 {x[0]}, {x[0]}, 31")
            em.salu(f"s_min_i32 {self.s_dl[qb]}, {x[0]}, {x[1]}")
        self.kv_bases(self.s_b, self.s_hq, self.s_kbase, self.s_vbase,
                      self.s_kst if self.split else None)
        self.out_desc()

    def next_info(self, l_done):
        """Decode the item of round r+1 into s_nb/s_nhq/s_nqt with its K/V
        bases, row limit and tile count (s_nnt = 0 when there is none)."""
        em = self.em
        l_none = self.lab("nonext")
        em.salu(f"s_add_u32 {self.s_y[0]}, {self.s_r}, 1")
        if self.split:
            self.decode(self.s_y[0], (self.s_nb, self.s_nhq, self.s_nqt, self.s_nsp), l_none)
            self.kv_range(self.s_nqt, self.s_nnt, self.s_nrl, self.s_nsp, self.s_y[1])
            self.kv_bases(self.s_nb, self.s_nhq, self.s_nkb, self.s_nvb, self.s_y[1])
        else:
            self.decode(self.s_y[0], (self.s_nb, self.s_nhq, self.s_nqt), l_none)
            self.kv_range(self.s_nqt, self.s_nnt, self.s_nrl)
            self.kv_bases(self.s_nb, self.s_nhq, self.s_nkb, self.s_nvb)
        em.salu(f"s_branch {l_done}")
        em.label(l_none)
        em.salu(f"s_mov_b32 {self.s_nnt}, 0")
        em.salu(f"s_mov_b32 {self.s_nrl}, 0")
        em.label(l_done)

    def emit_qo_desc(self, rs, base, b, hq):
        """Q (base s8) or O (base s14) buffer resource of (b, hq)."""
        em, D, x = self.em, self.D, self.s_x
        em.salu(f"s_mul_i32 {x[0]}, s19, s21")
        em.salu(f"s_mul_i32 {x[4]}, {b}, {x[0]}")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {hq}")
        em.salu(f"s_mul_i32 {x[2]}, {x[4]}, {D * 2}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[4]}, {D * 2}")
        em.salu(f"s_sub_u32 {x[5]}, {x[0]}, {hq}")
        em.salu(f"s_mul_i32 {x[5]}, {x[5]}, {D * 2}")
        em.salu(f"s_add_u32 {rs.r(0)}, s{base}, {x[2]}")
        em.salu(f"s_addc_u32 {rs.r(1)}, s{base + 1}, {x[3]}")
        em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
        em.salu(f"s_mov_b32 {rs.r(2)}, {x[5]}")
        em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")

    def out_desc(self):
        """O and LSE buffer resources of the current item (with key ranges:
        its slices of the partial buffers, O fp32 [range][B][Hq][Sq][D] and
        LSE fp32 [range][B][Hq][Sq])."""
        em, x = self.em, self.s_x
        if self.split:
            D = self.D
            em.salu(f"s_mul_i32 {x[4]}, {self.s_sp}, s18")
            em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_b}")
            em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s21")
            em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_hq}")
            em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s19")                  # row index
            for rs, base, rb in ((self.s_ro, 14, D * 4), (self.s_rl, 16, 4)):
                em.salu(f"s_mul_i32 {x[2]}, {x[4]}, {rb}")
                em.salu(f"s_mul_hi_u32 {x[3]}, {x[4]}, {rb}")
                em.salu(f"s_add_u32 {rs.r(0)}, s{base}, {x[2]}")
                em.salu(f"s_addc_u32 {rs.r(1)}, s{base + 1}, {x[3]}")
                em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
                em.salu(f"s_mul_i32 {rs.r(2)}, s19, {rb}")
                em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")
            return
        self.emit_qo_desc(self.s_ro, 14, self.s_b, self.s_hq)
        em.salu(f"s_mul_i32 {x[4]}, {self.s_b}, s21")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_hq}")
        em.salu(f"s_mul_i32 {x[4]}, {x[4]}, s19")
        em.salu(f"s_mul_i32 {x[2]}, {x[4]}, 4")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[4]}, 4")
        em.salu(f"s_add_u32 {self.s_rl.r(0)}, s16, {x[2]}")
        em.salu(f"s_addc_u32 {self.s_rl.r(1)}, s17, {x[3]}")
        em.salu(f"s_and_b32 {self.s_rl.r(1)}, {self.s_rl.r(1)}, 0xffff")
        em.salu(f"s_lshl_b32 {self.s_rl.r(2)}, s19, 2")
        em.salu(f"s_mov_b32 {self.s_rl.r(3)}, 0x20000")
        em.salu(f"s_or_b32 {x[0]}, s16, s17")
        em.salu(f"s_cmp_eq_u32 {x[0]}, 0")
        em.salu(f"s_cselect_b32 {self.s_rl.r(2)}, 0, {self.s_rl.r(2)}")

    def row_of_block(self, qb, dst):
        """dst = query row of this lane in block qb (rb + lane % 32)."""
        em = self.em
        em.valu(f"v_and_b32 {dst}, 31, v0", dst=[dst], src=["v0"])
        em.valu(f"v_add_u32 {dst}, {self.s_rb[qb]}, {dst}", dst=[dst], src=[dst])

    def load_q(self, b, hq, qt):
        """Q rows of the wave (blocks w and 15-w of query tile qt of (b, hq))
        straight into the Q AGPRs (16 loads)."""
        em, x, t = self.em, self.s_x, self.v_t
        self.emit_qo_desc(self.s_rq, 8, b, hq)
        em.salu(f"s_mul_i32 {x[0]}, s21, {self.D * 2}")
        em.salu(f"s_lshl_b32 {x[1]}, {qt}, 9")
        em.salu(f"s_lshl_b32 {x[2]}, {self.s_w}, 5")
        em.salu(f"s_add_u32 {x[3]}, {x[1]}, {x[2]}")                 # row base, block 0
        em.salu(f"s_sub_u32 {x[4]}, {x[1]}, {x[2]}")
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {32 * 15}")               # block 1
        em.valu(f"v_lshrrev_b32 {t.r(2)}, 5, v0", dst=[t.r(2)], src=["v0"])
        em.valu(f"v_lshlrev_b32 {t.r(2)}, 4, {t.r(2)}", dst=[t.r(2)], src=[t.r(2)])
        for qb in range(2):
            r_ = t.r(qb)
            em.valu(f"v_and_b32 {r_}, 31, v0", dst=[r_], src=["v0"])
            em.valu(f"v_add_u32 {r_}, {x[3 + qb]}, {r_}", dst=[r_], src=[r_])
            em.valu(f"v_mul_lo_u32 {r_}, {r_}, {x[0]}", dst=[r_], src=[r_])
            em.valu(f"v_add_u32 {r_}, {r_}, {t.r(2)}", dst=[r_], src=[r_, t.r(2)])
        for qb in range(2):
            for s_ in range(self.NS):
                dst = str(self.a_Q[qb][s_])
                em.vmem_load_to(f"buffer_load_dwordx4 {dst}, {t.r(qb)}, {self.s_rq}, 0 offen offset:{32 * s_}",
                                dst, src=[t.r(qb)])

    # ------------------------------------------------------------------------
    # K/V DMA
    # ------------------------------------------------------------------------
    def emit_dma_desc(self, tile, kb, vb, rowlim):
        """Buffer resources s_rk / s_rv of tile `tile` (sgpr) of the K/V rows at
        kb / vb: base + 64*tile*rowb, size = the bytes up to rowlim (0 past it)."""
        em, y, rb = self.em, self.s_y, self.s_rowb
        em.salu(f"s_lshl_b32 {y[0]}, {tile}, 6")
        em.salu(f"s_sub_i32 {y[1]}, {rowlim}, {y[0]}")
        em.salu(f"s_max_i32 {y[1]}, {y[1]}, 0")
        em.salu(f"s_mul_i32 {y[2]}, {y[1]}, {rb}")
        em.salu(f"s_mul_hi_u32 {y[3]}, {y[1]}, {rb}")
        em.salu(f"s_cmp_eq_u32 {y[3]}, 0")
        em.salu(f"s_cselect_b32 {y[2]}, {y[2]}, 0x7fffffff")
        em.salu(f"s_min_u32 {y[2]}, {y[2]}, 0x7fffffff")
        em.salu(f"s_mul_i32 {y[3]}, {y[0]}, {rb}")
        em.salu(f"s_mul_hi_u32 {y[4]}, {y[0]}, {rb}")
        for rs, bb in ((self.s_rk, kb), (self.s_rv, vb)):
            em.salu(f"s_add_u32 {rs.r(0)}, {bb.r(0)}, {y[3]}")
            em.salu(f"s_addc_u32 {rs.r(1)}, {bb.r(1)}, {y[4]}")
            em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
            em.salu(f"s_mov_b32 {rs.r(2)}, {y[2]}")
            em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")

    def emit_dma(self, g):
        """The wave's 2 K and 2 V row loads of stream tile g (sgpr, counted from
        the current item's tile 0): the current item's tile g when g < n,
        else the next item's tile g - n.  A tile with keys goes to LDS slot
        (ring + g) % 4; a tile past its item's last (all zeros) goes to the
        spare region, so it never overwrites a slot in use."""
        em, y, x = self.em, self.s_y, self.s_x
        l_next, l_go, l_slot = self.lab("dnext"), self.lab("dgo"), self.lab("dslot")
        em.salu(f"s_cmp_lt_u32 {g}, {self.s_ntiles}")
        em.salu(f"s_cbranch_scc0 {l_next}")
        self.emit_dma_desc(g, self.s_kbase, self.s_vbase, self.s_rowlim)
        em.salu(f"s_branch {l_slot}")
        em.label(l_next)
        em.salu(f"s_sub_u32 {x[5]}, {g}, {self.s_ntiles}")
        self.emit_dma_desc(x[5], self.s_nkb, self.s_nvb, self.s_nrl)
        em.salu(f"s_cmp_lt_u32 {x[5]}, {self.s_nnt}")
        em.salu(f"s_cbranch_scc1 {l_slot}")
        em.salu(f"s_add_u32 {y[5]}, {self.s_wrow}, {self.DUMP}")          # K rows of the wave
        em.salu(f"s_add_u32 {y[1]}, {y[5]}, {self.TILE}")                 # V rows of the wave
        em.salu(f"s_branch {l_go}")
        em.label(l_slot)
        em.salu(f"s_add_u32 {y[5]}, {g}, {self.s_ring}")
        em.salu(f"s_and_b32 {y[5]}, {y[5]}, {SLOTS - 1}")
        em.salu(f"s_mul_i32 {y[5]}, {y[5]}, {self.TILE}")
        em.salu(f"s_add_u32 {y[5]}, {y[5]}, {self.s_wrow}")              # K rows of the wave
        em.salu(f"s_add_u32 {y[1]}, {y[5]}, {self.VREG}")                # V rows of the wave
        em.label(l_go)
        for desc, slot, voff in ((self.s_rk, y[5], self.v_kdma), (self.s_rv, y[1], self.v_vdma)):
            for i in range(self.DPW):
                em.salu(f"s_add_u32 m0, {slot}, {self.RPD * i * self.ROW}")
                em.salu("s_nop 0")                 # SALU write of M0 -> LDS DMA: one wait state
                em.vmem(f"buffer_load_dwordx4 {voff.r(i)}, {desc}, 0 offen lds", src=[voff.r(i)])

    # ------------------------------------------------------------------------
    # operand fragments and the MFMA phase
    # ------------------------------------------------------------------------
    def frag_v(self, kb, db, th):
        """V^T fragment (dims 32db.., keys 16th.. of sub-tile kb of the V tile
        at v_vb): two transposing reads.  Returns (reads(buf, tmp), mfmas(buf))."""
        em = self.em

        def reads(buf, _tmp):
            R = self.v_R[buf]
            tmp = self.v_t.r(2 + db % 2)
            if th == 0:
                em.valu(f"v_xor_b32 {tmp}, {db << 6}, {self.v_vb}", dst=[tmp], src=[str(self.v_vb)])
            for e in range(2):
                off = (32 * kb + 16 * th + 8 * e) * self.ROW
                em.ds_read(f"ds_read_b64_tr_b16 {R.r(2 * e, 2)}, {tmp} offset:{off}", R.r(2 * e, 2), tmp)
        return reads, ("v", db, th)

    def frag_k(self, kb, s):
        """K fragment (keys of sub-tile kb of the K tile at v_kb, dims 16s..)."""
        em = self.em

        def reads(buf, tmp):
            R = self.v_R[buf]
            em.valu(f"v_xor_b32 {tmp}, {s << 5}, {self.v_kb}", dst=[tmp], src=[str(self.v_kb)])
            em.ds_read(f"ds_read_b128 {R}, {tmp} offset:{kb * 32 * self.ROW}", str(R), tmp)
        return reads, ("k", s)

    def frag_mfma(self, tag, buf, qb, first_pv=False):
        em = self.em
        R = str(self.v_R[buf])
        if tag[0] == "v":
            _, db, th = tag
            o = str(self.v_O[qb][db])
            c = "0" if (first_pv and th == 0) else o
            em.mfma(self.mfma_op, o, R, self.v_S[qb].r(4 * th, 4), c)
        else:
            _, s = tag
            d = str(self.v_S[qb])
            em.mfma(self.mfma_op, d, R, str(self.a_Q[qb][s]), "0" if s == 0 else d)

    def pv_frags(self, kb):
        return [self.frag_v(kb, db, th) for db in range(self.NDB) for th in range(2)]

    def qk_frags(self, kb):
        return [self.frag_k(kb, s) for s in range(self.NS)]

    def prefetch(self, frags):
        """Reads of the first two fragments of the next MFMA phase (buffers 0, 1)."""
        t = self.v_t
        for i in range(min(2, len(frags))):
            frags[i][0](i, t.r(i))

    def m_phase(self, pv, qk, first_pv=False, pv_blocks=(0, 1), qk_blocks=(0, 1)):
        """MFMAs of the P.V fragments `pv` (for the query blocks pv_blocks)
        then of the S^T fragments `qk` (for qk_blocks), each fragment once for
        each of its blocks.  The first two fragments of pv + qk are already in
        flight (buffers 0, 1); fragment i+2 is read into the buffer of
        fragment i-1 after the first MFMA of fragment i."""
        t = self.v_t
        full = list(pv) + list(qk)
        frags = [(f, pv_blocks) for f in (pv if pv_blocks else [])] + \
                [(f, qk_blocks) for f in (qk if qk_blocks else [])]
        n = len(frags)
        if [f for f, _ in frags[:2]] != full[:2]:
            for i in range(min(2, n)):
                frags[i][0][0](i, t.r(i))
        for i, ((reads, tag), blocks) in enumerate(frags):
            buf = i % 3
            for k, qb in enumerate(blocks):
                self.frag_mfma(tag, buf, qb, first_pv)
                if k == 0 and i + 2 < n:
                    frags[i + 2][0][0]((i + 2) % 3, t.r((i + 2) % 2))

    def m_phase_sel(self, pv, qk, first_pv=False):
        """The MFMA phase with MFMAs only for live query blocks.  A block is
        live for a sub-tile whose first key k0 is at most dl_b, the last key
        any of its rows sees (block 0's rows come first, so it dies first).
        At the phase start s_k0 is the first key of the S^T sub-tile; the
        P.V sub-tile starts 32 keys earlier.  Every block live is the common
        case; the other combinations run out of line."""
        em, k0, dl, x = self.em, self.s_k0, self.s_dl, self.s_x[0]
        l_v, l_join = self.lab("mvar"), self.lab("mjoin")
        # the wave in its MFMA phase issues ahead of the SIMD's other wave (in
        # its softmax phase), so the matrix core is fed first
        em.salu("s_setprio 1")
        test = dl[0]
        if not qk:                                 # P.V only: the previous sub-tile
            em.salu(f"s_sub_u32 {x}, {k0}, 32")
            em.salu(f"s_cmp_le_i32 {x}, {dl[0]}")
        else:
            em.salu(f"s_cmp_le_i32 {k0}, {dl[0]}")
        em.salu(f"s_cbranch_scc0 {l_v}")
        snap = em.snapshot()
        self.m_phase(pv, qk, first_pv)
        em.label(l_join)
        em.salu("s_setprio 0")

        def variants():
            # block 0 is not live for the S^T sub-tile (or, P.V only, for P.V)
            B = (1,)
            if not qk:
                l00 = self.lab("m00")
                em.salu(f"s_cmp_le_i32 {x}, {dl[1]}")
                em.salu(f"s_cbranch_scc0 {l00}")
                self._mvar(snap, l_join, pv, qk, first_pv, B, ())
                em.label(l00)
                self._mvar(snap, l_join, pv, qk, first_pv, (), ())
                return
            if not pv:
                l0 = self.lab("m00")
                em.salu(f"s_cmp_le_i32 {k0}, {dl[1]}")
                em.salu(f"s_cbranch_scc0 {l0}")
                self._mvar(snap, l_join, pv, qk, first_pv, (), B)
                em.label(l0)
                self._mvar(snap, l_join, pv, qk, first_pv, (), ())
                return
            l_pv2, l_22, l_32, l_00 = self.lab("mpv2"), self.lab("m22"), self.lab("m32"), self.lab("m00")
            em.salu(f"s_sub_u32 {x}, {k0}, 32")
            em.salu(f"s_cmp_le_i32 {x}, {dl[0]}")
            em.salu(f"s_cbranch_scc0 {l_pv2}")
            em.salu(f"s_cmp_le_i32 {k0}, {dl[1]}")
            em.salu(f"s_cbranch_scc1 {l_32}")
            self._mvar(snap, l_join, pv, qk, first_pv, (0, 1), ())
            em.label(l_32)
            self._mvar(snap, l_join, pv, qk, first_pv, (0, 1), B)
            em.label(l_pv2)
            em.salu(f"s_cmp_le_i32 {x}, {dl[1]}")
            em.salu(f"s_cbranch_scc0 {l_00}")
            em.salu(f"s_cmp_le_i32 {k0}, {dl[1]}")
            em.salu(f"s_cbranch_scc1 {l_22}")
            self._mvar(snap, l_join, pv, qk, first_pv, B, ())
            em.label(l_22)
            self._mvar(snap, l_join, pv, qk, first_pv, B, B)
            em.label(l_00)
            self._mvar(snap, l_join, pv, qk, first_pv, (), ())

        self.deferred.append((snap, l_v, None, variants))

    def _mvar(self, snap, l_join, pv, qk, first_pv, pvb, qkb):
        em = self.em
        em.restore(snap)
        self.m_phase(pv, qk, first_pv, pvb, qkb)
        em.drain()
        em.salu(f"s_branch {l_join}")

    # ------------------------------------------------------------------------
    # softmax phase
    # ------------------------------------------------------------------------
    def emit_mask(self, blocks=(0, 1)):
        """S entries of keys past each row's last visible key -> -inf.
        Register i of a block holds key k0 + 8*(i >> 2) + 4h + (i & 3); the
        last visible key is min(row + off, Skv - 1) (causal) or Skv - 1."""
        em = self.em
        t = self.v_t
        d, h4, ninf = t.r(0), t.r(1), t.r(2)
        x = self.s_x
        em.valu(f"v_lshrrev_b32 {h4}, 5, v0", dst=[h4], src=["v0"])
        em.valu(f"v_lshlrev_b32 {h4}, 2, {h4}", dst=[h4], src=[h4])          # 4h
        em.salu(f"s_sub_i32 {x[1]}, s20, 1")                                  # Skv - 1
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {x[2]}, s20, {self.s_off}")                  # row offset of the limit
        em.valu(f"v_mov_b32 {ninf}, 0xff800000", dst=[ninf])
        for qb in blocks:
            S = self.v_S[qb]
            self.row_of_block(qb, d)
            em.valu(f"v_add_u32 {d}, {x[2]}, {d}", dst=[d], src=[d])
            em.valu(f"v_min_i32 {d}, {x[1]}, {d}", dst=[d], src=[d])
            em.valu(f"v_sub_u32 {d}, {d}, {h4}", dst=[d], src=[d, h4])
            em.valu(f"v_subrev_u32 {d}, {self.s_k0}, {d}", dst=[d], src=[d])
            for i in range(16):
                ci = 8 * (i >> 2) + (i & 3)
                em.valu(f"v_cmp_lt_i32 vcc, {d}, {ci}", src=[d])
                em.valu(f"v_cndmask_b32 {S.r(i)}, {S.r(i)}, {ninf}, vcc", dst=[S.r(i)], src=[S.r(i), ninf])

    def emit_rowmax_init(self, blocks=(0, 1)):
        """First sub-tile: mc = c * rowmax (0 for rows with every key masked,
        and for blocks without a visible key)."""
        em = self.em
        t = self.v_t
        for qb in range(2):
            mc = self.v_mc.r(qb)
            if qb not in blocks:
                em.valu(f"v_mov_b32 {mc}, 0", dst=[mc])
                continue
            S, mx, tmp = self.v_S[qb], t.r(0), t.r(1)
            em.valu(f"v_max3_f32 {mx}, {S.r(0)}, {S.r(1)}, {S.r(2)}", dst=[mx], src=[S.r(0), S.r(1), S.r(2)])
            for i in range(3, 15, 2):
                em.valu(f"v_max3_f32 {mx}, {mx}, {S.r(i)}, {S.r(i + 1)}", dst=[mx], src=[mx, S.r(i), S.r(i + 1)])
            em.valu(f"v_max_f32 {mx}, {mx}, {S.r(15)}", dst=[mx], src=[mx, S.r(15)])
            em.valu(f"v_mov_b32 {tmp}, {mx}", dst=[tmp], src=[mx])
            em.valu(f"v_permlane32_swap_b32 {mx}, {tmp}", dst=[mx, tmp], src=[mx, tmp])
            em.valu(f"v_max_f32 {mx}, {mx}, {tmp}", dst=[mx], src=[mx, tmp])
            em.valu(f"v_mul_f32 {mc}, s24, {mx}", dst=[mc], src=[mx])
            em.valu(f"v_cmp_eq_f32 vcc, 0xff800000, {mx}", src=[mx])
            em.valu(f"v_cndmask_b32 {mc}, {mc}, 0, vcc", dst=[mc], src=[mc])

    def softmax_ops(self, blocks=(0, 1)):
        """In place: S = 2^(c*S - mc); rs = lane sums per block; P = S rounded
        (over the first 8 registers of each block); the trigger masks.  Blocks
        outside `blocks` get rs = 0 and a clear trigger mask."""
        em = self.em
        out = []
        E = []
        for qb in range(2):
            S, mc = self.v_S[qb], self.v_mc.r(qb)
            e = []
            for c4 in range(4):
                for i in range(4 * c4, 4 * c4 + 4):
                    e.append(lambda S=S, mc=mc, i=i: em.valu(
                        f"v_fma_f32 {S.r(i)}, {S.r(i)}, s24, -{mc}", dst=[S.r(i)], src=[S.r(i), mc]))
                for i in range(4 * c4, 4 * c4 + 4):
                    e.append(lambda S=S, i=i: em.valu(
                        f"v_exp_f32 {S.r(i)}, {S.r(i)}", dst=[S.r(i)], src=[S.r(i)], trans=True))
            E.append(e)
        # sums: two chains per block (rs and a temp), folded at the end
        Ssum = []
        for qb in range(2):
            S, ra, rb = self.v_S[qb], self.v_rs.r(qb), self.v_t.r(qb)
            s = [lambda S=S, ra=ra: em.valu(f"v_add_f32 {ra}, {S.r(0)}, {S.r(1)}", dst=[ra], src=[S.r(0), S.r(1)]),
                 lambda S=S, rb=rb: em.valu(f"v_add_f32 {rb}, {S.r(2)}, {S.r(3)}", dst=[rb], src=[S.r(2), S.r(3)])]
            for i in range(4, 16):
                acc = ra if i % 2 == 0 else rb
                s.append(lambda S=S, acc=acc, i=i: em.valu(
                    f"v_add_f32 {acc}, {acc}, {S.r(i)}", dst=[acc], src=[acc, S.r(i)]))
            s.append(lambda ra=ra, rb=rb: em.valu(f"v_add_f32 {ra}, {ra}, {rb}", dst=[ra], src=[ra, rb]))
            Ssum.append(s)
        # order: exponentials of the blocks chunk by chunk, the sums of a
        # chunk one chunk later
        for c4 in range(4):
            for qb in blocks:
                out += E[qb][8 * c4:8 * c4 + 8]
            if c4 >= 1:
                for qb in blocks:
                    out += Ssum[qb][4 * (c4 - 1):4 * c4]
        for qb in blocks:
            out += Ssum[qb][12:]
        for qb, msk in ((0, self.s_m1), (1, self.s_m2)):
            if qb in blocks:
                out.append(lambda qb=qb, msk=msk: em.valu(
                    f"v_cmp_lt_f32 {msk}, {self.s_thr}, {self.v_rs.r(qb)}", src=[self.v_rs.r(qb)]))
            else:
                out.append(lambda qb=qb, msk=msk: (
                    em.valu(f"v_mov_b32 {self.v_rs.r(qb)}, 0", dst=[self.v_rs.r(qb)]),
                    em.salu(f"s_mov_b64 {msk}, 0")))
        for qb in blocks:
            S = self.v_S[qb]
            for k in range(8):
                lo, hi = S.r(2 * k), S.r(2 * k + 1)
                out.append(lambda S=S, k=k, lo=lo, hi=hi: em.valu(
                    f"{self.cvt_op} {S.r(k)}, {lo}, {hi}", dst=[S.r(k)], src=[lo, hi]))
        return out

    def emit_softmax(self, blocks=(0, 1)):
        for f in self.softmax_ops(blocks):
            f()

    def emit_l(self, first=False):
        em = self.em
        for qb in range(2):
            l, rs = self.v_l.r(qb), self.v_rs.r(qb)
            if first:
                em.valu(f"v_mov_b32 {l}, {rs}", dst=[l], src=[rs])
            else:
                em.valu(f"v_add_f32 {l}, {l}, {rs}", dst=[l], src=[l, rs])

    def emit_state_branch(self, body, tag):
        """Emit body(states) for the block states of the sub-tile at k0:
        'F' every row sees every key (k0 <= fu_b), 'D' no row sees a key
        (k0 > dl_b), else 'M' (masked).  Block 0 is never ahead of block 1,
        so the common case is one compare ((F, F)); the others, (M, F), (M, M),
        (D, F), (D, M) and (D, D), run out of line."""
        em, k0, fu, dl = self.em, self.s_k0, self.s_fu, self.s_dl
        l_v, l_join = self.lab(f"vvar{tag}"), self.lab(f"vjoin{tag}")
        em.salu(f"s_cmp_le_i32 {k0}, {fu[0]}")
        em.salu(f"s_cbranch_scc0 {l_v}")
        snap = em.snapshot()
        body(("F", "F"))
        em.label(l_join)

        def one(st):
            em.restore(snap)
            body(st)
            em.drain()
            em.salu(f"s_branch {l_join}")

        def variants():
            l_d, l_mf, l_df, l_dd = self.lab("vd"), self.lab("vmf"), self.lab("vdf"), self.lab("vdd")
            em.salu(f"s_cmp_gt_i32 {k0}, {dl[0]}")
            em.salu(f"s_cbranch_scc1 {l_d}")
            em.salu(f"s_cmp_le_i32 {k0}, {fu[1]}")
            em.salu(f"s_cbranch_scc1 {l_mf}")
            one(("M", "M"))
            em.label(l_mf)
            one(("M", "F"))
            em.label(l_d)
            em.salu(f"s_cmp_le_i32 {k0}, {fu[1]}")
            em.salu(f"s_cbranch_scc1 {l_df}")
            em.salu(f"s_cmp_gt_i32 {k0}, {dl[1]}")
            em.salu(f"s_cbranch_scc1 {l_dd}")
            one(("D", "M"))
            em.label(l_df)
            one(("D", "F"))
            em.label(l_dd)
            one(("D", "D"))

        self.deferred.append((snap, l_v, None, variants))

    def emit_slow(self, kb):
        """Out-of-line slow path of the softmax of sub-tile kb of the K tile at
        v_kb: recompute S^T, move mc to c * max(m, rowmax), rescale O and l,
        redo the exponentials."""
        em = self.em
        t = self.v_t
        l_slow, l_back = self.lab("slow"), self.lab("back")
        em.salu(f"s_or_b64 {self.s_m1}, {self.s_m1}, {self.s_m2}")
        em.salu(f"s_cbranch_scc1 {l_slow}")
        snap = em.snapshot()

        def body():
            em.drain()
            frags = self.qk_frags(kb)
            for i, (reads, tag) in enumerate(frags):
                reads(i % 3, t.r(0))
                for qb in range(2):
                    self.frag_mfma(tag, i % 3, qb)
            em.drain()
            l_nm = self.lab("slownm")
            em.salu(f"s_cmp_gt_i32 {self.s_k0}, {self.s_fu[0]}")
            em.salu(f"s_cbranch_scc0 {l_nm}")
            self.emit_mask()
            em.drain()
            em.label(l_nm)
            for qb in range(2):
                S, mx, tmp, a = self.v_S[qb], t.r(0), t.r(1), t.r(2)
                em.valu(f"v_max3_f32 {mx}, {S.r(0)}, {S.r(1)}, {S.r(2)}", dst=[mx], src=[S.r(0), S.r(1), S.r(2)])
                for i in range(3, 15, 2):
                    em.valu(f"v_max3_f32 {mx}, {mx}, {S.r(i)}, {S.r(i + 1)}", dst=[mx], src=[mx, S.r(i), S.r(i + 1)])
                em.valu(f"v_max_f32 {mx}, {mx}, {S.r(15)}", dst=[mx], src=[mx, S.r(15)])
                em.valu(f"v_mov_b32 {tmp}, {mx}", dst=[tmp], src=[mx])
                em.valu(f"v_permlane32_swap_b32 {mx}, {tmp}", dst=[mx, tmp], src=[mx, tmp])
                em.valu(f"v_max_f32 {mx}, {mx}, {tmp}", dst=[mx], src=[mx, tmp])
                mc, l = self.v_mc.r(qb), self.v_l.r(qb)
                # new mc = max(mc, c*mx) (rows without a visible key keep 0)
                em.valu(f"v_mul_f32 {mx}, s24, {mx}", dst=[mx], src=[mx])
                em.valu(f"v_max_f32 {mx}, {mc}, {mx}", dst=[mx], src=[mc, mx])
                em.valu(f"v_sub_f32 {a}, {mc}, {mx}", dst=[a], src=[mc, mx])
                em.valu(f"v_exp_f32 {a}, {a}", dst=[a], src=[a], trans=True)
                em.valu(f"v_mov_b32 {mc}, {mx}", dst=[mc], src=[mx])
                em.valu(f"v_mul_f32 {l}, {l}, {a}", dst=[l], src=[l, a])
                for db in range(self.NDB):
                    blk = self.v_O[qb][db]
                    for i in range(16):
                        em.valu(f"v_mul_f32 {blk.r(i)}, {blk.r(i)}, {a}", dst=[blk.r(i)], src=[blk.r(i), a])
            self.emit_softmax()
            self.emit_l()
            em.drain()
            em.salu(f"s_branch {l_back}")

        self.deferred.append((snap, l_slow, None, body))
        self.emit_l()
        em.label(l_back)

    def v_phase(self, kb, first=False, dma=False, next_frags=(), vb_tile=None):
        """Softmax of the sub-tile at k0 (sub-tile kb of the K tile at v_kb);
        then the DMA of tile u+AHEAD (odd sub-tiles), the V base of the next
        P.V and the prefetch of the next MFMA phase's first fragments."""
        em = self.em

        def body(st):
            live = tuple(qb for qb in (0, 1) if st[qb] != "D")
            masked = tuple(qb for qb in (0, 1) if st[qb] == "M")
            if masked:
                self.emit_mask(masked)
            if first:
                self.emit_rowmax_init(live)
            self.emit_softmax(live)

        self.emit_state_branch(body, "f" if first else "")
        if first:
            self.emit_l(first=True)
        else:
            self.emit_slow(kb)
        if dma:
            # the item's last softmax phase: Q of the next item (the Q AGPRs
            # are free after the last S^T), ahead of its tile 2
            l_noq = self.lab("noq")
            em.salu(f"s_add_u32 {self.s_x[0]}, {self.s_u}, 1")
            em.salu(f"s_cmp_eq_u32 {self.s_x[0]}, {self.s_ntiles}")
            em.salu(f"s_cbranch_scc0 {l_noq}")
            em.salu(f"s_cmp_eq_u32 {self.s_nnt}, 0")
            em.salu(f"s_cbranch_scc1 {l_noq}")
            self.load_q(self.s_nb, self.s_nhq, self.s_nqt)
            em.label(l_noq)
            em.salu(f"s_add_u32 {self.s_y[5]}, {self.s_u}, {AHEAD}")
            self.emit_dma(self.s_y[5])
        if vb_tile is not None:
            self.set_vb(vb_tile)
        self.prefetch(list(next_frags))
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        em.salu("s_barrier")

    def zero_dead_blocks(self):
        """O^T of a query block none of whose rows sees a key of the item's
        range (dl_b below its first key: a causal mask with Sq > Skv, or a key
        range past the block's diagonal) is never accumulated into: clear it
        (out of line, MFMAs of zero operands)."""
        em = self.em
        first = self.s_kst if self.split else 0
        l_z, l_back = self.lab("zero"), self.lab("zback")
        em.salu(f"s_cmp_lt_i32 {self.s_dl[0]}, {first}")
        em.salu(f"s_cbranch_scc1 {l_z}")
        snap = em.snapshot()
        em.label(l_back)

        def body():
            Z = self.v_R[2]
            for i in range(4):
                em.valu(f"v_mov_b32 {Z.r(i)}, 0", dst=[Z.r(i)])
            for qb in range(2):
                l_skip = self.lab("zskip")
                em.salu(f"s_cmp_lt_i32 {self.s_dl[qb]}, {first}")
                em.salu(f"s_cbranch_scc0 {l_skip}")
                for db in range(self.NDB):
                    em.mfma(self.mfma_op, str(self.v_O[qb][db]), str(Z), str(Z), "0")
                em.drain()
                em.label(l_skip)
            em.drain()
            em.salu(f"s_branch {l_back}")

        self.deferred.append((snap, l_z, None, body))

    def set_kb(self, tile):
        """v_kb = K operand base of the item's tile `tile` (sgpr or constant)."""
        em, x = self.em, self.s_x[4]
        em.salu(f"s_add_u32 {x}, {tile}, {self.s_ring}")
        em.salu(f"s_and_b32 {x}, {x}, {SLOTS - 1}")
        em.salu(f"s_mul_i32 {x}, {x}, {self.TILE}")
        em.valu(f"v_add_u32 {self.v_kb}, {x}, {self.v_klane}", dst=[str(self.v_kb)], src=[str(self.v_klane)])

    def set_vb(self, tile):
        """v_vb = V operand base of the item's tile `tile` (sgpr or constant)."""
        em, x = self.em, self.s_x[4]
        em.salu(f"s_add_u32 {x}, {tile}, {self.s_ring}")
        em.salu(f"s_and_b32 {x}, {x}, {SLOTS - 1}")
        em.salu(f"s_mul_i32 {x}, {x}, {self.TILE}")
        em.valu(f"v_add_u32 {self.v_vb}, {x}, {self.v_vlane}", dst=[str(self.v_vb)], src=[str(self.v_vlane)])

    # ------------------------------------------------------------------------
    # epilogue
    # ------------------------------------------------------------------------
    def epilogue(self, empty=False):
        """O / l rounded to the input dtype and LSE = ln2 * (mc + log2 l) (-inf
        when l = 0), for the wave's two query blocks.  With `empty`, zeros
        and -inf (an item with no visible key)."""
        em = self.em
        em.drain()
        F = [self.v_S[0], self.v_S[1]]
        t = self.v_R[1]                   # scratch: rows, offsets, scale
        u = self.v_R[2]
        em.valu(f"v_lshrrev_b32 {t.r(0)}, 5, v0", dst=[t.r(0)], src=["v0"])
        em.valu(f"v_lshlrev_b32 {t.r(3)}, 4, {t.r(0)}", dst=[t.r(3)], src=[t.r(0)])   # 16h
        # row stride: BSHD output, or the fp32 partial rows of a key range
        em.salu(f"s_mul_i32 {self.s_x[0]}, s21, {self.D * 2}")
        if self.split:
            em.salu(f"s_mov_b32 {self.s_x[0]}, {self.D * 4}")
            if empty:
                for c in range(4):
                    em.valu(f"v_mov_b32 {F[0].r(8 + c)}, 0", dst=[F[0].r(8 + c)])
        for qb in range(2):
            l = self.v_l.r(qb)
            if empty:
                em.valu(f"v_mov_b32 {t.r(1)}, 0", dst=[t.r(1)])
                em.valu(f"v_mov_b32 {l}, 0", dst=[l])
            else:
                em.valu(f"v_mov_b32 {t.r(0)}, {l}", dst=[t.r(0)], src=[l])
                em.valu(f"v_permlane32_swap_b32 {l}, {t.r(0)}", dst=[l, t.r(0)], src=[l, t.r(0)])
                em.valu(f"v_add_f32 {l}, {l}, {t.r(0)}", dst=[l], src=[l, t.r(0)])
                em.valu(f"v_rcp_f32 {t.r(1)}, {l}", dst=[t.r(1)], src=[l], trans=True)
                em.valu(f"v_cmp_lt_f32 vcc, 0, {l}", src=[l])
                em.valu(f"v_cndmask_b32 {t.r(1)}, 0, {t.r(1)}, vcc", dst=[t.r(1)], src=[t.r(1)])
            self.row_of_block(qb, u.r(0))
            em.valu(f"v_mul_lo_u32 {t.r(2)}, {u.r(0)}, {self.s_x[0]}", dst=[t.r(2)], src=[u.r(0)])
            em.valu(f"v_add_u32 {t.r(2)}, {t.r(2)}, {t.r(3)}", dst=[t.r(2)], src=[t.r(2), t.r(3)])
            for db in range(self.NDB if self.split else 0):
                # fp32 partial O: lane (l, h) holds dims 32db + 8j + 4h .. +3 in
                # registers 4j .. 4j+3, 16 contiguous bytes of the row
                blk = self.v_O[qb][db]
                for j in range(4):
                    src = F[0].r(8, 4)
                    if not empty:
                        for r in range(4):
                            x_ = blk.r(4 * j + r)
                            em.valu(f"v_mul_f32 {x_}, {x_}, {t.r(1)}", dst=[x_], src=[x_, t.r(1)])
                        src = blk.r(4 * j, 4)
                    em.vmem(f"buffer_store_dwordx4 {src}, {t.r(2)}, {self.s_ro}, 0 offen "
                            f"offset:{128 * db + 32 * j}", src=[src, t.r(2)])
            for db in range(0 if self.split else self.NDB):
                blk = self.v_O[qb][db]
                for jp in range(2):
                    k = 2 * db + jp
                    Fk, o = F[k % 2], 8 + 4 * ((k // 2) % 2)
                    if empty:
                        for c in range(4):
                            em.valu(f"v_mov_b32 {Fk.r(o + c)}, 0", dst=[Fk.r(o + c)])
                    else:
                        for jj in range(2):
                            j = 2 * jp + jj
                            for r in range(4):
                                x_ = blk.r(4 * j + r)
                                em.valu(f"v_mul_f32 {x_}, {x_}, {t.r(1)}", dst=[x_], src=[x_, t.r(1)])
                            for c in range(2):
                                a, b = blk.r(4 * j + 2 * c), blk.r(4 * j + 2 * c + 1)
                                em.valu(f"{self.cvt_op} {Fk.r(o + 2 * jj + c)}, {a}, {b}",
                                        dst=[Fk.r(o + 2 * jj + c)], src=[a, b])
                        for c in range(2):
                            xx, yy = Fk.r(o + c), Fk.r(o + 2 + c)
                            em.valu(f"v_permlane32_swap_b32 {xx}, {yy}", dst=[xx, yy], src=[xx, yy])
                    em.vmem(f"buffer_store_dwordx4 {Fk.r(o, 4)}, {t.r(2)}, {self.s_ro}, 0 offen "
                            f"offset:{64 * db + 32 * jp}", src=[Fk.r(o, 4), t.r(2)])
            # LSE
            em.valu(f"v_lshlrev_b32 {u.r(1)}, 2, {u.r(0)}", dst=[u.r(1)], src=[u.r(0)])
            if empty:
                em.valu(f"v_mov_b32 {u.r(2)}, 0xff800000", dst=[u.r(2)])
            else:
                em.valu(f"v_log_f32 {u.r(2)}, {l}", dst=[u.r(2)], src=[l], trans=True)
                em.valu(f"v_add_f32 {u.r(2)}, {self.v_mc.r(qb)}, {u.r(2)}", dst=[u.r(2)],
                        src=[self.v_mc.r(qb), u.r(2)])
                em.valu(f"v_mul_f32 {u.r(2)}, {f32_hex(LN2)}, {u.r(2)}", dst=[u.r(2)], src=[u.r(2)])
                em.valu(f"v_mov_b32 {u.r(3)}, 0xff800000", dst=[u.r(3)])
                em.valu(f"v_cndmask_b32 {u.r(2)}, {u.r(3)}, {u.r(2)}, vcc", dst=[u.r(2)], src=[u.r(2), u.r(3)])
            # one lane per row stores its LSE (lanes >= 32 hold the same rows)
            em.vmem(f"buffer_store_dword {u.r(2)}, {u.r(1)}, {self.s_rl}, 0 offen", src=[u.r(2), u.r(1)])

    # ------------------------------------------------------------------------
    def cur_ids(self):
        ids = (self.s_b, self.s_hq, self.s_qt)
        return ids + (self.s_sp,) if self.split else ids

    def epilogue_stores(self):
        """Buffer stores one epilogue issues (the vmcnt accounting needs it)."""
        return 2 * (self.NDB * 4 + 1) if self.split else 2 * (self.NDB * 2 + 1)

    def item_start(self):
        """Tile counters and operand bases of the (just derived) item."""
        em = self.em
        em.salu(f"s_mov_b32 {self.s_u}, 0")
        em.salu(f"s_mov_b32 {self.s_k0}, {self.s_kst if self.split else 0}")
        self.set_kb(0)
        self.set_vb(0)

    def body(self):
        em = self.em
        self.alloc()
        self.kernel_setup()
        self.lane_consts()
        em.drain()
        l_exit, l_empty, l_item = self.lab("exit"), self.lab("empty"), self.lab("item")
        l_loop, l_last, l_end = self.lab("loop"), self.lab("last"), self.lab("end")
        # ---- the first item: Q and its tiles 0 .. AHEAD-1 ------------------------
        # (every item with keys has at least AHEAD tiles: the launcher checks)
        self.decode(self.s_r, self.cur_ids(), l_exit)
        self.derive()
        em.salu(f"s_cmp_eq_u32 {self.s_ntiles}, 0")
        em.salu(f"s_cbranch_scc1 {l_empty}")
        self.next_info(self.lab("nd"))
        self.load_q(self.s_b, self.s_hq, self.s_qt)
        for tt in range(AHEAD):
            em.salu(f"s_mov_b32 {self.s_y[5]}, {tt}")
            self.emit_dma(self.s_y[5])
        self.item_start()
        em.drain()
        em.salu(f"s_waitcnt vmcnt({self.LPT * (AHEAD - 1)})")     # Q and tile 0
        em.salu("s_barrier")
        self.zero_dead_blocks()
        self.prefetch(self.qk_frags(0))
        # waves 4-7 run one phase behind
        l_g0 = self.lab("g0")
        em.salu(f"s_cmp_lt_u32 {self.s_w}, 4")
        em.salu(f"s_cbranch_scc1 {l_g0}")
        em.salu("s_barrier")
        em.label(l_g0)
        # ---- one item: tile 0 ---------------------------------------------------------
        em.label(l_item)
        self.m_phase_sel([], self.qk_frags(0))
        em.salu("s_barrier")
        self.v_phase(0, first=True, next_frags=self.pv_frags(0))
        self.m_phase_sel(self.pv_frags(0), self.qk_frags(1), first_pv=True)
        em.salu(f"s_waitcnt vmcnt({self.LPT})")               # stream tile 1
        em.salu("s_barrier")
        self.v_phase(1, dma=True, next_frags=self.pv_frags(1))
        em.salu(f"s_add_u32 {self.s_u}, {self.s_u}, 1")
        em.drain()
        # ---- tiles 1 .. n-1 ---------------------------------------------------------
        em.label(l_loop)
        em.salu(f"s_cmp_ge_u32 {self.s_u}, {self.s_ntiles}")
        em.salu(f"s_cbranch_scc1 {l_last}")
        self.set_kb(self.s_u)
        self.m_phase_sel(self.pv_frags(1), self.qk_frags(0))
        em.salu("s_barrier")
        self.v_phase(0, next_frags=self.pv_frags(0), vb_tile=self.s_u)
        self.m_phase_sel(self.pv_frags(0), self.qk_frags(1))
        em.salu(f"s_waitcnt vmcnt({self.LPT})")               # stream tile u+1
        em.salu("s_barrier")
        self.v_phase(1, dma=True, next_frags=self.pv_frags(1))
        em.salu(f"s_add_u32 {self.s_u}, {self.s_u}, 1")
        em.drain()
        em.salu(f"s_branch {l_loop}")
        # ---- last P.V; the epilogue phase (the other group's last P.V runs
        # next to it); then the next item, whose Q and first tiles are in -----
        em.label(l_last)
        self.m_phase_sel(self.pv_frags(1), [])
        em.salu("s_barrier")
        self.epilogue()
        em.salu(f"s_add_u32 {self.s_ring}, {self.s_ring}, {self.s_ntiles}")
        em.salu(f"s_and_b32 {self.s_ring}, {self.s_ring}, {SLOTS - 1}")
        em.salu(f"s_cmp_eq_u32 {self.s_nnt}, 0")
        em.salu(f"s_cbranch_scc1 {l_end}")
        em.salu(f"s_mov_b32 {self.s_b}, {self.s_nb}")
        em.salu(f"s_mov_b32 {self.s_hq}, {self.s_nhq}")
        em.salu(f"s_mov_b32 {self.s_qt}, {self.s_nqt}")
        if self.split:
            em.salu(f"s_mov_b32 {self.s_sp}, {self.s_nsp}")
        em.salu(f"s_add_u32 {self.s_r}, {self.s_r}, 1")
        self.derive()
        self.next_info(self.lab("nd"))
        self.item_start()
        self.zero_dead_blocks()
        # Q of this item (its tile 2 and the previous epilogue's stores came later)
        em.salu(f"s_waitcnt vmcnt({self.LPT + self.epilogue_stores()})")
        self.prefetch(self.qk_frags(0))
        em.salu("s_barrier")
        em.drain()
        em.salu(f"s_branch {l_item}")
        # ---- end of the items with keys: waves 0-3 balance the barrier count
        em.label(l_end)
        em.salu("s_barrier")
        l_g1 = self.lab("g1")
        em.salu(f"s_cmp_ge_u32 {self.s_w}, 4")
        em.salu(f"s_cbranch_scc1 {l_g1}")
        em.salu("s_barrier")
        em.label(l_g1)
        em.salu(f"s_add_u32 {self.s_r}, {self.s_r}, 1")
        self.decode(self.s_r, self.cur_ids(), l_exit)
        self.derive()
        em.drain()
        # ---- items without a visible key (they come after every item with keys)
        em.label(l_empty)
        self.epilogue(empty=True)
        em.salu(f"s_add_u32 {self.s_r}, {self.s_r}, 1")
        self.decode(self.s_r, self.cur_ids(), l_exit)
        self.derive()
        em.drain()
        em.salu(f"s_branch {l_empty}")
        em.label(l_exit)
        em.salu("s_waitcnt vmcnt(0)")
        em.salu("s_endpgm")
        for snap, l_from, l_join, fn in self.deferred:
            em.restore(snap)
            em.label(l_from)
            fn()
            em.drain()
            if l_join is not None:
                em.salu(f"s_branch {l_join}")

    # ------------------------------------------------------------------------
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
            ("kernarg_size", 96), ("user_sgpr_count", 2),
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
        return "\n".join(out) + "\n", dict(name=name, nv=nv, na=na, total=total, lds=self.LDS,
                                          ns=self.nsgpr + 2, wg=BM)
