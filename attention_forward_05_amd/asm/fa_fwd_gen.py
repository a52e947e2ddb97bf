"""Generator of the gfx950 (MI355X) fused attention forward kernel.

Emits AMDGPU assembly for one (dtype, head dimension) variant.  The kernel
computes, per workgroup, BM = 256 query rows of one (batch, q-head) against
all visible keys of its kv-head, in tiles of 64 keys, with the tiled
online-softmax recurrence of the flash-attention forward pass (JAX Pallas
FlashAttention3 page, `kv_loop`; Croqtile `flash_atten` page, the exp2
form with the logit scale folded into the exponent):

    m_new = max(m, rowmax(S)),  alpha = 2^(c*m - c*m_new),
    P = 2^(c*S - c*m_new),      l = l*alpha + rowsum(P),  O = O*alpha + P.V

with c = scale * log2(e), and at the end O / l and LSE = ln2*(c*m + log2 l).

Layout on the chip (per wave of 64 lanes, 64 query rows):

* S^T = K.Q^T and O^T = V^T.P^T on v_mfma_f32_32x32x16_{bf16,f16}: lane l
  owns query column (l % 32) of each 32-row block, so row max / row sum are
  in-lane plus one v_permlane32_swap, and the alpha rescale is per lane.
* O^T accumulators and Q live in AGPRs (MFMA reads and accumulates there);
  S, P and the K / V operands live in VGPRs, where the softmax runs.
* K and V tiles move from HBM to LDS with buffer_load ... lds (16 bytes per
  lane), two tiles ahead of use through a three-slot K ring and a four-slot
  V ring; buffer loads give zeros past the end of the keys.
* K is read row-major (ds_read_b128); V is read with ds_read_b64_tr_b16,
  which hands each lane one head dimension for four keys.
* Software pipeline over 32-key sub-tiles j: while the P.V MFMAs of j run,
  the VALU computes the row max and exponentials of j+1; while the S^T
  MFMAs of j+2 run, it finishes the exponentials of j+1.  The reference max
  only moves when it rises by more than 2^8 (lazy rescale; rare slow path).
* Causal masking only on sub-tiles that cross a wave's diagonal or the key
  tail; tiles wholly above the diagonal are never loaded.
"""
from __future__ import annotations

import math

from .regs import Alloc, Emitter, Op, weave

BM = 256          # query rows per workgroup
BN = 64           # keys per tile
WAVES = 4
KSLOTS = 4        # K tiles held in LDS
VSLOTS = 5        # V tiles held in LDS
PREFETCH = 4      # tiles loaded ahead of the tile whose keys are multiplied next
THRESH = 32768.0  # lazy-rescale trigger: a half-row sum of p above 2^15
KERNARG_BYTES = 96
LN2 = 0.6931471805599453

# kernarg offsets
KA = dict(q=0, k=8, v=16, o=24, lse=32, B=40, Sq=44, Skv=48, Hq=52, Hkv=56,
          causal=60, c=64, nq_grid=68, gmagic=72, hq_xcd=76, log2split=80)   # nq_grid = nq | G << 16


def kernel_name(dtype: str, D: int) -> str:
    return f"fa_fwd_{dtype}_d{D}_gfx950"


def f32_hex(x: float) -> str:
    import struct
    return "0x%08x" % struct.unpack("<I", struct.pack("<f", x))[0]


class Gen:
    def __init__(self, dtype: str, D: int):
        assert dtype in ("bf16", "f16") and D in (64, 128)
        self.dtype, self.D = dtype, D
        self.name = kernel_name(dtype, D)
        self.mfma_op = "v_mfma_f32_32x32x16_bf16" if dtype == "bf16" else "v_mfma_f32_32x32x16_f16"
        self.cvt_op = "v_cvt_pk_bf16_f32" if dtype == "bf16" else "v_cvt_pk_f16_f32"
        self.NS = D // 16            # k-steps of S^T
        self.NDB = D // 32           # 32-dim blocks of O^T
        self.ROW = D * 2             # bytes per K/V row in LDS
        self.TILE = BN * self.ROW    # bytes per K or V tile
        self.CH = D // 8             # 16-byte chunks per row
        self.RPD = 64 // self.CH     # rows per 64-lane DMA instruction
        self.DPW = (BN // WAVES) // self.RPD  # DMA instructions per wave per K (or V) tile
        self.VBASE = 0
        self.KBASE = VSLOTS * self.TILE
        self.LDS = (VSLOTS + KSLOTS) * self.TILE
        self.em = Emitter()
        self._lab = 0

    # ------------------------------------------------------------------------
    def lab(self, tag):
        self._lab += 1
        return f".L{self.dtype}{self.D}_{tag}_{self._lab}"

    def kswz(self, r: int) -> int:
        return (r & 15) if self.D == 128 else ((r >> 1) & 7)

    def vswz(self, r: int) -> int:
        return 4 * (r & 3) if self.D == 128 else 4 * ((r >> 1) & 1)

    # ------------------------------------------------------------------------
    def alloc(self):
        D, NS, NDB = self.D, self.NS, self.NDB
        V = Alloc("v", 0, 512)
        A = Alloc("a", 0, 256)
        S = Alloc("s", 28, 102)
        self.v_tid = V.take("tid", 1)          # v0 on entry
        r = self.__dict__
        # per-lane constants
        r["v_koff"] = V.take("koff", NS)       # K read offsets (without slot)
        r["v_kaddr"] = V.take("kaddr", NS)     # K read addresses (with slot)
        r["v_voff"] = V.take("voff", NDB)
        r["v_vaddr"] = V.take("vaddr", NDB)
        r["v_kdma"] = V.take("kdma", self.DPW)
        r["v_vdma"] = V.take("vdma", self.DPW)
        r["v_limh"] = V.take("limh", 2)        # per query block: last visible key - 4h
        r["v_qoff"] = V.take("qoff", 2)        # per query block: byte offset of the row in Q/O
        r["v_lseoff"] = V.take("lseoff", 2)
        r["v_m"] = V.take("m", 2)
        r["v_l"] = V.take("l", 2)
        r["v_mc"] = V.take("mc", 2)
        r["v_mx"] = V.take("mx", 2)
        r["v_t"] = V.take("tmp", 8)
        r["v_rs"] = V.take("rs", 2)            # half-row sums of the sub-tile
        r["v_rb"] = V.take("rsb", 2)           # second partial sums
        r["v_d"] = V.take("dmask", 2)
        r["v_ninf"] = V.take("ninf", 1)       # -inf
        r["v_thr"] = V.take("thr", 1)         # lazy-rescale trigger
        r["v_c"] = V.take("c", 1)             # scale * log2(e)
        # S double buffer: S[buf][qb] 16 regs each; E: fp32 exponentials
        r["v_S"] = [[V.take(f"S{b}{q}", 16, 4) for q in range(2)] for b in range(2)]
        r["v_E"] = [V.take(f"E{q}", 16, 4) for q in range(2)]
        # P double buffer: P[buf][qb][th] 4 regs each
        r["v_P"] = [[[V.take(f"P{b}{q}{t}", 4, 4) for t in range(2)] for q in range(2)]
                    for b in range(2)]
        r["v_KO"] = [V.take(f"KO{s}", 4, 4) for s in range(NS)]
        self.nvgpr = (V.next + 7) // 8 * 8
        # AGPRs: O^T accumulators, Q, and the V operands, double buffered
        # VO[buf][th][db] (LDS reads may target AGPRs; MFMA reads them as A)
        r["a_O"] = [[A.take(f"O{q}{d}", 16, 4) for d in range(NDB)] for q in range(2)]
        r["a_Q"] = [[A.take(f"Q{q}{s}", 4, 4) for s in range(NS)] for q in range(2)]
        r["v_VO"] = [[[A.take(f"VO{b}{t}{d}", 4, 4) for d in range(NDB)] for t in range(2)]
                     for b in range(2)]
        self.nagpr = (A.next + 7) // 8 * 8
        assert self.nvgpr <= 256 and self.nagpr <= 256, (self.nvgpr, self.nagpr)
        # SGPRs (s0:1 kernarg ptr, s2..s4 workgroup ids, s8..s27 kernargs)
        t = S.take
        r["s_hq"], r["s_qt"], r["s_b"], r["s_hk"] = t("hq", 1), t("qt", 1), t("b", 1), t("hk", 1)
        r["s_w"], r["s_qw0"], r["s_off"], r["s_ntiles"] = t("w", 1), t("qw0", 1), t("off", 1), t("nt", 1)
        r["s_kvfull"], r["s_rowlim"], r["s_rowb"], r["s_t"] = t("kvf", 1), t("rowlim", 1), t("rowb", 1), t("t", 1)
        r["s_ro"] = t("ro", 4, 4)
        r["s_rl"] = t("rl", 4, 4)
        r["s_rk"] = t("rk", 4, 4)
        # Q is loaded before the first K DMA descriptor is built: same registers
        r["s_rq"] = r["s_rk"]
        r["s_g"], r["s_r"] = t("wg", 1), t("round", 1)
        r["s_nitems"], r["s_P"] = t("nitems", 1), t("pairs", 1)
        r["s_rv"] = t("rv", 4, 4)
        r["s_kb"] = t("kbase", 2, 2)
        r["s_vb"] = t("vbase", 2, 2)
        # ring slots (byte offsets): K read slot of tile t+1 (relative to KBASE),
        # K DMA slot of tile t+PREFETCH (relative), V slots of tiles t, t+1 and
        # t+PREFETCH; the DMA slots with the wave's 16-row offset folded in
        r["s_ksl"], r["s_kdsl"] = t("ksl", 1), t("kdsl", 1)
        r["s_vsl0"], r["s_vsl1"], r["s_vdsl"] = t("vsl0", 1), t("vsl1", 1), t("vdsl", 1)
        r["s_kdw"], r["s_vdw"], r["s_wrow"] = t("kdw", 1), t("vdw", 1), t("wrow", 1)
        r["s_k0"] = t("k0", 1)
        r["s_x"] = [t(f"x{i}", 1) for i in range(6)]
        r["s_y"] = [t(f"y{i}", 1) for i in range(6)]   # DMA stream scratch
        r["s_m1"], r["s_m2"] = t("msk1", 2, 2), t("msk2", 2, 2)
        r["s_neg"] = t("neginf", 1)
        r["s_row"] = t("row", 1)
        r["s_tlast"] = t("tlast", 1)
        r["s_or"] = t("orpair", 2, 2)
        self.nsgpr = S.next

    # convenience accessors ----------------------------------------------------
    def S_(self, buf, qb, i=None):
        b = self.v_S[buf][qb]
        return str(b) if i is None else b.r(i)

    # ------------------------------------------------------------------------
    # prologue: kernargs, block mapping, ranges, descriptors, per-lane constants
    # ------------------------------------------------------------------------
    # Persistent schedule: workgroup g of G takes, in round r, item
    # r*G + (g if r is even else G-1-g) of the list of (batch, q-head, q-tile)
    # items sorted longest first (causal: last q-tile first); the snake order
    # gives every workgroup about the same number of key tiles.
    # ------------------------------------------------------------------------
    def kernel_setup(self):
        """Once per workgroup: kernel arguments, wave index, constants."""
        em, D = self.em, self.D
        em.comment("kernel arguments")
        em.salu("s_load_dwordx16 s[8:23], s[0:1], 0x0")
        em.salu("s_load_dwordx4 s[24:27], s[0:1], 0x40")
        # wave index: v0 (the work-item id, written at wave launch) >> 6
        em.valu(f"v_readfirstlane_b32 {self.s_w}, v0", src=["v0"])
        em.salu(f"s_lshr_b32 {self.s_w}, {self.s_w}, 6")
        em.valu("v_and_b32 v0, 63, v0", dst=["v0"], src=["v0"])  # lane
        em.salu(f"s_mov_b32 {self.s_g}, s2")
        em.salu(f"s_mov_b32 {self.s_r}, 0")
        em.salu("s_waitcnt lgkmcnt(0)")
        em.salu(f"s_mov_b32 {self.s_neg}, 0xff800000")
        em.salu(f"s_mov_b32 {self.s_row}, {self.ROW}")
        em.salu(f"s_mul_i32 {self.s_rowb}, s22, {D * 2}")          # K/V row stride
        em.salu(f"s_mul_i32 {self.s_P}, s18, s21")                 # (batch, head) pairs
        em.salu(f"s_and_b32 {self.s_x[0]}, s25, 0xffff")           # query tiles
        em.salu(f"s_mul_i32 {self.s_nitems}, {self.s_P}, {self.s_x[0]}")
        em.salu(f"s_mul_i32 {self.s_wrow}, {self.s_w}, {16 * self.ROW}")

    def emit_div(self, num, den, q, rem):
        """q = num / den, rem = num - q*den for num, den < 2^24 (VGPR num,
        SGPR den): float reciprocal estimate, then one correction each way."""
        em, t = self.em, self.v_t
        dv = t.r(6)
        em.valu(f"v_mov_b32 {dv}, {den}", dst=[dv])
        em.valu(f"v_cvt_f32_u32 {q}, {num}", dst=[q], src=[num])
        em.valu(f"v_cvt_f32_u32 {rem}, {dv}", dst=[rem], src=[dv])
        em.valu(f"v_rcp_f32 {rem}, {rem}", dst=[rem], src=[rem], trans=True)
        em.valu(f"v_mul_f32 {q}, {q}, {rem}", dst=[q], src=[q, rem])
        em.valu(f"v_cvt_u32_f32 {q}, {q}", dst=[q], src=[q])
        em.valu(f"v_mul_lo_u32 {rem}, {q}, {dv}", dst=[rem], src=[q, dv])
        em.valu(f"v_sub_u32 {rem}, {num}, {rem}", dst=[rem], src=[num, rem])
        # rem < 0 (as signed): q -= 1, rem += den
        em.valu(f"v_cmp_gt_i32 vcc, 0, {rem}", src=[rem])
        em.valu(f"v_cndmask_b32 {t.r(7)}, 0, -1, vcc", dst=[t.r(7)])
        em.valu(f"v_add_u32 {q}, {q}, {t.r(7)}", dst=[q], src=[q, t.r(7)])
        em.valu(f"v_cndmask_b32 {t.r(7)}, 0, {dv}, vcc", dst=[t.r(7)], src=[dv])
        em.valu(f"v_add_u32 {rem}, {rem}, {t.r(7)}", dst=[rem], src=[rem, t.r(7)])
        # rem >= den: q += 1, rem -= den
        em.valu(f"v_cmp_le_u32 vcc, {dv}, {rem}", src=[rem, dv])
        em.valu(f"v_cndmask_b32 {t.r(7)}, 0, 1, vcc", dst=[t.r(7)])
        em.valu(f"v_add_u32 {q}, {q}, {t.r(7)}", dst=[q], src=[q, t.r(7)])
        em.valu(f"v_cndmask_b32 {t.r(7)}, 0, {dv}, vcc", dst=[t.r(7)], src=[dv])
        em.valu(f"v_sub_u32 {rem}, {rem}, {t.r(7)}", dst=[rem], src=[rem, t.r(7)])

    def item_setup_a(self, l_exit):
        """Decode this round's item; set the block's rows, key range and
        buffer resources.  Jumps to l_exit when the workgroup has no item left."""
        em, D = self.em, self.D
        x, t = self.s_x, self.v_t
        # idx = r*G + (r odd ? G-1-g : g)
        em.salu(f"s_lshr_b32 {x[1]}, s25, 16")                     # G
        em.salu(f"s_mul_i32 {x[0]}, {self.s_r}, {x[1]}")
        em.salu(f"s_sub_u32 {x[2]}, {x[1]}, 1")
        em.salu(f"s_sub_u32 {x[2]}, {x[2]}, {self.s_g}")            # G-1-g
        em.salu(f"s_bitcmp1_b32 {self.s_r}, 0")
        em.salu(f"s_cselect_b32 {x[2]}, {x[2]}, {self.s_g}")
        em.salu(f"s_add_u32 {x[0]}, {x[0]}, {x[2]}")                # idx
        em.salu(f"s_cmp_ge_u32 {x[0]}, {self.s_nitems}")
        em.salu(f"s_cbranch_scc1 {l_exit}")
        # level = idx / P, within = idx % P; b = within / Hq, slot = within % Hq
        em.valu(f"v_mov_b32 {t.r(0)}, {x[0]}", dst=[t.r(0)])
        self.emit_div(t.r(0), self.s_P, t.r(1), t.r(2))
        self.emit_div(t.r(2), "s21", t.r(4), t.r(5))
        em.valu(f"v_readfirstlane_b32 {x[3]}, {t.r(1)}", src=[t.r(1)])    # level
        em.valu(f"v_readfirstlane_b32 {self.s_b}, {t.r(4)}", src=[t.r(4)])  # b
        em.valu(f"v_readfirstlane_b32 {x[4]}, {t.r(5)}", src=[t.r(5)])    # head slot
        # hq: spread contiguous head groups over the 8 XCDs (workgroup g -> XCD g % 8)
        em.salu("s_cmp_eq_u32 s27, 0")
        em.salu(f"s_cselect_b32 {x[5]}, 0, 7")
        em.salu(f"s_and_b32 {self.s_hq}, {x[4]}, {x[5]}")
        em.salu(f"s_mul_i32 {self.s_hq}, {self.s_hq}, s27")
        em.salu(f"s_cmp_eq_u32 s27, 0")
        em.salu(f"s_cselect_b32 {x[5]}, 0, 3")
        em.salu(f"s_lshr_b32 {x[5]}, {x[4]}, {x[5]}")
        em.salu(f"s_add_u32 {self.s_hq}, {self.s_hq}, {x[5]}")
        # query tile: longest causal tiles first
        em.salu(f"s_and_b32 {x[5]}, s25, 0xffff")
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, 1")
        em.salu(f"s_sub_u32 {x[5]}, {x[5]}, {x[3]}")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {self.s_qt}, {x[3]}, {x[5]}")
        # kv-head: hq / (Hq / Hkv) as (hq * magic) >> 20
        em.salu(f"s_mul_i32 {self.s_hk}, {self.s_hq}, s26")
        em.salu(f"s_lshr_b32 {self.s_hk}, {self.s_hk}, 20")
        # rows of this wave: qw0 = qt*256 + 64*w
        em.salu(f"s_lshl_b32 {x[1]}, {self.s_qt}, 8")              # q0
        em.salu(f"s_lshl_b32 {x[0]}, {self.s_w}, 6")
        em.salu(f"s_add_u32 {self.s_qw0}, {x[1]}, {x[0]}")
        em.salu(f"s_sub_i32 {self.s_off}, s20, s19")              # Skv - Sq
        # key tiles of the workgroup: kv_end = causal ? min(Skv, min(q0+256, Sq) + off) : Skv
        em.salu(f"s_add_u32 {x[0]}, {x[1]}, {BM}")
        em.salu(f"s_min_i32 {x[0]}, {x[0]}, s19")
        em.salu(f"s_add_i32 {x[0]}, {x[0]}, {self.s_off}")
        em.salu(f"s_min_i32 {x[0]}, {x[0]}, s20")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {x[0]}, s20, {x[0]}")
        em.salu(f"s_max_i32 {x[0]}, {x[0]}, 0")
        em.salu(f"s_add_u32 {x[0]}, {x[0]}, {BN - 1}")
        em.salu(f"s_lshr_b32 {self.s_ntiles}, {x[0]}, 6")
        em.salu(f"s_lshl_b32 {x[0]}, {self.s_ntiles}, 6")
        em.salu(f"s_min_u32 {self.s_rowlim}, {x[0]}, s20")
        # keys below kv_full are visible to every row of this wave
        em.salu(f"s_add_i32 {x[0]}, {self.s_qw0}, {self.s_off}")
        em.salu(f"s_add_i32 {x[0]}, {x[0]}, 1")
        em.salu(f"s_min_i32 {x[0]}, {x[0]}, s20")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {self.s_kvfull}, s20, {x[0]}")
        # K/V batch/head bases (bytes)
        em.salu(f"s_mul_i32 {x[0]}, {self.s_b}, s20")              # b*Skv
        em.salu(f"s_mul_i32 {x[2]}, {x[0]}, {self.s_rowb}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[0]}, {self.s_rowb}")
        em.salu(f"s_mul_i32 {x[4]}, {self.s_hk}, {D * 2}")
        em.salu(f"s_add_u32 {x[2]}, {x[2]}, {x[4]}")
        em.salu(f"s_addc_u32 {x[3]}, {x[3]}, 0")
        em.salu(f"s_add_u32 {self.s_kb.r(0)}, s10, {x[2]}")
        em.salu(f"s_addc_u32 {self.s_kb.r(1)}, s11, {x[3]}")
        em.salu(f"s_add_u32 {self.s_vb.r(0)}, s12, {x[2]}")
        em.salu(f"s_addc_u32 {self.s_vb.r(1)}, s13, {x[3]}")
        self.emit_qo_desc(self.s_rq, 8)

    def emit_qo_desc(self, rs, base):
        """Q (base s8) or O (base s14) buffer resource of the item:
        base = batch + head, records = (Sq*Hq - hq)*D*2."""
        em, D, x = self.em, self.D, self.s_x
        em.salu(f"s_mul_i32 {x[0]}, s19, s21")                     # Sq*Hq
        em.salu(f"s_mul_i32 {x[4]}, {self.s_b}, {x[0]}")           # b*Sq*Hq
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_hq}")
        em.salu(f"s_mul_i32 {x[2]}, {x[4]}, {D * 2}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[4]}, {D * 2}")
        em.salu(f"s_sub_u32 {x[5]}, {x[0]}, {self.s_hq}")
        em.salu(f"s_mul_i32 {x[5]}, {x[5]}, {D * 2}")
        em.salu(f"s_add_u32 {rs.r(0)}, s{base}, {x[2]}")
        em.salu(f"s_addc_u32 {rs.r(1)}, s{base + 1}, {x[3]}")
        em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
        em.salu(f"s_mov_b32 {rs.r(2)}, {x[5]}")
        em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")

    def item_setup_b(self):
        """The parts of an item's set-up that the previous item's epilogue
        must not see overwritten: the O and LSE buffer resources and the
        per-lane row offsets."""
        em, x = self.em, self.s_x
        self.emit_qo_desc(self.s_ro, 14)
        # LSE descriptor: base = lse + ((b*Hq + hq)*Sq)*4, records = Sq*4 (0 if no lse)
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
        self.lane_rows()

    def lane_rows(self):
        """Per-lane query rows: Q/O and LSE byte offsets, last visible key."""
        em, D = self.em, self.D
        t = self.v_t
        lane = "v0"
        # l32 = lane & 31 -> t0 ; h = lane >> 5 -> t1
        em.valu(f"v_and_b32 {t.r(0)}, 31, {lane}", dst=[t.r(0)], src=[lane])
        em.valu(f"v_lshrrev_b32 {t.r(1)}, 5, {lane}", dst=[t.r(1)], src=[lane])
        # rows of the two query blocks: q = qw0 + 32 qb + l32
        em.valu(f"v_add_u32 {t.r(2)}, {self.s_qw0}, {t.r(0)}", dst=[t.r(2)], src=[t.r(0)])
        em.valu(f"v_add_u32 {t.r(3)}, 32, {t.r(2)}", dst=[t.r(3)], src=[t.r(2)])
        em.salu(f"s_mul_i32 {self.s_x[0]}, s21, {D * 2}")   # Q/O row stride bytes
        em.salu(f"s_sub_i32 {self.s_x[1]}, s20, 1")          # Skv - 1
        for qb in range(2):
            q = t.r(2 + qb)
            # Q/O byte offset of row q (+ 16 bytes for lanes of the upper half: dims 8h..)
            em.valu(f"v_mul_lo_u32 {self.v_qoff.r(qb)}, {q}, {self.s_x[0]}", dst=[self.v_qoff.r(qb)], src=[q])
            em.valu(f"v_lshlrev_b32 {self.v_lseoff.r(qb)}, 2, {q}", dst=[self.v_lseoff.r(qb)], src=[q])
            # last visible key: causal ? min(q + off, Skv-1) : Skv-1 ; then minus 4h
            em.valu(f"v_add_u32 {t.r(4)}, {self.s_off}, {q}", dst=[t.r(4)], src=[q])
            em.valu(f"v_min_i32 {t.r(4)}, {self.s_x[1]}, {t.r(4)}", dst=[t.r(4)], src=[t.r(4)])
            em.valu(f"v_mov_b32 {t.r(5)}, {self.s_x[1]}", dst=[t.r(5)])
            em.salu("s_cmp_eq_u32 s23, 0")
            em.salu(f"s_cselect_b64 {self.s_m1}, -1, 0")
            em.valu(f"v_cndmask_b32 {t.r(4)}, {t.r(4)}, {t.r(5)}, {self.s_m1}", dst=[t.r(4)], src=[t.r(4), t.r(5)])
            em.valu(f"v_lshlrev_b32 {self.v_limh.r(qb)}, 2, {t.r(1)}", dst=[self.v_limh.r(qb)], src=[t.r(1)])
            em.valu(f"v_sub_u32 {self.v_limh.r(qb)}, {t.r(4)}, {self.v_limh.r(qb)}",
                    dst=[self.v_limh.r(qb)], src=[t.r(4), self.v_limh.r(qb)])

    def lane_dma(self):
        """Per-lane source offsets of the K/V DMA rows (with the LDS swizzles)."""
        em, D = self.em, self.D
        t = self.v_t
        lane = "v0"
        # l32 = lane & 31 -> t0 ; h = lane >> 5 -> t1
        em.valu(f"v_and_b32 {t.r(0)}, 31, {lane}", dst=[t.r(0)], src=[lane])
        em.valu(f"v_lshrrev_b32 {t.r(1)}, 5, {lane}", dst=[t.r(1)], src=[lane])
        # DMA source offsets: row r = 16w + RPD*i + lane/CH, physical chunk p = lane % CH
        CH = self.CH
        em.valu(f"v_lshrrev_b32 {t.r(2)}, {int(math.log2(CH))}, {lane}", dst=[t.r(2)], src=[lane])
        em.valu(f"v_and_b32 {t.r(3)}, {CH - 1}, {lane}", dst=[t.r(3)], src=[lane])
        em.salu(f"s_lshl_b32 {self.s_x[0]}, {self.s_w}, 4")
        em.valu(f"v_add_u32 {t.r(2)}, {self.s_x[0]}, {t.r(2)}", dst=[t.r(2)], src=[t.r(2)])  # r (i=0)
        for i in range(self.DPW):
            em.valu(f"v_add_u32 {t.r(4)}, {self.RPD * i}, {t.r(2)}", dst=[t.r(4)], src=[t.r(2)])
            em.valu(f"v_mul_lo_u32 {t.r(5)}, {t.r(4)}, {self.s_rowb}", dst=[t.r(5)], src=[t.r(4)])
            # K swizzle of row r
            if D == 128:
                em.valu(f"v_and_b32 {t.r(6)}, 15, {t.r(4)}", dst=[t.r(6)], src=[t.r(4)])
            else:
                em.valu(f"v_bfe_u32 {t.r(6)}, {t.r(4)}, 1, 3", dst=[t.r(6)], src=[t.r(4)])
            em.valu(f"v_xor_b32 {t.r(6)}, {t.r(6)}, {t.r(3)}", dst=[t.r(6)], src=[t.r(6), t.r(3)])
            em.valu(f"v_lshl_add_u32 {self.v_kdma.r(i)}, {t.r(6)}, 4, {t.r(5)}",
                    dst=[self.v_kdma.r(i)], src=[t.r(6), t.r(5)])
            # V swizzle of row r
            if D == 128:
                em.valu(f"v_and_b32 {t.r(6)}, 3, {t.r(4)}", dst=[t.r(6)], src=[t.r(4)])
            else:
                em.valu(f"v_bfe_u32 {t.r(6)}, {t.r(4)}, 1, 1", dst=[t.r(6)], src=[t.r(4)])
            em.valu(f"v_lshlrev_b32 {t.r(6)}, 2, {t.r(6)}", dst=[t.r(6)], src=[t.r(6)])
            em.valu(f"v_xor_b32 {t.r(6)}, {t.r(6)}, {t.r(3)}", dst=[t.r(6)], src=[t.r(6), t.r(3)])
            em.valu(f"v_lshl_add_u32 {self.v_vdma.r(i)}, {t.r(6)}, 4, {t.r(5)}",
                    dst=[self.v_vdma.r(i)], src=[t.r(6), t.r(5)])

    def lane_kv(self):
        """Per-lane LDS read offsets of the K and V operands."""
        em, D = self.em, self.D
        t = self.v_t
        lane = "v0"
        # l32 = lane & 31 -> t0 ; h = lane >> 5 -> t1
        em.valu(f"v_and_b32 {t.r(0)}, 31, {lane}", dst=[t.r(0)], src=[lane])
        em.valu(f"v_lshrrev_b32 {t.r(1)}, 5, {lane}", dst=[t.r(1)], src=[lane])
        # K operand offsets: KBASE + l32*ROW + (((2s+h) ^ kswz(l32)) << 4)
        if D == 128:
            em.valu(f"v_and_b32 {t.r(2)}, 15, {t.r(0)}", dst=[t.r(2)], src=[t.r(0)])
        else:
            em.valu(f"v_bfe_u32 {t.r(2)}, {t.r(0)}, 1, 3", dst=[t.r(2)], src=[t.r(0)])
        em.valu(f"v_xor_b32 {t.r(2)}, {t.r(2)}, {t.r(1)}", dst=[t.r(2)], src=[t.r(2), t.r(1)])  # sw ^ h
        em.valu(f"v_mul_u32_u24 {t.r(3)}, {self.ROW}, {t.r(0)}", dst=[t.r(3)], src=[t.r(0)])
        em.valu(f"v_add_u32 {t.r(3)}, {self.KBASE}, {t.r(3)}", dst=[t.r(3)], src=[t.r(3)])
        for s in range(self.NS):
            # ((2s) ^ (sw ^ h)) since 2s has bit 0 clear: (2s + h) ^ sw = 2s ^ (sw ^ h)
            em.valu(f"v_xor_b32 {t.r(4)}, {2 * s}, {t.r(2)}", dst=[t.r(4)], src=[t.r(2)])
            em.valu(f"v_lshl_add_u32 {self.v_koff.r(s)}, {t.r(4)}, 4, {t.r(3)}",
                    dst=[self.v_koff.r(s)], src=[t.r(4), t.r(3)])
        # V operand offsets (transposing reads): tr_i = lane & 15, tr_dh = (lane>>4)&1,
        # tr_row = 4h + (tr_i >> 2), tr_c = tr_i & 3, sw = vswz(tr_row)
        em.valu(f"v_bfe_u32 {t.r(2)}, {lane}, 2, 2", dst=[t.r(2)], src=[lane])      # tr_i >> 2
        em.valu(f"v_lshl_add_u32 {t.r(2)}, {t.r(1)}, 2, {t.r(2)}", dst=[t.r(2)], src=[t.r(1), t.r(2)])  # tr_row
        if D == 128:
            em.valu(f"v_and_b32 {t.r(3)}, 3, {t.r(2)}", dst=[t.r(3)], src=[t.r(2)])
            em.valu(f"v_lshlrev_b32 {t.r(3)}, 2, {t.r(3)}", dst=[t.r(3)], src=[t.r(3)])  # sw
        else:
            em.valu(f"v_bfe_u32 {t.r(3)}, {t.r(2)}, 1, 1", dst=[t.r(3)], src=[t.r(2)])
            em.valu(f"v_lshlrev_b32 {t.r(3)}, 2, {t.r(3)}", dst=[t.r(3)], src=[t.r(3)])
        em.valu(f"v_bfe_u32 {t.r(4)}, {lane}, 4, 1", dst=[t.r(4)], src=[lane])       # tr_dh
        em.valu(f"v_bfe_u32 {t.r(5)}, {lane}, 1, 1", dst=[t.r(5)], src=[lane])       # tr_c >> 1
        em.valu(f"v_lshl_add_u32 {t.r(4)}, {t.r(4)}, 1, {t.r(5)}", dst=[t.r(4)], src=[t.r(4), t.r(5)])  # 2dh + c>>1
        em.valu(f"v_and_b32 {t.r(5)}, 1, {lane}", dst=[t.r(5)], src=[lane])          # tr_c & 1
        em.valu(f"v_lshlrev_b32 {t.r(5)}, 3, {t.r(5)}", dst=[t.r(5)], src=[t.r(5)])  # *8
        em.valu(f"v_mad_u32_u24 {t.r(5)}, {t.r(2)}, {self.s_row}, {t.r(5)}", dst=[t.r(5)], src=[t.r(2), t.r(5)])
        for db in range(self.NDB):
            em.valu(f"v_add_u32 {t.r(6)}, {4 * db}, {t.r(4)}", dst=[t.r(6)], src=[t.r(4)])
            em.valu(f"v_xor_b32 {t.r(6)}, {t.r(6)}, {t.r(3)}", dst=[t.r(6)], src=[t.r(6), t.r(3)])
            em.valu(f"v_lshl_add_u32 {self.v_voff.r(db)}, {t.r(6)}, 4, {t.r(5)}",
                    dst=[self.v_voff.r(db)], src=[t.r(6), t.r(5)])

    # ------------------------------------------------------------------------
    # Q load into AGPRs, state init
    # ------------------------------------------------------------------------
    def load_q(self):
        """Issue the loads of the wave's 64 Q rows straight into the Q AGPRs
        (lanes of the upper half take dims 8..15 of each 16-dim step)."""
        em, t = self.em, self.v_t
        # row q = qw0 + 32 qb + l32; address q*Hq*D*2 + 16h
        em.valu(f"v_and_b32 {t.r(0)}, 31, v0", dst=[t.r(0)], src=["v0"])
        em.valu(f"v_add_u32 {t.r(0)}, {self.s_qw0}, {t.r(0)}", dst=[t.r(0)], src=[t.r(0)])
        em.salu(f"s_mul_i32 {self.s_x[0]}, s21, {self.D * 2}")
        em.valu(f"v_lshrrev_b32 {t.r(4)}, 5, v0", dst=[t.r(4)], src=["v0"])
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 4, {t.r(4)}", dst=[t.r(4)], src=[t.r(4)])
        for qb in range(2):
            if qb:
                em.valu(f"v_add_u32 {t.r(0)}, 32, {t.r(0)}", dst=[t.r(0)], src=[t.r(0)])
            em.valu(f"v_mul_lo_u32 {t.r(5 + qb)}, {t.r(0)}, {self.s_x[0]}", dst=[t.r(5 + qb)], src=[t.r(0)])
            em.valu(f"v_add_u32 {t.r(5 + qb)}, {t.r(5 + qb)}, {t.r(4)}",
                    dst=[t.r(5 + qb)], src=[t.r(5 + qb), t.r(4)])
        for qb in range(2):
            for s in range(self.NS):
                dst = str(self.a_Q[qb][s])
                em.vmem_load_to(f"buffer_load_dwordx4 {dst}, {t.r(5 + qb)}, {self.s_rq}, 0 offen offset:{32 * s}",
                                dst, src=[t.r(5 + qb)])

    def init_state(self):
        """Constants, m = -inf, l = 0, and O = 0 (by MFMAs of zero operands,
        eight instructions instead of 128 AGPR writes)."""
        em = self.em
        em.valu(f"v_mov_b32 {self.v_ninf}, {self.s_neg}", dst=[str(self.v_ninf)])
        em.valu(f"v_mov_b32 {self.v_thr}, {f32_hex(THRESH)}", dst=[str(self.v_thr)])
        em.valu(f"v_mov_b32 {self.v_c}, s24", dst=[str(self.v_c)])
        for qb in range(2):
            em.valu(f"v_mov_b32 {self.v_m.r(qb)}, {self.s_neg}", dst=[self.v_m.r(qb)])
            em.valu(f"v_mov_b32 {self.v_l.r(qb)}, 0", dst=[self.v_l.r(qb)])
            em.valu(f"v_mov_b32 {self.v_mc.r(qb)}, 0", dst=[self.v_mc.r(qb)])
        z = self.v_KO[0]
        for i in range(4):
            em.valu(f"v_mov_b32 {z.r(i)}, 0", dst=[z.r(i)])
        for qb in range(2):
            for db in range(self.NDB):
                em.mfma(self.mfma_op, str(self.a_O[qb][db]), str(z), str(z), "0")

    # ------------------------------------------------------------------------
    # K/V DMA: wave w copies rows 16w .. 16w+15 of a 64-key tile into its LDS
    # slot, RPD rows per buffer_load ... lds (16 bytes per lane).  Loads past
    # the last visible key return zeros.
    # ------------------------------------------------------------------------
    def _salu_op(self, *lines):
        em = self.em

        def f():
            for l in lines:
                em.salu(l)
        return Op(f, 0.25 * len(lines))

    def ops_dma_desc(self, tile):
        """Buffer resources s_rk / s_rv of the tile whose index is in sgpr
        `tile`: base = batch/head base + key0 * rowb, size = the bytes up to
        row_lim (0 past it).  SCC producer/consumer pairs stay in one op."""
        y, rb, sa = self.s_y, self.s_rowb, self._salu_op
        ops = [
            sa(f"s_lshl_b32 {y[0]}, {tile}, 6"),                       # key0
            sa(f"s_sub_i32 {y[1]}, {self.s_rowlim}, {y[0]}"),
            sa(f"s_max_i32 {y[1]}, {y[1]}, 0"),
            sa(f"s_mul_i32 {y[2]}, {y[1]}, {rb}"),
            sa(f"s_mul_hi_u32 {y[3]}, {y[1]}, {rb}"),
            sa(f"s_cmp_eq_u32 {y[3]}, 0", f"s_cselect_b32 {y[2]}, {y[2]}, 0x7fffffff"),
            sa(f"s_min_u32 {y[2]}, {y[2]}, 0x7fffffff"),
            sa(f"s_mul_i32 {y[3]}, {y[0]}, {rb}"),
            sa(f"s_mul_hi_u32 {y[4]}, {y[0]}, {rb}"),
        ]
        for rs, bb in ((self.s_rk, self.s_kb), (self.s_rv, self.s_vb)):
            ops += [
                sa(f"s_add_u32 {rs.r(0)}, {bb.r(0)}, {y[3]}", f"s_addc_u32 {rs.r(1)}, {bb.r(1)}, {y[4]}"),
                sa(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff"),
                sa(f"s_mov_b32 {rs.r(2)}, {y[2]}"),
                sa(f"s_mov_b32 {rs.r(3)}, 0x20000"),
            ]
        return ops

    def ops_dma_issue(self, which):
        """The wave's DPW loads of the K (or V) rows of the tile described by
        s_rk (s_rv) into the slot whose wave-adjusted address is s_kdw (s_vdw).
        M0 is set by the same op that issues the load."""
        em = self.em
        desc, slot, voff = ((self.s_rk, self.s_kdw, self.v_kdma) if which == "k"
                            else (self.s_rv, self.s_vdw, self.v_vdma))
        ops = []
        for i in range(self.DPW):
            def f(i=i):
                em.salu(f"s_add_u32 m0, {slot}, {self.RPD * i * self.ROW}")
                em.salu("s_nop 0")                 # SALU write of M0 -> LDS DMA: one wait state
                em.vmem(f"buffer_load_dwordx4 {voff.r(i)}, {desc}, 0 offen lds", src=[voff.r(i)])
            ops.append(Op(f, 0.75))
        return ops

    def wait_vm(self, n):
        self.em.salu(f"s_waitcnt vmcnt({n})")

    # ------------------------------------------------------------------------
    # building blocks: lists of Op (one instruction, or an indivisible group)
    # ------------------------------------------------------------------------
    def ops_addr(self, dst, off, n, sgpr):
        em = self.em
        return [Op(lambda i=i: em.valu(f"v_add_u32 {dst.r(i)}, {sgpr}, {off.r(i)}",
                                       dst=[dst.r(i)], src=[off.r(i)]), 1.0) for i in range(n)]

    def ops_k_loads(self, kb):
        """K operands of sub-tile kb of the tile addressed by v_kaddr."""
        em = self.em
        return [Op(lambda s=s: em.ds_read(
            f"ds_read_b128 {self.v_KO[s]}, {self.v_kaddr.r(s)} offset:{kb * 32 * self.ROW}",
            str(self.v_KO[s]), self.v_kaddr.r(s)), 0.5) for s in range(self.NS)]

    def ops_v_loads(self, kb, vb):
        """V operands of sub-tile kb of the tile addressed by v_vaddr, into VO[vb]."""
        em = self.em
        out = []
        for th in range(2):
            for db in range(self.NDB):
                for e in range(2):
                    def f(th=th, db=db, e=e):
                        off = (32 * kb + 16 * th + 8 * e) * self.ROW
                        dst = self.v_VO[vb][th][db].r(2 * e, 2)
                        em.ds_read(f"ds_read_b64_tr_b16 {dst}, {self.v_vaddr.r(db)} offset:{off}",
                                   dst, self.v_vaddr.r(db))
                    out.append(Op(f, 0.5))
        return out

    def mf_qk(self, buf):
        """S^T = K . Q^T into S[buf], query block 0 first (its result is final
        half-way through)."""
        em = self.em
        out = []
        for qb in range(2):
            for s in range(self.NS):
                def f(s=s, qb=qb):
                    d = str(self.v_S[buf][qb])
                    em.mfma(self.mfma_op, d, str(self.v_KO[s]), str(self.a_Q[qb][s]), "0" if s == 0 else d)
                out.append(f)
        return out

    def mf_pv(self, pbuf, vbuf):
        """O^T += V^T . P^T with P[pbuf] and the V operands VO[vbuf]."""
        em = self.em
        out = []
        for th in range(2):
            for db in range(self.NDB):
                for qb in range(2):
                    def f(th=th, db=db, qb=qb):
                        o = str(self.a_O[qb][db])
                        em.mfma(self.mfma_op, o, str(self.v_VO[vbuf][th][db]), str(self.v_P[pbuf][qb][th]), o)
                    out.append(f)
        return out

    def ops_softmax(self, sb, pn):
        """Softmax numerators of S[sb] against the reference max:
        E = 2^(c*S - mc) (fp32), rs = per-half row sums, P[pn] = E rounded
        to the input dtype.  Returns (exponentials, sums, conversions)."""
        em = self.em
        ops_e, ops_s, ops_c = [], [], []
        for qb in range(2):
            S, E, mc = self.v_S[sb][qb], self.v_E[qb], self.v_mc.r(qb)
            for c4 in range(4):
                for i in range(4 * c4, 4 * c4 + 4):
                    ops_e.append(Op(lambda S=S, E=E, mc=mc, i=i: em.valu(
                        f"v_fma_f32 {E.r(i)}, {S.r(i)}, s24, -{mc}", dst=[E.r(i)], src=[S.r(i), mc]), 1.0))
                for i in range(4 * c4, 4 * c4 + 4):
                    ops_e.append(Op(lambda E=E, i=i: em.valu(
                        f"v_exp_f32 {E.r(i)}, {E.r(i)}", dst=[E.r(i)], src=[E.r(i)], trans=True), 1.5))
            ra, rb = self.v_rs.r(qb), self.v_rb.r(qb)
            ops_s.append(Op(lambda E=E, ra=ra: em.valu(f"v_add_f32 {ra}, {E.r(0)}, {E.r(1)}", dst=[ra], src=[E.r(0), E.r(1)]), 1.0))
            ops_s.append(Op(lambda E=E, rb=rb: em.valu(f"v_add_f32 {rb}, {E.r(2)}, {E.r(3)}", dst=[rb], src=[E.r(2), E.r(3)]), 1.0))
            for i in range(4, 16):
                acc = ra if i % 2 == 0 else rb
                ops_s.append(Op(lambda E=E, acc=acc, i=i: em.valu(
                    f"v_add_f32 {acc}, {acc}, {E.r(i)}", dst=[acc], src=[acc, E.r(i)]), 1.0))
            ops_s.append(Op(lambda ra=ra, rb=rb: em.valu(f"v_add_f32 {ra}, {ra}, {rb}", dst=[ra], src=[ra, rb]), 1.0))
            for th in range(2):
                P = self.v_P[pn][qb][th]
                for jj in range(4):
                    lo, hi = E.r(8 * th + 2 * jj), E.r(8 * th + 2 * jj + 1)
                    ops_c.append(Op(lambda P=P, jj=jj, lo=lo, hi=hi: em.valu(
                        f"{self.cvt_op} {P.r(jj)}, {lo}, {hi}", dst=[P.r(jj)], src=[lo, hi]), 1.0))
        return ops_e, ops_s, ops_c

    def ops_test(self):
        """s_m1 / s_m2: lanes whose half-row sum passed the trigger (some p of
        the sub-tile is above it, so the reference max must move)."""
        em = self.em
        return [Op(lambda qb=qb, msk=msk: em.valu(
            f"v_cmp_gt_f32 {msk}, {self.v_rs.r(qb)}, {self.v_thr}", src=[self.v_rs.r(qb), str(self.v_thr)]), 1.0)
            for qb, msk in ((0, self.s_m1), (1, self.s_m2))]

    def ops_mask(self, sb):
        """Set S[sb] entries of keys past each row's last visible key to -inf.
        Key of register i = k0 + 8*(i>>2) + 4h + (i&3); limh = lim - 4h."""
        em = self.em
        out = []
        for qb in range(2):
            S = self.v_S[sb][qb]
            d = self.v_d.r(qb)
            out.append(lambda d=d, qb=qb: em.valu(f"v_subrev_u32 {d}, {self.s_k0}, {self.v_limh.r(qb)}",
                                                  dst=[d], src=[self.v_limh.r(qb)]))
            for i in range(16):
                ci = 8 * (i >> 2) + (i & 3)
                out.append(lambda d=d, ci=ci: em.valu(f"v_cmp_lt_i32 vcc, {d}, {ci}", src=[d]))
                out.append(lambda S=S, i=i: em.valu(f"v_cndmask_b32 {S.r(i)}, {S.r(i)}, {self.v_ninf}, vcc",
                                                    dst=[S.r(i)], src=[S.r(i), str(self.v_ninf)]))
        return out

    def ops_rowmax(self, sb, qb):
        """Row max of S[sb][qb] over both lane halves into v_mx[qb]."""
        em = self.em
        S, mx, tmp = self.v_S[sb][qb], self.v_mx.r(qb), self.v_t.r(6 + qb)
        out = [lambda: em.valu(f"v_max3_f32 {mx}, {S.r(0)}, {S.r(1)}, {S.r(2)}", dst=[mx], src=[S.r(0), S.r(1), S.r(2)])]
        for i in range(3, 15, 2):
            out.append(lambda i=i: em.valu(f"v_max3_f32 {mx}, {mx}, {S.r(i)}, {S.r(i + 1)}",
                                           dst=[mx], src=[mx, S.r(i), S.r(i + 1)]))
        out.append(lambda: em.valu(f"v_max_f32 {mx}, {mx}, {S.r(15)}", dst=[mx], src=[mx, S.r(15)]))
        out.append(lambda: em.valu(f"v_mov_b32 {tmp}, {mx}", dst=[tmp], src=[mx]))
        out.append(lambda: em.valu(f"v_permlane32_swap_b32 {mx}, {tmp}", dst=[mx, tmp], src=[mx, tmp]))
        out.append(lambda: em.valu(f"v_max_f32 {mx}, {mx}, {tmp}", dst=[mx], src=[mx, tmp]))
        return out

    def emit_all(self, ops):
        for f in ops:
            f()

    def emit_set_mc(self, qb):
        """mc = c*m, or 0 while m = -inf (so masked logits stay -inf)."""
        em = self.em
        m, mc = self.v_m.r(qb), self.v_mc.r(qb)
        em.valu(f"v_mul_f32 {mc}, s24, {m}", dst=[mc], src=[m])
        em.valu(f"v_cmp_eq_f32 vcc, {self.s_neg}, {m}", src=[m])
        em.valu(f"v_cndmask_b32 {mc}, {mc}, 0, vcc", dst=[mc], src=[mc])

    def emit_rescale(self, sb, pn):
        """Slow path: move the reference max of every row to max(m, rowmax of
        S[sb]), rescale O and l by alpha = 2^(c*m_old - c*m_new), then redo the
        softmax numerators of S[sb] and add their sums to l."""
        em, t = self.em, self.v_t
        em.drain()
        for qb in range(2):
            self.emit_all(self.ops_rowmax(sb, qb))
            m, mx, l = self.v_m.r(qb), self.v_mx.r(qb), self.v_l.r(qb)
            mn, a, b = t.r(0), t.r(1), t.r(2)
            em.valu(f"v_max_f32 {mn}, {m}, {mx}", dst=[mn], src=[m, mx])
            em.valu(f"v_mul_f32 {a}, s24, {m}", dst=[a], src=[m])
            em.valu(f"v_mul_f32 {b}, s24, {mn}", dst=[b], src=[mn])
            em.valu(f"v_sub_f32 {a}, {a}, {b}", dst=[a], src=[a, b])
            em.valu(f"v_exp_f32 {a}, {a}", dst=[a], src=[a], trans=True)
            em.valu(f"v_cmp_eq_f32 vcc, {self.s_neg}, {mn}", src=[mn])
            em.valu(f"v_cndmask_b32 {a}, {a}, 1.0, vcc", dst=[a], src=[a])   # alpha = 1 while all -inf
            em.valu(f"v_mov_b32 {m}, {mn}", dst=[m], src=[mn])
            self.emit_set_mc(qb)
            em.valu(f"v_mul_f32 {l}, {l}, {a}", dst=[l], src=[l, a])
            for db in range(self.NDB):
                blk = self.a_O[qb][db]
                for i in range(16):
                    tmp = t.r(5 + (i & 1))
                    em.valu(f"v_accvgpr_read_b32 {tmp}, {blk.r(i)}", dst=[tmp], src=[blk.r(i)])
                    em.valu(f"v_mul_f32 {tmp}, {tmp}, {a}", dst=[tmp], src=[tmp, a])
                    em.valu(f"v_accvgpr_write_b32 {blk.r(i)}, {tmp}", dst=[blk.r(i)], src=[tmp])
        e, s_, c = self.ops_softmax(sb, pn)
        self.emit_all(e + s_ + c)
        self.emit_l_update()
        em.drain()

    def emit_l_update(self):
        em = self.em
        for qb in range(2):
            l, rs = self.v_l.r(qb), self.v_rs.r(qb)
            em.valu(f"v_add_f32 {l}, {l}, {rs}", dst=[l], src=[l, rs])

    # ------------------------------------------------------------------------
    # One pipeline step j (j_par = j % 2):
    #   MFMA: P.V(j) [P[j%2], VO[j%2]] and, for kind "full", S^T(j+2) into
    #         S[j%2] (K operands loaded in this step);
    #   other units: the softmax numerators of sub-tile j+1 [S[(j+1)%2] ->
    #         P[(j+1)%2]], the V operands of sub-tile j+1 [-> VO[(j+1)%2]] and
    #         the caller's extra ops (addresses, DMA).
    # The sub-tile is masked first when it holds keys past some row's last
    # visible key (an out-of-line copy of the step); when a half-row sum
    # passes the trigger an out-of-line slow path moves the reference max.
    # ------------------------------------------------------------------------
    def step(self, jp, kind, kb_k=0, kb_v=0, pre=(), extra=()):
        em = self.em
        sb = pn = vn = 1 - jp

        def build():
            mf = self.mf_pv(jp, jp)
            if kind == "pvonly":
                return mf, list(pre) + list(extra)
            others = list(pre)
            if kind == "full":
                mf += self.mf_qk(jp)
                others += self.ops_k_loads(kb_k)
            e, s_, c = self.ops_softmax(sb, pn)
            vl = self.ops_v_loads(kb_v, vn)
            ex = list(extra)
            # exponentials first; V operand loads and extras spread through
            # the middle; sums, conversions and the trigger test last
            half = len(e) // 2
            others += e[:half] + vl[:len(vl) // 2] + ex[:len(ex) // 2] + e[half:] \
                + vl[len(vl) // 2:] + ex[len(ex) // 2:] + s_ + self.ops_test() + c
            return mf, others

        if kind == "pvonly":
            mf, others = build()
            weave(em, mf, others)
            return
        # masked copy out of line when sub-tile j+1 reaches past kv_full
        l_mask, l_join = self.lab("mask"), self.lab("join")
        em.salu(f"s_add_u32 {self.s_x[0]}, {self.s_k0}, 32")
        em.salu(f"s_cmp_gt_i32 {self.s_x[0]}, {self.s_kvfull}")
        em.salu(f"s_cbranch_scc1 {l_mask}")
        snap = em.snapshot()
        mf, others = build()
        weave(em, mf, others)
        em.label(l_join)
        self.deferred.append(("mask", snap, l_mask, l_join, sb, build))
        # trigger test -> slow path
        l_slow, l_back = self.lab("slow"), self.lab("back")
        em.salu(f"s_or_b64 {self.s_or}, {self.s_m1}, {self.s_m2}")
        em.salu(f"s_cbranch_scc1 {l_slow}")
        snap2 = em.snapshot()
        self.emit_l_update()
        em.label(l_back)
        self.deferred.append(("slow", snap2, l_slow, l_back, sb, pn))

    def emit_deferred(self):
        em = self.em
        for item in self.deferred:
            if item[0] == "mask":
                _, snap, l_mask, l_join, sb, build = item
                em.restore(snap)
                em.label(l_mask)
                self.emit_all(self.ops_mask(sb))
                mf, others = build()
                weave(em, mf, others)
                em.drain()
                em.salu(f"s_branch {l_join}")
            else:
                _, snap, l_slow, l_back, sb, pn = item
                em.restore(snap)
                em.label(l_slow)
                self.emit_rescale(sb, pn)
                em.salu(f"s_branch {l_back}")

    def epilogue(self):
        em, t = self.em, self.v_t
        # (the next item's Q and K/V loads may be in flight: the epilogue reads
        # none of the registers or LDS they write)
        em.drain()
        # Lane (l, h) holds dims 32db + 8j + 4h .. +3 of row l%32 in O^T block
        # registers 4j .. 4j+3.  For each pair j = 2jp, 2jp+1, one
        # v_permlane32_swap per packed dword gives lanes < 32 dims 8(2jp) .. +7
        # and lanes >= 32 dims 8(2jp+1) .. +7: 16 contiguous bytes per lane,
        # stored at qoff + 16h + 64db + 32jp.  The E buffers are free here; four
        # rotating output sets keep each store's data untouched after it issues.
        em.valu(f"v_lshrrev_b32 {t.r(0)}, 5, v0", dst=[t.r(0)], src=["v0"])      # h
        em.valu(f"v_lshlrev_b32 {t.r(7)}, 4, {t.r(0)}", dst=[t.r(7)], src=[t.r(0)])  # 16h
        E = self.v_E
        for qb in range(2):
            l = self.v_l.r(qb)
            em.valu(f"v_mov_b32 {t.r(0)}, {l}", dst=[t.r(0)], src=[l])
            em.valu(f"v_permlane32_swap_b32 {l}, {t.r(0)}", dst=[l, t.r(0)], src=[l, t.r(0)])
            em.valu(f"v_add_f32 {l}, {l}, {t.r(0)}", dst=[l], src=[l, t.r(0)])
            em.valu(f"v_rcp_f32 {t.r(1)}, {l}", dst=[t.r(1)], src=[l], trans=True)
            em.valu(f"v_cmp_lt_f32 vcc, 0, {l}", src=[l])
            em.valu(f"v_cndmask_b32 {t.r(1)}, 0, {t.r(1)}, vcc", dst=[t.r(1)], src=[t.r(1)])
            em.valu(f"v_add_u32 {t.r(2)}, {self.v_qoff.r(qb)}, {t.r(7)}", dst=[t.r(2)],
                    src=[self.v_qoff.r(qb), t.r(7)])
            for db in range(self.NDB):
                blk = self.a_O[qb][db]
                for jp in range(2):
                    k = 2 * db + jp
                    F, o = E[k % 2], 8 + 4 * ((k // 2) % 2)
                    for jj in range(2):
                        j = 2 * jp + jj
                        for r in range(4):
                            dst = F.r(4 * jj + r)
                            em.valu(f"v_accvgpr_read_b32 {dst}, {blk.r(4 * j + r)}", dst=[dst],
                                    src=[blk.r(4 * j + r)])
                            em.valu(f"v_mul_f32 {dst}, {dst}, {t.r(1)}", dst=[dst], src=[dst, t.r(1)])
                        for c in range(2):
                            a, b = F.r(4 * jj + 2 * c), F.r(4 * jj + 2 * c + 1)
                            em.valu(f"{self.cvt_op} {F.r(o + 2 * jj + c)}, {a}, {b}",
                                    dst=[F.r(o + 2 * jj + c)], src=[a, b])
                    for c in range(2):
                        x, y = F.r(o + c), F.r(o + 2 + c)
                        em.valu(f"v_permlane32_swap_b32 {x}, {y}", dst=[x, y], src=[x, y])
                    em.vmem(f"buffer_store_dwordx4 {F.r(o, 4)}, {t.r(2)}, {self.s_ro}, 0 offen "
                            f"offset:{64 * db + 32 * jp}", src=[F.r(o, 4), t.r(2)])
            # LSE = ln2 * (mc + log2 l), -inf when l = 0 (vcc still holds l > 0)
            em.valu(f"v_log_f32 {t.r(3)}, {l}", dst=[t.r(3)], src=[l], trans=True)
            em.valu(f"v_add_f32 {t.r(3)}, {self.v_mc.r(qb)}, {t.r(3)}", dst=[t.r(3)], src=[self.v_mc.r(qb), t.r(3)])
            em.valu(f"v_mul_f32 {t.r(3)}, {f32_hex(LN2)}, {t.r(3)}", dst=[t.r(3)], src=[t.r(3)])
            em.valu(f"v_cndmask_b32 {t.r(3)}, {self.v_ninf}, {t.r(3)}, vcc", dst=[t.r(3)],
                    src=[t.r(3), str(self.v_ninf)])
            em.vmem(f"buffer_store_dword {t.r(3)}, {self.v_lseoff.r(qb)}, {self.s_rl}, 0 offen",
                    src=[t.r(3), self.v_lseoff.r(qb)])

    # ------------------------------------------------------------------------
    def body(self):
        em = self.em
        self.alloc()
        self.kernel_setup()
        self.deferred = []
        y = self.s_y
        T, DPW = self.TILE, self.DPW
        self.lane_dma()
        self.lane_kv()
        # ---- items (batch, q-head, q-tile), one per pass.  The next item's Q and
        # first K/V tiles are requested before the current item's epilogue, so
        # their latency is spent storing O.
        l_exit, l_body, l_final = self.lab("exit"), self.lab("body"), self.lab("final")
        em.drain()
        self.item_setup_a(l_exit)
        self.issue_item_loads()
        em.drain()
        em.label(l_body)
        self.item_setup_b()
        self.init_state()
        em.salu("s_waitcnt vmcnt(0)")      # Q, the first tiles, the previous item's stores
        em.salu("s_barrier")
        l_empty = self.lab("empty")
        em.salu(f"s_cmp_eq_u32 {self.s_ntiles}, 0")
        em.salu(f"s_cbranch_scc1 {l_empty}")
        # ---- sub-tile 0: S^T(0); its row max sets m; S^T(1) next to softmax(0) ----
        self.emit_all(self.ops_addr(self.v_kaddr, self.v_koff, self.NS, 0))
        self.emit_all(self.ops_k_loads(0))
        self.emit_all(self.mf_qk(0))
        self.emit_all(self.ops_k_loads(1))
        em.salu(f"s_mov_b32 {self.s_k0}, 0")
        l_skip = self.lab("nomask0")
        em.salu(f"s_cmp_gt_i32 32, {self.s_kvfull}")
        em.salu(f"s_cbranch_scc0 {l_skip}")
        snap = em.snapshot()
        self.emit_all(self.ops_mask(0))
        em.label(l_skip)
        em.restore(snap)
        for qb in range(2):
            self.emit_all(self.ops_rowmax(0, qb))
            m, mx = self.v_m.r(qb), self.v_mx.r(qb)
            em.valu(f"v_mov_b32 {m}, {mx}", dst=[m], src=[mx])
            self.emit_set_mc(qb)
        self.emit_all(self.ops_addr(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl0))
        e, s_, c = self.ops_softmax(0, 0)
        weave(em, self.mf_qk(1), e + self.ops_v_loads(0, 0) + s_ + c)
        self.emit_l_update()
        # (tiles 0 .. PREFETCH-1 are resident: waited for at the item start)
        em.salu(f"s_mov_b32 {self.s_k0}, 32")
        em.salu(f"s_mov_b32 {self.s_t}, 0")
        em.salu(f"s_sub_u32 {self.s_tlast}, {self.s_ntiles}, 1")
        l_last, l_loop = self.lab("last"), self.lab("loop")
        rel_pre = em.rel_state()
        em.salu(f"s_cmp_eq_u32 {self.s_tlast}, 0")
        em.salu(f"s_cbranch_scc1 {l_last}")
        # ---- main loop over tiles t = 0 .. n_tiles-2.  The body is emitted from
        # the merge of the entry state and its own back-edge state (re-emitted
        # until that merge is a fixed point), so no drain is needed at the edge.
        em.label(l_loop)
        mark = (len(em.lines), self._lab, len(self.deferred))
        rel_in = rel_pre
        for _ in range(4):
            em.apply_rel(rel_in)
            self.emit_iteration()
            merged = Emitter.merge_rel(rel_pre, em.rel_state())
            if merged == rel_in:
                break
            del em.lines[mark[0]:]
            self._lab = mark[1]
            del self.deferred[mark[2]:]
            rel_in = merged
        else:
            raise RuntimeError("loop hazard state did not converge")
        em.salu(f"s_cbranch_scc1 {l_loop}")
        rel_exit = em.rel_state()
        # ---- last tile: P.V(2n-2) next to softmax(2n-1), then P.V(2n-1) ------------
        em.label(l_last)
        em.apply_rel(Emitter.merge_rel(rel_exit, rel_pre))
        self.step(0, "noqk", kb_v=1, pre=self.ops_addr(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl0))
        self.step(1, "pvonly")
        em.label(l_empty)
        em.drain()
        # every wave is done with this item's LDS before the next item fills it
        em.salu("s_barrier")
        em.salu(f"s_add_u32 {self.s_r}, {self.s_r}, 1")
        self.item_setup_a(l_final)
        self.issue_item_loads()
        self.epilogue()                     # the finished item's O and LSE
        em.drain()
        em.salu(f"s_branch {l_body}")
        em.label(l_final)
        self.epilogue()
        em.label(l_exit)
        # nothing may be in flight when the wave ends and its registers and
        # LDS are reused by another workgroup
        em.salu("s_waitcnt vmcnt(0)")
        em.salu("s_endpgm")
        self.emit_deferred()

    def issue_item_loads(self):
        """Q of the item (into the Q AGPRs) and its first PREFETCH K/V tiles,
        with the ring slots set for the first tile iteration."""
        em, y = self.em, self.s_y
        T = self.TILE
        self.load_q()
        for tt in range(PREFETCH):
            em.salu(f"s_mov_b32 {y[5]}, {tt}")
            em.salu(f"s_add_u32 {self.s_kdw}, {self.s_wrow}, {self.KBASE + (tt % KSLOTS) * T}")
            em.salu(f"s_add_u32 {self.s_vdw}, {self.s_wrow}, {self.VBASE + (tt % VSLOTS) * T}")
            self.emit_all(self.ops_dma_desc(y[5]) + self.ops_dma_issue("k") + self.ops_dma_issue("v"))
        # ring slots for iteration t = 0: K read tile 1, DMA tile PREFETCH; V tiles 0, 1
        em.salu(f"s_mov_b32 {self.s_ksl}, {T}")
        em.salu(f"s_mov_b32 {self.s_kdsl}, {(PREFETCH % KSLOTS) * T}")
        em.salu(f"s_mov_b32 {self.s_vsl0}, 0")
        em.salu(f"s_mov_b32 {self.s_vsl1}, {T}")
        em.salu(f"s_mov_b32 {self.s_vdsl}, {(PREFETCH % VSLOTS) * T}")
        em.salu(f"s_add_u32 {self.s_kdw}, {self.s_wrow}, {self.KBASE + (PREFETCH % KSLOTS) * T}")
        em.salu(f"s_add_u32 {self.s_vdw}, {self.s_wrow}, {(PREFETCH % VSLOTS) * T}")

    def emit_iteration(self):
        """Tile t: steps j = 2t and 2t+1, then the ring hand-over."""
        em, x, y = self.em, self.s_x, self.s_y
        T, DPW = self.TILE, self.DPW
        # step 2t: K operands of tile t+1 (sub-tile 0), V operands of tile t
        # (sub-tile 1); DMA of tile t+PREFETCH: its descriptors and K rows
        pre = (self.ops_addr(self.v_kaddr, self.v_koff, self.NS, self.s_ksl)
               + self.ops_addr(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl0))
        dma_k = ([self._salu_op(f"s_add_u32 {y[5]}, {self.s_t}, {PREFETCH}")]
                 + self.ops_dma_desc(y[5]) + self.ops_dma_issue("k"))
        self.step(0, "full", kb_k=0, kb_v=1, pre=pre, extra=dma_k)
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        # step 2t+1: K operands of tile t+1 (sub-tile 1), V operands of tile t+1
        # (sub-tile 0); V rows of tile t+PREFETCH
        self.step(1, "full", kb_k=1, kb_v=0,
                  pre=self.ops_addr(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl1),
                  extra=self.ops_dma_issue("v"))
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        # tile t+2 resident for the next tile; the slots read here become free
        self.wait_vm(2 * 2 * DPW)
        em.salu("s_barrier")
        em.salu(f"s_add_u32 {self.s_ksl}, {self.s_ksl}, {T}")
        em.salu(f"s_and_b32 {self.s_ksl}, {self.s_ksl}, {KSLOTS * T - 1}")
        em.salu(f"s_add_u32 {self.s_kdsl}, {self.s_kdsl}, {T}")
        em.salu(f"s_and_b32 {self.s_kdsl}, {self.s_kdsl}, {KSLOTS * T - 1}")
        em.salu(f"s_mov_b32 {self.s_vsl0}, {self.s_vsl1}")
        for r in (self.s_vsl1, self.s_vdsl):
            em.salu(f"s_add_u32 {r}, {r}, {T}")
            em.salu(f"s_sub_u32 {x[1]}, {r}, {VSLOTS * T}")
            em.salu(f"s_cselect_b32 {r}, {r}, {x[1]}")
        em.salu(f"s_add_u32 {self.s_kdw}, {self.s_kdsl}, {self.s_wrow}")
        em.salu(f"s_add_u32 {self.s_kdw}, {self.s_kdw}, {self.KBASE}")
        em.salu(f"s_add_u32 {self.s_vdw}, {self.s_vdsl}, {self.s_wrow}")
        em.salu(f"s_add_u32 {self.s_t}, {self.s_t}, 1")
        em.salu(f"s_cmp_lt_u32 {self.s_t}, {self.s_tlast}")

    # ------------------------------------------------------------------------
    def assemble_text(self) -> str:
        self.body()
        name = self.name
        nv, na = self.nvgpr, self.nagpr
        total = nv + na
        out = []
        out.append('\t.amdgcn_target "amdgcn-amd-amdhsa--gfx950"')
        out.append("\t.amdhsa_code_object_version 6")
        out.append("\t.text")
        out.append(f"\t.globl {name}")
        out.append("\t.p2align 8")
        out.append(f"\t.type {name},@function")
        out.append(f"{name}:")
        out.append(self.em.text())
        out.append(f"\t.size {name}, .-{name}")
        out.append("\t.rodata")
        out.append("\t.p2align 6")
        out.append(f"\t.amdhsa_kernel {name}")
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
        return "\n".join(out) + "\n", dict(name=name, nv=nv, na=na, total=total, lds=self.LDS, ns=self.nsgpr + 2)


def metadata(kernels) -> str:
    lines = ["\t.amdgpu_metadata", "---", "amdhsa.kernels:"]
    for k in kernels:
        lines += [
            f"  - .agpr_count: {k['na']}",
            "    .args:",
        ]
        # pointer arguments (offset, access), then 4-byte values up to the end
        ptrs = k.get("ptrs", [(0, "read_only"), (8, "read_only"), (16, "read_only"),
                              (24, "write_only"), (32, "write_only")])
        size = k.get("kernarg", KERNARG_BYTES)
        for off, access in ptrs:
            lines += [f"      - .actual_access: {access}", "        .address_space: global",
                      f"        .offset: {off}", "        .size: 8", "        .value_kind: global_buffer"]
        for off in range(ptrs[-1][0] + 8, size, 4):
            lines += [f"      - .offset: {off}", "        .size: 4", "        .value_kind: by_value"]
        lines += [
            f"    .group_segment_fixed_size: {k['lds']}",
            "    .kernarg_segment_align: 8",
            f"    .kernarg_segment_size: {size}",
            f"    .max_flat_workgroup_size: {k.get('wg', 256)}",
            f"    .name: {k['name']}",
            "    .private_segment_fixed_size: 0",
            f"    .sgpr_count: {k['ns']}",
            "    .sgpr_spill_count: 0",
            f"    .symbol: {k['name']}.kd",
            "    .uniform_work_group_size: 1",
            "    .uses_dynamic_stack: false",
            f"    .vgpr_count: {k['total']}",
            "    .vgpr_spill_count: 0",
            "    .wavefront_size: 64",
        ]
    lines += ["amdhsa.target: amdgcn-amd-amdhsa--gfx950", "amdhsa.version:", "  - 1", "  - 2",
              "...", "\t.end_amdgpu_metadata"]
    return "\n".join(lines) + "\n"


VARIANTS = [("bf16", 128), ("bf16", 64), ("f16", 128), ("f16", 64)]


def generate_all() -> str:
    """Every kernel of the library: the four-wave variants, then the
    eight-wave D = 128 variants (fa_fwd_x8), whole key ranges and split,
    the eight-wave D = 64 variants on whole key ranges, and the backward's
    dK/dV and dQ kernels (fa_bwd_gen)."""
    from .fa_fwd_x8 import Gen8
    texts, metas = [], []
    for dt, D in VARIANTS:
        g = Gen(dt, D)
        txt, info = g.assemble_text()
        texts.append(txt)
        metas.append(info)
    for split in (False, True):
        for dt in ("bf16", "f16"):
            txt, info = Gen8(dt, split).assemble_text()
            texts.append(txt)
            metas.append(info)
    for dt in ("bf16", "f16"):
        txt, info = Gen8(dt, False, 64).assemble_text()
        texts.append(txt)
        metas.append(info)
    from .fa_bwd_gen import GenBwd, VARIANTS as BWD_VARIANTS
    for kind, dt, D in BWD_VARIANTS:
        txt, info = GenBwd(kind, dt, D).assemble_text()
        texts.append(txt)
        metas.append(info)
    return "".join(texts) + metadata(metas)


if __name__ == "__main__":
    import sys
    out = sys.argv[1] if len(sys.argv) > 1 else "fa_fwd_gfx950.s"
    with open(out, "w") as f:
        f.write(generate_all())
    print(out)
