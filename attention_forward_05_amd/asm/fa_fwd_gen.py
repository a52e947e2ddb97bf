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

from .regs import Alloc, Emitter, interleave

BM = 256          # query rows per workgroup
BN = 64           # keys per tile
WAVES = 4
RESCALE = 8.0     # lazy-rescale threshold (exp2 units)
KERNARG_BYTES = 80
LN2 = 0.6931471805599453

# kernarg offsets
KA = dict(q=0, k=8, v=16, o=24, lse=32, B=40, Sq=44, Skv=48, Hq=52, Hkv=56,
          causal=60, c=64, nq=68, gmagic=72, hq_xcd=76)


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
        self.VSLOTS, self.KSLOTS = 4, 3
        self.VBASE = 0
        self.KBASE = self.VSLOTS * self.TILE
        self.LDS = (self.VSLOTS + self.KSLOTS) * self.TILE
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
        V = Alloc("v", 0, 256)
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
        r["v_rs"] = V.take("rs", 2)
        r["v_d"] = V.take("dmask", 2)
        r["v_ninf"] = V.take("ninf", 1)       # -inf
        r["v_resc"] = V.take("resc", 1)       # lazy-rescale threshold
        r["v_c"] = V.take("c", 1)             # scale * log2(e)
        # S double buffer: S[buf][qb] 16 regs each
        r["v_S"] = [[V.take(f"S{b}{q}", 16, 4) for q in range(2)] for b in range(2)]
        # P double buffer: P[buf][qb][th] 4 regs each
        r["v_P"] = [[[V.take(f"P{b}{q}{t}", 4, 4) for t in range(2)] for q in range(2)]
                    for b in range(2)]
        r["v_KO"] = [V.take(f"KO{s}", 4, 4) for s in range(NS)]
        r["v_VO"] = [[V.take(f"VO{t}{d}", 4, 4) for d in range(NDB)] for t in range(2)]
        self.nvgpr = (V.next + 7) // 8 * 8
        # AGPRs: O^T accumulators and Q
        r["a_O"] = [[A.take(f"O{q}{d}", 16, 4) for d in range(NDB)] for q in range(2)]
        r["a_Q"] = [[A.take(f"Q{q}{s}", 4, 4) for s in range(NS)] for q in range(2)]
        self.nagpr = (A.next + 7) // 8 * 8
        # SGPRs (s0:1 kernarg ptr, s2..s4 workgroup ids, s8..s27 kernargs)
        t = S.take
        r["s_hq"], r["s_qt"], r["s_b"], r["s_hk"] = t("hq", 1), t("qt", 1), t("b", 1), t("hk", 1)
        r["s_w"], r["s_qw0"], r["s_off"], r["s_ntiles"] = t("w", 1), t("qw0", 1), t("off", 1), t("nt", 1)
        r["s_kvfull"], r["s_rowlim"], r["s_rowb"], r["s_t"] = t("kvf", 1), t("rowlim", 1), t("rowb", 1), t("t", 1)
        r["s_rq"] = t("rq", 4, 4)
        r["s_ro"] = t("ro", 4, 4)
        r["s_rl"] = t("rl", 4, 4)
        r["s_rk"] = t("rk", 4, 4)
        r["s_rv"] = t("rv", 4, 4)
        r["s_kb"] = t("kbase", 2, 2)
        r["s_vb"] = t("vbase", 2, 2)
        r["s_ksl"], r["s_kdsl"] = t("ksl", 1), t("kdsl", 1)   # K slot read (t+1), K slot DMA (t+3)
        r["s_vsl0"], r["s_vsl1"], r["s_vdsl"] = t("vsl0", 1), t("vsl1", 1), t("vdsl", 1)
        r["s_k0"] = t("k0", 1)
        r["s_x"] = [t(f"x{i}", 1) for i in range(6)]
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
    def prologue(self):
        em, D = self.em, self.D
        x = self.s_x
        em.comment("kernel arguments")
        em.salu("s_load_dwordx16 s[8:23], s[0:1], 0x0")
        em.salu("s_load_dwordx4 s[24:27], s[0:1], 0x40")
        # wave index: v0 (the work-item id, written at wave launch) >> 6
        em.valu(f"v_readfirstlane_b32 {self.s_w}, v0", src=["v0"])
        em.salu(f"s_lshr_b32 {self.s_w}, {self.s_w}, 6")
        em.valu("v_and_b32 v0, 63, v0", dst=["v0"], src=["v0"])  # lane
        em.salu("s_waitcnt lgkmcnt(0)")
        em.salu(f"s_mov_b32 {self.s_neg}, 0xff800000")
        em.salu(f"s_mov_b32 {self.s_row}, {self.ROW}")
        # hq: spread contiguous head groups over the 8 XCDs (workgroup x -> XCD x % 8)
        l_no, l_done = self.lab("noxcd"), self.lab("xcd")
        em.salu("s_cmp_eq_u32 s27, 0")
        em.salu(f"s_cbranch_scc1 {l_no}")
        em.salu(f"s_and_b32 {self.s_hq}, s2, 7")
        em.salu(f"s_mul_i32 {self.s_hq}, {self.s_hq}, s27")
        em.salu(f"s_lshr_b32 {x[0]}, s2, 3")
        em.salu(f"s_add_u32 {self.s_hq}, {self.s_hq}, {x[0]}")
        em.salu(f"s_branch {l_done}")
        em.label(l_no)
        em.salu(f"s_mov_b32 {self.s_hq}, s2")
        em.label(l_done)
        # query tile: longest causal tiles first
        em.salu(f"s_sub_u32 {x[0]}, s25, 1")
        em.salu(f"s_sub_u32 {x[0]}, {x[0]}, s3")
        em.salu("s_cmp_eq_u32 s23, 0")
        em.salu(f"s_cselect_b32 {self.s_qt}, s3, {x[0]}")
        em.salu(f"s_mov_b32 {self.s_b}, s4")
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
        # K/V row stride and batch/head bases (bytes)
        em.salu(f"s_mul_i32 {self.s_rowb}, s22, {D * 2}")
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
        # Q / O descriptors: base = batch + head, records = (Sq*Hq - hq)*D*2
        em.salu(f"s_mul_i32 {x[0]}, s19, s21")                     # Sq*Hq
        em.salu(f"s_mul_i32 {x[4]}, {self.s_b}, {x[0]}")           # b*Sq*Hq
        em.salu(f"s_add_u32 {x[4]}, {x[4]}, {self.s_hq}")
        em.salu(f"s_mul_i32 {x[2]}, {x[4]}, {D * 2}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[4]}, {D * 2}")
        em.salu(f"s_sub_u32 {x[5]}, {x[0]}, {self.s_hq}")
        em.salu(f"s_mul_i32 {x[5]}, {x[5]}, {D * 2}")
        for rs, base in ((self.s_rq, 8), (self.s_ro, 14)):
            em.salu(f"s_add_u32 {rs.r(0)}, s{base}, {x[2]}")
            em.salu(f"s_addc_u32 {rs.r(1)}, s{base + 1}, {x[3]}")
            em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
            em.salu(f"s_mov_b32 {rs.r(2)}, {x[5]}")
            em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")
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
        em.salu("s_or_b32 s16, s16, s17")
        em.salu("s_cmp_eq_u32 s16, 0")
        em.salu(f"s_cselect_b32 {self.s_rl.r(2)}, 0, {self.s_rl.r(2)}")

    def lane_constants(self):
        em, D = self.em, self.D
        if self.debug_point == "start":
            vals = ["v0"]
            for i, sg in enumerate(["s32", "s19", "s21", "s14", "s15", "s44", "s45", "s46", "s47", "s2", "s3", "s4"]):
                em.valu(f"v_mov_b32 v{100 + i}, {sg}", dst=[f"v{100 + i}"])
                vals.append(f"v{100 + i}")
            self.debug_dump("start", vals)
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
        # Q byte offsets also include 16 h (dims 8h .. 8h+7 of each 16-dim step)
        em.valu(f"v_lshlrev_b32 {t.r(4)}, 4, {t.r(1)}", dst=[t.r(4)], src=[t.r(1)])
        self.v_h16 = t.r(4)

    # ------------------------------------------------------------------------
    # Q load into AGPRs, state init
    # ------------------------------------------------------------------------
    def load_q_and_init(self):
        em0 = self.em
        em0.valu(f"v_mov_b32 {self.v_t.r(7)}, {self.s_w}", dst=[self.v_t.r(7)])
        em0.valu(f"v_mov_b32 {self.v_t.r(3)}, {self.s_qw0}", dst=[self.v_t.r(3)])
        self.debug_dump("ids", ["v0", self.v_t.r(7), self.v_t.r(3), self.v_qoff.r(0), self.v_qoff.r(1), self.v_h16])
        self._load_q_and_init()

    def _load_q_and_init(self):
        """Q into VGPRs (the S / P buffers are free here), then into AGPRs."""
        em, t = self.em, self.v_t
        for qb in range(2):
            em.valu(f"v_add_u32 {t.r(5 + qb)}, {self.v_qoff.r(qb)}, {self.v_h16}",
                    dst=[t.r(5 + qb)], src=[self.v_qoff.r(qb), self.v_h16])
        stage = [self.v_S[0][0], self.v_S[0][1], self.v_S[1][0], self.v_S[1][1]]
        def qtmp(qb, s):
            k = qb * self.NS + s           # 4-register slot k of 16
            return stage[k // 4].r(4 * (k % 4), 4)
        for qb in range(2):
            for s in range(self.NS):
                em.vmem_load_to(f"buffer_load_dwordx4 {qtmp(qb, s)}, {t.r(5 + qb)}, {self.s_rq}, 0 offen offset:{32 * s}",
                                qtmp(qb, s), src=[t.r(5 + qb)])
        em.salu("s_waitcnt vmcnt(0)")
        self.debug_dump("qv", [qtmp(qb, s).replace(":", ":").split(":")[0].replace("[", "") + "" for qb in range(2) for s in range(self.NS)])
        for qb in range(2):
            for s in range(self.NS):
                src = qtmp(qb, s)
                base = int(src[2:src.index(":")])
                for i in range(4):
                    em.valu(f"v_accvgpr_write_b32 {self.a_Q[qb][s].r(i)}, v{base + i}",
                            dst=[self.a_Q[qb][s].r(i)], src=[f"v{base + i}"])
        for qb in range(2):
            for db in range(self.NDB):
                blk = self.a_O[qb][db]
                for i in range(16):
                    em.valu(f"v_accvgpr_write_b32 {blk.r(i)}, 0", dst=[blk.r(i)])
        em.valu(f"v_mov_b32 {self.v_ninf}, {self.s_neg}", dst=[str(self.v_ninf)])
        em.valu(f"v_mov_b32 {self.v_resc}, {f32_hex(RESCALE)}", dst=[str(self.v_resc)])
        em.valu(f"v_mov_b32 {self.v_c}, s24", dst=[str(self.v_c)])
        for qb in range(2):
            em.valu(f"v_mov_b32 {self.v_m.r(qb)}, {self.s_neg}", dst=[self.v_m.r(qb)])
            em.valu(f"v_mov_b32 {self.v_l.r(qb)}, 0", dst=[self.v_l.r(qb)])
            em.valu(f"v_mov_b32 {self.v_mc.r(qb)}, 0", dst=[self.v_mc.r(qb)])

    # ------------------------------------------------------------------------
    # DMA of K(t) and V(t): tile index in sgpr `st`, LDS slot bases in sgprs
    # ------------------------------------------------------------------------
    def dma_tile(self, st, kslot_sgpr, vslot_sgpr):
        em, x = self.em, self.s_x
        # bytes left from the tile's first row to row_lim (0 when past it)
        em.salu(f"s_lshl_b32 {x[0]}, {st}, 6")                      # key0
        em.salu(f"s_sub_i32 {x[1]}, {self.s_rowlim}, {x[0]}")
        em.salu(f"s_max_i32 {x[1]}, {x[1]}, 0")
        em.salu(f"s_mul_i32 {x[2]}, {x[1]}, {self.s_rowb}")
        em.salu(f"s_mul_hi_u32 {x[3]}, {x[1]}, {self.s_rowb}")
        em.salu(f"s_cmp_eq_u32 {x[3]}, 0")
        em.salu(f"s_cselect_b32 {x[2]}, {x[2]}, 0x7fffffff")
        em.salu(f"s_min_u32 {x[2]}, {x[2]}, 0x7fffffff")
        # base = batch base + key0 * rowb
        em.salu(f"s_mul_i32 {x[4]}, {x[0]}, {self.s_rowb}")
        em.salu(f"s_mul_hi_u32 {x[5]}, {x[0]}, {self.s_rowb}")
        for rs, bb in ((self.s_rk, self.s_kb), (self.s_rv, self.s_vb)):
            em.salu(f"s_add_u32 {rs.r(0)}, {bb.r(0)}, {x[4]}")
            em.salu(f"s_addc_u32 {rs.r(1)}, {bb.r(1)}, {x[5]}")
            em.salu(f"s_and_b32 {rs.r(1)}, {rs.r(1)}, 0xffff")
            em.salu(f"s_mov_b32 {rs.r(2)}, {x[2]}")
            em.salu(f"s_mov_b32 {rs.r(3)}, 0x20000")
        # wave w fills rows 16w .. 16w+15: M0 = slot + (16w + RPD*i)*ROW
        em.salu(f"s_mul_i32 {x[0]}, {self.s_w}, {16 * self.ROW}")
        for i in range(self.DPW):
            em.salu(f"s_add_u32 {x[1]}, {kslot_sgpr}, {x[0]}")
            if i:
                em.salu(f"s_add_u32 {x[1]}, {x[1]}, {self.RPD * i * self.ROW}")
            em.salu(f"s_mov_b32 m0, {x[1]}")
            em.vmem(f"buffer_load_dwordx4 {self.v_kdma.r(i)}, {self.s_rk}, 0 offen lds", src=[self.v_kdma.r(i)])
        for i in range(self.DPW):
            em.salu(f"s_add_u32 {x[1]}, {vslot_sgpr}, {x[0]}")
            if i:
                em.salu(f"s_add_u32 {x[1]}, {x[1]}, {self.RPD * i * self.ROW}")
            em.salu(f"s_mov_b32 m0, {x[1]}")
            em.vmem(f"buffer_load_dwordx4 {self.v_vdma.r(i)}, {self.s_rv}, 0 offen lds", src=[self.v_vdma.r(i)])

    def wait_vm(self, n):
        self.em.salu(f"s_waitcnt vmcnt({n})")

    # ------------------------------------------------------------------------
    # building blocks; each returns a list of callables emitting one instruction
    # ------------------------------------------------------------------------
    def ops_k_loads(self, kb):
        """K operands of one sub-tile (kb of the tile in the K read slot)."""
        em = self.em
        out = []
        for s in range(self.NS):
            def f(s=s):
                em.ds_read(f"ds_read_b128 {self.v_KO[s]}, {self.v_kaddr.r(s)} offset:{kb * 32 * self.ROW}",
                           str(self.v_KO[s]), self.v_kaddr.r(s))
            out.append(f)
        return out

    def ops_v_loads(self, kb):
        """V operands of one sub-tile (kb of the tile addressed by v_vaddr)."""
        em = self.em
        out = []
        for th in range(2):
            for db in range(self.NDB):
                for e in range(2):
                    def f(th=th, db=db, e=e):
                        off = (32 * kb + 16 * th + 8 * e) * self.ROW
                        dst = self.v_VO[th][db].r(2 * e, 2)
                        em.ds_read(f"ds_read_b64_tr_b16 {dst}, {self.v_vaddr.r(db)} offset:{off}",
                                   dst, self.v_vaddr.r(db))
                    out.append(f)
        return out

    def ops_qk(self, buf):
        """S^T(sub-tile) = K . Q^T into S[buf]; 2*NS MFMAs."""
        em = self.em
        out = []
        for s in range(self.NS):
            for qb in range(2):
                def f(s=s, qb=qb):
                    d = self.S_(buf, qb)
                    em.mfma(self.mfma_op, d, str(self.v_KO[s]), str(self.a_Q[qb][s]), "0" if s == 0 else d)
                out.append(f)
        return out

    def ops_pv(self, pbuf):
        """O^T += V^T . P^T with P[pbuf]; 4*NDB MFMAs."""
        em = self.em
        out = []
        for th in range(2):
            for db in range(self.NDB):
                for qb in range(2):
                    def f(th=th, db=db, qb=qb):
                        o = str(self.a_O[qb][db])
                        em.mfma(self.mfma_op, o, str(self.v_VO[th][db]), str(self.v_P[pbuf][qb][th]), o)
                    out.append(f)
        return out

    def ops_max(self, buf):
        """Row max of S[buf] per query block into v_mx (both lane halves)."""
        em = self.em
        out = []
        for qb in range(2):
            S = self.v_S[buf][qb]
            mx = self.v_mx.r(qb)
            out.append(lambda S=S, mx=mx: em.valu(f"v_max3_f32 {mx}, {S.r(0)}, {S.r(1)}, {S.r(2)}",
                                                  dst=[mx], src=[S.r(0), S.r(1), S.r(2)]))
            for i in range(3, 15, 2):
                out.append(lambda S=S, mx=mx, i=i: em.valu(
                    f"v_max3_f32 {mx}, {mx}, {S.r(i)}, {S.r(i + 1)}", dst=[mx], src=[mx, S.r(i), S.r(i + 1)]))
            out.append(lambda S=S, mx=mx: em.valu(f"v_max_f32 {mx}, {mx}, {S.r(15)}", dst=[mx], src=[mx, S.r(15)]))
            tmp = self.v_t.r(6 + qb)
            out.append(lambda mx=mx, tmp=tmp: em.valu(f"v_mov_b32 {tmp}, {mx}", dst=[tmp], src=[mx]))
            out.append(lambda mx=mx, tmp=tmp: em.valu(f"v_permlane32_swap_b32 {mx}, {tmp}", dst=[mx, tmp], src=[mx, tmp]))
            out.append(lambda mx=mx, tmp=tmp: em.valu(f"v_max_f32 {mx}, {mx}, {tmp}", dst=[mx], src=[mx, tmp]))
        return out

    def ops_raise_test(self):
        """raise[qb] = c*mx > c*m + RESCALE, into s_m1 (qb 0) and s_m2 (qb 1)."""
        em, t = self.em, self.v_t
        out = []
        for qb, msk in ((0, self.s_m1), (1, self.s_m2)):
            a, b = t.r(2 + 2 * qb), t.r(3 + 2 * qb)
            out.append(lambda qb=qb, a=a: em.valu(f"v_mul_f32 {a}, s24, {self.v_mx.r(qb)}", dst=[a], src=[self.v_mx.r(qb)]))
            out.append(lambda qb=qb, b=b: em.valu(f"v_fma_f32 {b}, {self.v_m.r(qb)}, {self.v_c}, {self.v_resc}",
                                                  dst=[b], src=[self.v_m.r(qb), str(self.v_c), str(self.v_resc)]))
            out.append(lambda a=a, b=b, msk=msk: em.valu(f"v_cmp_gt_f32 {msk}, {a}, {b}", src=[a, b]))
        return out

    def ops_exp(self, buf, qb, pbuf):
        """P[pbuf][qb] = round(2^(c*S - mc)); rs[qb] = sum; S[buf][qb] holds p (fp32)."""
        em = self.em
        S = self.v_S[buf][qb]
        mc = self.v_mc.r(qb)
        rs = self.v_rs.r(qb)
        out = []
        for i in range(16):
            out.append(lambda i=i: em.valu(f"v_fma_f32 {S.r(i)}, {S.r(i)}, s24, -{mc}", dst=[S.r(i)], src=[S.r(i), mc]))
            out.append(lambda i=i: em.valu(f"v_exp_f32 {S.r(i)}, {S.r(i)}", dst=[S.r(i)], src=[S.r(i)], trans=True))
        out.append(lambda: em.valu(f"v_add_f32 {rs}, {S.r(0)}, {S.r(1)}", dst=[rs], src=[S.r(0), S.r(1)]))
        for i in range(2, 16):
            out.append(lambda i=i: em.valu(f"v_add_f32 {rs}, {rs}, {S.r(i)}", dst=[rs], src=[rs, S.r(i)]))
        out.append(lambda: em.valu(f"v_add_f32 {self.v_l.r(qb)}, {self.v_l.r(qb)}, {rs}",
                                   dst=[self.v_l.r(qb)], src=[self.v_l.r(qb), rs]))
        for th in range(2):
            P = self.v_P[pbuf][qb][th]
            for jj in range(4):
                lo, hi = S.r(8 * th + 2 * jj), S.r(8 * th + 2 * jj + 1)
                out.append(lambda P=P, jj=jj, lo=lo, hi=hi: em.valu(
                    f"{self.cvt_op} {P.r(jj)}, {lo}, {hi}", dst=[P.r(jj)], src=[lo, hi]))
        return out

    def ops_mask(self, buf, qb):
        """Set S[buf][qb] entries with key > last visible key to -inf.
        key of register i = k0 + 8*(i>>2) + 4h + (i&3); limh = lim - 4h."""
        em = self.em
        S = self.v_S[buf][qb]
        d = self.v_d.r(qb)
        out = [lambda: em.valu(f"v_subrev_u32 {d}, {self.s_k0}, {self.v_limh.r(qb)}", dst=[d], src=[self.v_limh.r(qb)])]
        for i in range(16):
            ci = 8 * (i >> 2) + (i & 3)
            out.append(lambda i=i, ci=ci: em.valu(f"v_cmp_lt_i32 vcc, {d}, {ci}", src=[d]))
            out.append(lambda i=i: em.valu(f"v_cndmask_b32 {S.r(i)}, {S.r(i)}, {self.v_ninf}, vcc",
                                           dst=[S.r(i)], src=[S.r(i), str(self.v_ninf)]))
        return out

    def emit_all(self, ops):
        for f in ops:
            f()

    # ------------------------------------------------------------------------
    def rescale(self):
        """Slow path body: move the reference max of raising rows, rescale O
        and l by alpha = 2^(c*m_old - c*m_new).  Masks in s_m1 / s_m2."""
        em, t = self.em, self.v_t
        em.drain()
        for qb, msk in ((0, self.s_m1), (1, self.s_m2)):
            m, mx = self.v_m.r(qb), self.v_mx.r(qb)
            a = t.r(2)
            em.valu(f"v_mul_f32 {t.r(3)}, s24, {m}", dst=[t.r(3)], src=[m])
            em.valu(f"v_mul_f32 {t.r(4)}, s24, {mx}", dst=[t.r(4)], src=[mx])
            em.valu(f"v_sub_f32 {a}, {t.r(3)}, {t.r(4)}", dst=[a], src=[t.r(3), t.r(4)])
            em.valu(f"v_exp_f32 {a}, {a}", dst=[a], src=[a], trans=True)
            em.valu(f"v_cndmask_b32 {a}, 1.0, {a}, {msk}", dst=[a], src=[a])
            em.valu(f"v_cndmask_b32 {m}, {m}, {mx}, {msk}", dst=[m], src=[m, mx])
            em.valu(f"v_mul_f32 {self.v_l.r(qb)}, {self.v_l.r(qb)}, {a}", dst=[self.v_l.r(qb)], src=[self.v_l.r(qb), a])
            # mc = c*m, or 0 while m = -inf
            em.valu(f"v_mul_f32 {self.v_mc.r(qb)}, s24, {m}", dst=[self.v_mc.r(qb)], src=[m])
            em.valu(f"v_cmp_eq_f32 vcc, {self.s_neg}, {m}", src=[m])
            em.valu(f"v_cndmask_b32 {self.v_mc.r(qb)}, {self.v_mc.r(qb)}, 0, vcc",
                    dst=[self.v_mc.r(qb)], src=[self.v_mc.r(qb)])
            for db in range(self.NDB):
                blk = self.a_O[qb][db]
                for i in range(16):
                    tmp = t.r(5 + (i & 1))
                    em.valu(f"v_accvgpr_read_b32 {tmp}, {blk.r(i)}", dst=[tmp], src=[blk.r(i)])
                    em.valu(f"v_mul_f32 {tmp}, {tmp}, {a}", dst=[tmp], src=[tmp, a])
                    em.valu(f"v_accvgpr_write_b32 {blk.r(i)}, {tmp}", dst=[blk.r(i)], src=[tmp])
        em.drain()

    # ------------------------------------------------------------------------
    # one pipelined step j:
    #   half A: P.V(j) [P buffer pb, V operands in VO] next to the row max of
    #           sub-tile j+1 [S buffer sb], the lazy-rescale test, the
    #           exponentials of j+1 for query block 0 and the K operand loads
    #           for S^T(j+2) (sub-tile kb_k of the tile in the K read slot);
    #   half B: S^T(j+2) into S[1-sb] next to the exponentials of j+1 for
    #           query block 1 and the V operand loads for P.V(j+1) (sub-tile
    #           kb_v of the tile addressed by v_vaddr).
    # The slow path (some row's max rose by more than 2^8) is recorded and
    # emitted out of line by emit_slow().
    # ------------------------------------------------------------------------
    def step(self, sb, pb, kb_k, kb_v, do_soft=True, do_qk=True, do_vload=True):
        em = self.em
        pv = self.ops_pv(pb)
        slow = None
        if do_soft:
            # mask sub-tile j+1 (keys s_k0 .. s_k0+31) when it crosses the
            # wave's diagonal or the key tail
            l_skip = self.lab("nomask")
            em.salu(f"s_add_u32 {self.s_x[0]}, {self.s_k0}, 32")
            em.salu(f"s_cmp_gt_i32 {self.s_x[0]}, {self.s_kvfull}")
            em.salu(f"s_cbranch_scc0 {l_skip}")
            snap = em.snapshot()
            for qb in range(2):
                self.emit_all(self.ops_mask(sb, qb))
            em.label(l_skip)
            # the masked path only resolved hazards the skip path still has
            em.restore(snap)
            lead = 4
            interleave(em, pv[:lead], self.ops_max(sb) + self.ops_raise_test())
            em.salu(f"s_or_b64 {self.s_or}, {self.s_m1}, {self.s_m2}")
            l_slow, l_back = self.lab("slow"), self.lab("back")
            em.salu(f"s_cbranch_scc1 {l_slow}")
            snap = em.snapshot()
            kl = self.ops_k_loads(kb_k) if do_qk else []
            interleave(em, pv[lead:], kl + self.ops_exp(sb, 0, 1 - pb))
            slow = (l_slow, l_back, snap, sb, pb, kb_k, do_qk, lead)
            # slow path rejoins here fully drained, which is safe for what follows
            em.label(l_back)
        else:
            kl = self.ops_k_loads(kb_k) if do_qk else []
            interleave(em, pv, kl)
        others = []
        if do_soft:
            others += self.ops_exp(sb, 1, 1 - pb)
        if do_vload:
            others += self.ops_v_loads(kb_v)
        if do_qk:
            interleave(em, self.ops_qk(1 - sb), others)
        else:
            self.emit_all(others)
        return slow

    def emit_slow(self, slow):
        """Out-of-line slow path: finish P.V(j), rescale O and l, then the
        exponentials of query block 0 and the K loads, and jump back."""
        em = self.em
        l_slow, l_back, snap, sb, pb, kb_k, do_qk, lead = slow
        em.restore(snap)
        em.label(l_slow)
        self.emit_all(self.ops_pv(pb)[lead:])
        self.rescale()
        self.emit_all(self.ops_exp(sb, 0, 1 - pb))
        if do_qk:
            self.emit_all(self.ops_k_loads(kb_k))
        em.drain()
        em.salu(f"s_branch {l_back}")

    # ------------------------------------------------------------------------
    debug_point = None   # debugging aid: name of a point where registers are dumped

    def debug_dump(self, point, regs):
        """At `point` (when it is the selected one), store `regs` (VGPR/AGPR
        names) raw to the O buffer at ((w*64 + lane) * len(regs) + r) * 4 and
        end the program."""
        if self.debug_point != point:
            return
        em, t = self.em, self.v_t
        em.drain()
        n = len(regs)
        em.salu(f"s_lshl_b32 {self.s_x[0]}, {self.s_w}, 6")
        em.valu(f"v_add_u32 {t.r(0)}, {self.s_x[0]}, v0", dst=[t.r(0)], src=["v0"])
        em.valu(f"v_mul_u32_u24 {t.r(0)}, {4 * n}, {t.r(0)}", dst=[t.r(0)], src=[t.r(0)])
        for i, r in enumerate(regs):
            src = r
            if r.startswith("a"):
                em.valu(f"v_accvgpr_read_b32 {t.r(1)}, {r}", dst=[t.r(1)], src=[r])
                src = t.r(1)
            em.vmem(f"buffer_store_dword {src}, {t.r(0)}, {self.s_ro}, 0 offen offset:{4 * i}",
                    src=[src, t.r(0)])
        em.salu("s_waitcnt vmcnt(0)")
        em.salu("s_endpgm")

    def slot_addr_update(self, vgpr_blk, off_blk, n, sgpr):
        for i in range(n):
            self.em.valu(f"v_add_u32 {vgpr_blk.r(i)}, {sgpr}, {off_blk.r(i)}",
                         dst=[vgpr_blk.r(i)], src=[off_blk.r(i)])

    def epilogue(self):
        em, t = self.em, self.v_t
        em.drain()
        self.debug_dump("epi", [self.v_l.r(0), self.v_l.r(1), self.v_mc.r(0), self.v_mc.r(1),
                                self.v_m.r(0), self.v_m.r(1)])
        # dims 32 db + 8 i4 + 4 h .. +3 of row q: bytes qoff + 8 h + 64 db + 16 i4
        em.valu(f"v_lshrrev_b32 {t.r(0)}, 5, v0", dst=[t.r(0)], src=["v0"])      # h
        em.valu(f"v_lshlrev_b32 {t.r(7)}, 3, {t.r(0)}", dst=[t.r(7)], src=[t.r(0)])  # 8h
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
                for i4 in range(4):
                    for k in range(4):
                        dst = t.r(3 + k)
                        em.valu(f"v_accvgpr_read_b32 {dst}, {blk.r(4 * i4 + k)}", dst=[dst],
                                src=[blk.r(4 * i4 + k)])
                        em.valu(f"v_mul_f32 {dst}, {dst}, {t.r(1)}", dst=[dst], src=[dst, t.r(1)])
                    em.valu(f"{self.cvt_op} {t.r(3)}, {t.r(3)}, {t.r(4)}", dst=[t.r(3)], src=[t.r(3), t.r(4)])
                    em.valu(f"{self.cvt_op} {t.r(4)}, {t.r(5)}, {t.r(6)}", dst=[t.r(4)], src=[t.r(5), t.r(6)])
                    off = 64 * db + 16 * i4
                    em.vmem(f"buffer_store_dwordx2 {t.r(3, 2)}, {t.r(2)}, {self.s_ro}, 0 offen offset:{off}",
                            src=[t.r(3, 2), t.r(2)])
            # LSE = ln2 * (mc + log2 l), -inf when l = 0 (vcc still holds l > 0)
            em.valu(f"v_log_f32 {t.r(3)}, {l}", dst=[t.r(3)], src=[l], trans=True)
            em.valu(f"v_add_f32 {t.r(3)}, {self.v_mc.r(qb)}, {t.r(3)}", dst=[t.r(3)], src=[self.v_mc.r(qb), t.r(3)])
            em.valu(f"v_mul_f32 {t.r(3)}, {f32_hex(LN2)}, {t.r(3)}", dst=[t.r(3)], src=[t.r(3)])
            em.valu(f"v_cndmask_b32 {t.r(3)}, {self.v_ninf}, {t.r(3)}, vcc", dst=[t.r(3)],
                    src=[t.r(3), str(self.v_ninf)])
            em.vmem(f"buffer_store_dword {t.r(3)}, {self.v_lseoff.r(qb)}, {self.s_rl}, 0 offen",
                    src=[t.r(3), self.v_lseoff.r(qb)])
        em.salu("s_endpgm")

    # ------------------------------------------------------------------------
    def body(self):
        em = self.em
        self.alloc()
        self.prologue()
        self.lane_constants()
        self.load_q_and_init()
        x = self.s_x
        l_epi = self.lab("epilogue")
        em.salu(f"s_cmp_eq_u32 {self.s_ntiles}, 0")
        em.salu(f"s_cbranch_scc1 {l_epi}")
        # ---- first three tiles into the rings ----------------------------------
        for tt in range(3):
            em.salu(f"s_mov_b32 {x[5]}, {tt}")
            em.salu(f"s_mov_b32 {self.s_kdsl}, {self.KBASE + tt * self.TILE}")
            em.salu(f"s_mov_b32 {self.s_vdsl}, {self.VBASE + tt * self.TILE}")
            self.dma_tile(x[5], self.s_kdsl, self.s_vdsl)
        self.wait_vm(2 * self.DPW)
        em.salu("s_barrier")
        # ---- pipeline prologue: S^T(0), max(0); S^T(1) next to exp(0) -----------
        em.salu(f"s_mov_b32 {self.s_ksl}, 0")
        self.slot_addr_update(self.v_kaddr, self.v_koff, self.NS, self.s_ksl)
        em.salu(f"s_mov_b32 {self.s_vsl0}, {self.VBASE}")
        self.slot_addr_update(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl0)
        self.debug_dump("q", [self.a_Q[q][s].r(i) for q in range(2) for s in range(self.NS) for i in range(4)])
        self.emit_all(self.ops_k_loads(0))
        self.debug_dump("ko0", [self.v_KO[s].r(i) for s in range(self.NS) for i in range(4)])
        self.emit_all(self.ops_qk(0))
        self.debug_dump("s0", [self.v_S[0][q].r(i) for q in range(2) for i in range(16)])
        self.emit_all(self.ops_k_loads(1))
        em.salu(f"s_mov_b32 {self.s_k0}, 0")
        l_skip = self.lab("nomask0")
        em.salu(f"s_cmp_gt_i32 32, {self.s_kvfull}")
        em.salu(f"s_cbranch_scc0 {l_skip}")
        snap = em.snapshot()
        for qb in range(2):
            self.emit_all(self.ops_mask(0, qb))
        em.label(l_skip)
        em.restore(snap)
        self.emit_all(self.ops_max(0))
        for qb in range(2):
            m, mx, mc = self.v_m.r(qb), self.v_mx.r(qb), self.v_mc.r(qb)
            em.valu(f"v_mov_b32 {m}, {mx}", dst=[m], src=[mx])
            em.valu(f"v_mul_f32 {mc}, s24, {m}", dst=[mc], src=[m])
            em.valu(f"v_cmp_eq_f32 vcc, {self.s_neg}, {m}", src=[m])
            em.valu(f"v_cndmask_b32 {mc}, {mc}, 0, vcc", dst=[mc], src=[mc])
        interleave(em, self.ops_qk(1), self.ops_exp(0, 0, 0) + self.ops_exp(0, 1, 0) + self.ops_v_loads(0))
        em.salu("s_barrier")
        # ---- main loop over tiles t = 0 .. n_tiles-2 -----------------------------
        slows = []
        l_last, l_loop = self.lab("last"), self.lab("loop")
        em.salu(f"s_mov_b32 {self.s_t}, 0")
        em.salu(f"s_sub_u32 {self.s_tlast}, {self.s_ntiles}, 1")
        em.salu(f"s_cmp_eq_u32 {self.s_tlast}, 0")
        em.salu(f"s_cbranch_scc1 {l_last}")
        em.drain()
        em.label(l_loop)
        snap_loop = em.snapshot()
        # ring slots for tile t: K read (t+1)%3, K dma t%3, V cur t%4, V next (t+1)%4, V dma (t+3)%4
        self.emit_slot_sgprs()
        em.salu(f"s_add_u32 {x[5]}, {self.s_t}, 3")
        self.dma_tile(x[5], self.s_kdsl, self.s_vdsl)
        self.slot_addr_update(self.v_kaddr, self.v_koff, self.NS, self.s_ksl)
        em.salu(f"s_lshl_b32 {self.s_k0}, {self.s_t}, 6")
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        slows.append(self.step(sb=1, pb=0, kb_k=0, kb_v=1))
        self.slot_addr_update(self.v_vaddr, self.v_voff, self.NDB, self.s_vsl1)
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        slows.append(self.step(sb=0, pb=1, kb_k=1, kb_v=0))
        self.wait_vm(2 * self.DPW)
        em.salu("s_barrier")
        em.salu(f"s_add_u32 {self.s_t}, {self.s_t}, 1")
        em.salu(f"s_cmp_lt_u32 {self.s_t}, {self.s_tlast}")
        em.drain()
        em.salu(f"s_cbranch_scc1 {l_loop}")
        # ---- last tile: P.V(2t) next to softmax(2t+1), then P.V(2t+1) -------------
        em.label(l_last)
        em.drain()
        em.salu(f"s_lshl_b32 {self.s_k0}, {self.s_t}, 6")
        em.salu(f"s_add_u32 {self.s_k0}, {self.s_k0}, 32")
        slows.append(self.step(sb=1, pb=0, kb_k=0, kb_v=1, do_qk=False))
        self.step(sb=0, pb=1, kb_k=1, kb_v=0, do_soft=False, do_qk=False, do_vload=False)
        em.label(l_epi)
        self.epilogue()
        # ---- out-of-line slow paths --------------------------------------------------
        for sl in slows:
            if sl is not None:
                self.emit_slow(sl)

    def emit_slot_sgprs(self):
        """Slot byte addresses for tile s_t (s_t % 3 and s_t % 4 from scratch)."""
        em, x = self.em, self.s_x
        # t % 3 via (t * 0xAAAB) >> 17 for t < 2^16 -> quotient; remainder = t - 3q
        em.salu(f"s_mul_i32 {x[0]}, {self.s_t}, 0xAAAB")
        em.salu(f"s_lshr_b32 {x[0]}, {x[0]}, 17")
        em.salu(f"s_mul_i32 {x[0]}, {x[0]}, 3")
        em.salu(f"s_sub_u32 {x[0]}, {self.s_t}, {x[0]}")            # t % 3
        em.salu(f"s_mul_i32 {self.s_kdsl}, {x[0]}, {self.TILE}")
        em.salu(f"s_add_u32 {self.s_kdsl}, {self.s_kdsl}, {self.KBASE}")   # K dma slot (t+3)%3 = t%3
        em.salu(f"s_add_u32 {x[1]}, {x[0]}, 1")
        em.salu(f"s_cmp_eq_u32 {x[1]}, 3")
        em.salu(f"s_cselect_b32 {x[1]}, 0, {x[1]}")
        em.salu(f"s_mul_i32 {self.s_ksl}, {x[1]}, {self.TILE}")           # K read slot (t+1)%3
        em.salu(f"s_and_b32 {x[0]}, {self.s_t}, 3")
        em.salu(f"s_mul_i32 {self.s_vsl0}, {x[0]}, {self.TILE}")           # V(t)
        em.salu(f"s_add_u32 {x[1]}, {x[0]}, 1")
        em.salu(f"s_and_b32 {x[1]}, {x[1]}, 3")
        em.salu(f"s_mul_i32 {self.s_vsl1}, {x[1]}, {self.TILE}")           # V(t+1)
        em.salu(f"s_add_u32 {x[1]}, {x[0]}, 3")
        em.salu(f"s_and_b32 {x[1]}, {x[1]}, 3")
        em.salu(f"s_mul_i32 {self.s_vdsl}, {x[1]}, {self.TILE}")           # V(t+3)

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
        for off, kind, access in [(0, "global_buffer", "read_only"), (8, "global_buffer", "read_only"),
                                  (16, "global_buffer", "read_only"), (24, "global_buffer", "write_only"),
                                  (32, "global_buffer", "write_only")]:
            lines += [f"      - .actual_access: {access}", "        .address_space: global",
                      f"        .offset: {off}", "        .size: 8", f"        .value_kind: {kind}"]
        for off in range(40, KERNARG_BYTES, 4):
            lines += [f"      - .offset: {off}", "        .size: 4", "        .value_kind: by_value"]
        lines += [
            f"    .group_segment_fixed_size: {k['lds']}",
            "    .kernarg_segment_align: 8",
            f"    .kernarg_segment_size: {KERNARG_BYTES}",
            "    .max_flat_workgroup_size: 256",
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
    texts, metas = [], []
    for dt, D in VARIANTS:
        g = Gen(dt, D)
        txt, info = g.assemble_text()
        texts.append(txt)
        metas.append(info)
    return "".join(texts) + metadata(metas)


if __name__ == "__main__":
    import sys
    out = sys.argv[1] if len(sys.argv) > 1 else "fa_fwd_gfx950.s"
    with open(out, "w") as f:
        f.write(generate_all())
    print(out)
