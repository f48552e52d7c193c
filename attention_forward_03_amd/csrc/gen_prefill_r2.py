"""Writes the main loop of the 64-rows-per-wave prefill kernel (head_dim 128, 16-bit
inputs) as the text of one inline-asm statement, with every register and every wait
chosen here.

Why generated: with one wave per SIMD the wave has to interleave the vector softmax with
its own matrix-core products instruction by instruction, while the output accumulators,
the Q fragments, two score tiles and two probability tiles stay resident. Left to the
compiler, the register allocation of such a loop is not stable (accumulators move
between AGPRs, Q fragments get staged before every product), so the schedule and the
register map are fixed here. The algorithm is the one described at the head of
fwd_r2_kernel in prefill.hip; this file only lays out its instruction stream.

Usage: python gen_prefill_r2.py OUT_DIR  -> OUT_DIR/prefill_r2_{bf16,f16}_m{0,1,2}.inc and
OUT_DIR/prefill_r2_clobbers.inc (a macro with the registers the statement writes). Each
.inc holds one string literal (the asm template; labels use %= so that every
instantiation has its own).

Modes: 0 = no mask at all (every tile full, no causal / window / ragged tail); 1 = a mask
(causal, window, tail); 2 = softcap, with or without a mask.

Schedule of a phase X(i) (one 32-key sub-tile): 32 steps, each with one matrix-core
product (even steps S(i+1) = K Q^T, odd steps O^T += V^T P(i-1)^T) and a slice of the
vector work on sub-tile i (emitted between the step's fragment read-ahead and its wait
and product), software-pipelined so that no step waits on its own results:
  step g: softcap / mask of score g (and, where row maxima are tracked, at odd g the max
  of the pair);   step g+1: FMA (scale, minus the reference) of score g;   step g+2:
  exp2 of score g;   step 2u+4: pack pair u to 16 bits;   steps 2u+4, 2u+5: add its two
  values to the row sum (in fp32: a packed dot product would hold up the matrix core for
  about 14 cycles).
The last four steps of that pipeline run in the first steps of the next phase. The wave
issues one instruction at a time, so every vector instruction in a step takes issue
slots from the 32 cycles of its product: the stream keeps the vector work per step to a
handful (no address arithmetic: every LDS address is a per-lane register plus an
immediate, the tile loop being unrolled over the three LDS buffers).

Two bodies per tile: "plain" (no mask, every row already has its reference max: no row
maxima at all; a running max of each phase's row sums guards against a probability
past the slack, checked once per pass) and "tracked" (mask, row maxima, and after each
phase one compare per row block: a row whose max passed its threshold sends the wave to
an out-of-line block that handles first unmasked keys and sets the redo flag).

Hardware rules the stream keeps (gfx950): a matrix-core result is not touched by any
other instruction for 12 wait states; a register written by a vector instruction is not
read by a product for 2; an exp2 / rcp / log result is not read in the next slot; a
permlane swap's operands are not touched for 2 before or after it; M0 is written one slot
before the LDS-DMA load that uses it; every LDS read is waited for (s_waitcnt lgkmcnt)
before its product, counting the reads issued after it in program order.

Register map:
  a[0:127]      O^T accumulators, block (rb, db) at a[(rb*4+db)*16 : +15]
  a[128:191]    Q fragments, (rb, ks) at a[128 + (rb*8+ks)*4 : +3]
  inputs (set by the C++ code before the statement):
  v[0:1] v[2:3]   Q fragment addresses (row block 0, 1)
  v[4:5] v[6:7]   O row addresses        v[8:9] v[10:11]  LSE addresses
  v12 v13         4*hi - key_lo          v14 v15          key_n (allowed keys per row)
  v16 v17         query rows             v19 v20          K / V load lane offsets (bytes)
  v21 v22         K / V LDS read lane offsets (bytes, within a buffer)
  s[40:41] s[42:43]  K / V bases    s44 s45  K / V token strides (elements)
  s46 Lk   s47 first key   s48 tiles   s49 score scale (log2 units, > 0)
  s50 softcap: scale / c   s51 softcap: c log2(e)   s53 wave   s54 Lq   s55 LSE wanted
  s56 LDS base (bytes)   s57 s58  the wave's keys that need no mask: [s57, s58)
LDS: K buffers 0..2, V buffers 3..5 (16 KiB each: 64 keys x 128 x 2 bytes, swizzled),
the redo flag after them.
"""
import os
import sys

TB = 16384       # bytes of one 64 x 128 K or V tile
HALF = 8192      # bytes of 32 rows
NKS = 8          # 16-wide k-steps of D
NDB = 4          # 32-wide blocks of D
RB = 2           # 32-row query blocks per wave
PF = 3           # fragments read ahead (ring of 4)
DMA_EVERY = 4    # steps between tile loads
NSTEP = 32       # products per phase
FLAG = 6 * TB    # LDS byte offset of the redo flag
LN2 = "0x3f317218"
RSRC_FLAGS = "0x20000"     # raw buffer, 32-bit elements

# VGPRs used by the stream (the epilogue's temporaries reuse the fragment rings)
S_X, S_Y = 24, 56      # scores of even / odd sub-tiles; row block rb at +16*rb
P_X, P_Y = 88, 104     # probabilities; (rb, t) at +(rb*2+t)*4
KF, VF = 120, 136      # fragment rings, 4 slots of 4
NMB = 152              # [rb] 16 copies of -MU: the first S product of a sub-tile starts there
ET = 184               # exp-pipeline temporaries, 4 per sub-tile parity
KR = 192               # [ks] K read address of fragment ks (buffer 0, rows 0..31)
VR = 200               # [db] V read address of column block db (buffer 3, rows 0..31)
KO = 204               # [n] K load lane offset of load n
VO = 208               # [n] V load lane offset of load n
ZERO = 212             # 4 registers
M, MU, L, LSUB, LSUB2 = 216, 218, 220, 222, 224   # [rb] each; LSUB: row sums of even
                                                   # sub-tiles, LSUB2: of odd ones
MT = 226               # [rb] threshold of the per-phase check (scores relative to MU)
LMX = 228              # [rb] running max of the phase row sums
MXA, KBASE = 230, 232  # [rb] running row max of a sub-tile; first key offset per lane
CM = 234               # [rb] softcap: c log2(e) - MU
MXS = 236              # [rb]
DELTA, MUOLD = 238, 240  # [rb] change of the reference, its old value (rare block, seed)
T0, T1, T2, T3 = 242, 243, 244, 245
VNINF, VM2C, VCAPK = 246, 247, 248
NVGPR = 249            # first unused
EP = KF                # 8 epilogue temporaries
INV = KF + 8           # [rb]
LT = KF + 10           # [rb]

# Persistent form: one workgroup per CU runs its work items one after another. Items are
# read from a table in LDS (one record of 16 dwords per item, written by the C++ code):
#   0-1 Q base, 2-3 O base, 4-5 LSE base, 6-7 K base, 8-9 V base (byte addresses; Q and O
#   at row 0 of the item's sequence, LSE at that row's entry, K and V at key 0 of the
#   sequence), 10 first query row of the item within its sequence, 11 Lq, 12 Lk,
#   13 first key tile start, 14 key tiles, 15 sink (log2 units).
# Extra inputs: s30 items, s31 table address (LDS bytes), s32 window, s33 causal, s34 / s35
# Q / O row strides (bytes), v249 = wave * 64 + lane % 32, v250 = lane / 32.
REC = 64               # bytes of a record
RECV = P_X             # 16 VGPRs the current record is read into (free between items)
QNEXT = 192            # a[192:255]: the next item's Q fragments, raw, loaded while this one ends
SK_ITEM, SK_FLAG = 96, 97   # item index; byte offset (0 / 4) of this item's redo-flag slot

# SGPRs used by the stream
SJ, SKT, ST, ST2, ST3 = 60, 61, 62, 63, 64
SKROW, SVROW, SWB, SKT2, SATT, SUNM = 65, 66, 67, 68, 69, 70
KSTEP, VSTEP, KEYK, KEYV, SK2, SV2 = 72, 73, 74, 75, 76, 77   # tile-load resource stepping
SMASK, SMASK2, SEXEC, SPAIR = 80, 82, 84, 86   # pairs
SCHK = SEXEC             # check of row block 0 (the loop), exec save (the epilogue)
RSK, RSV = 88, 92        # buffer resources (4 each)
NSGPR_LO, NSGPR_HI = 60, 96


def v(i, n=1):
    return f"v{i}" if n == 1 else f"v[{i}:{i + n - 1}]"


def a(i, n=1):
    return f"a{i}" if n == 1 else f"a[{i}:{i + n - 1}]"


def s(i, n=1):
    return f"s{i}" if n == 1 else f"s[{i}:{i + n - 1}]"


def kbuf(c, h):
    """Immediate offset of half h (rows 32h..32h+31) of buffer c (K: c, V: 3 + c)."""
    return c * TB + h * HALF


class Gen:
    def __init__(self, bf16, mode, persistent=False):
        self.bf16 = bf16
        self.mode = mode
        self.persistent = persistent
        # slack: P < 2^slack; fp16 probabilities must stay below 2^16
        self.slack_bits = "0x42200000" if bf16 else "0x41700000"   # 40 / 15
        self.sum_limit = "0x71800000" if bf16 else "0x47000000"    # 2^100 / 2^15
        self.out = []
        self.lds = []   # tags of LDS reads that may be in flight, in issue order
        self.n = 0
        self.rare = []
        self.et, self.lsub = ET, LSUB

    def emit(self, line):
        self.out.append(line)

    def uniq(self, name):
        self.n += 1
        return f"L_{name}{self.n}_%="

    # ------------------------------------------------------------------ LDS waits
    def lds_op(self, tag):
        self.lds.append(tag)

    def wait_for(self, tag):
        hits = [i for i, t in enumerate(self.lds) if t == tag]
        if not hits:  # already waited for
            return
        idx = max(hits)
        after = len(self.lds) - 1 - idx
        if after < 15:
            self.emit(f"s_waitcnt lgkmcnt({after})")
        self.lds = self.lds[idx + 1:]

    def relabel(self):
        # the read-ahead of the phase that just ended feeds the next phase
        self.lds = [("k", t[1]) if t[0] == "kn" else ("v", t[1]) if t[0] == "vn" else ("-", 0) for t in self.lds]

    # ------------------------------------------------------------------ pieces
    def mfma(self, d, av, bv, c):
        op = "v_mfma_f32_32x32x16_bf16" if self.bf16 else "v_mfma_f32_32x32x16_f16"
        self.emit(f"{op} {d}, {av}, {bv}, {c}")

    def read_k(self, ofs, ks, slot, tag):
        self.emit(f"ds_read_b128 {v(KF + 4 * slot, 4)}, {v(KR + ks)} offset:{ofs}")
        self.lds_op(tag)

    def read_v(self, ofs, f, slot, tag):
        t, db = f // NDB, f % NDB
        off = ofs + t * 16 * 256
        self.emit(f"ds_read_b64_tr_b16 {v(VF + 4 * slot, 2)}, {v(VR + db)} offset:{off}")
        self.emit(f"ds_read_b64_tr_b16 {v(VF + 4 * slot + 2, 2)}, {v(VR + db)} offset:{off + 8 * 256}")
        self.lds_op(tag)
        self.lds_op(tag)

    def score(self, sbase, g):
        """Register of score g (0..31) of a sub-tile: row block g // 16, element g % 16."""
        return sbase + 16 * (g // 16) + g % 16

    def pword(self, pbase, u):
        """Register of the packed probabilities of pair u (0..15)."""
        rr, e = u // 8, 2 * (u % 8)
        return pbase + (rr * 2 + e // 8) * 4 + (e % 8) // 2

    def exp_elem(self, sbase, g):
        """P of score g: its register holds the score in log2 units minus the reference."""
        self.emit(f"v_exp_f32 {v(self.et + g % 4)}, {v(self.score(sbase, g))}")

    def cvt_pair(self, pbase, u):
        g0 = 2 * u
        pw = self.pword(pbase, u)
        cvt = "v_cvt_pk_bf16_f32" if self.bf16 else "v_cvt_pk_f16_f32"
        self.emit(f"{cvt} {v(pw)}, {v(self.et + g0 % 4)}, {v(self.et + (g0 + 1) % 4)}")

    def sum_elem(self, g):
        """Row sum of the probabilities in fp32."""
        self.emit(f"v_add_f32 {v(self.lsub + g // 16)}, {v(self.et + g % 4)}, {v(self.lsub + g // 16)}")

    def exp_unit(self, sbase, pbase, u):
        """All of P for pair u at once (the rare path)."""
        g0 = 2 * u
        self.exp_elem(sbase, g0)
        self.exp_elem(sbase, g0 + 1)
        self.emit("s_nop 0")
        self.cvt_pair(pbase, u)
        self.sum_elem(g0)
        self.sum_elem(g0 + 1)
    def softcap(self, src, dst, rr):
        # capped - MU = (c log2 e - MU) - 2 c log2 e / (2^x + 1), x = 2 log2(e) s scale / c
        # (the product with Q pre-scaled by 2 log2(e) scale / c)
        self.emit(f"v_exp_f32 {v(T2)}, {v(src)}")
        self.emit("s_nop 0")
        self.emit(f"v_add_f32 {v(T2)}, 1.0, {v(T2)}")
        self.emit(f"v_rcp_f32 {v(T2)}, {v(T2)}")
        self.emit("s_nop 0")
        self.emit(f"v_fma_f32 {v(dst)}, {v(T2)}, {v(VM2C)}, {v(CM + rr)}")
    def softcap_filled(self, r, rr, fillers):
        """softcap() of score register r in place, with independent instructions (callables
        from fillers) in the slots after the exp2 and the reciprocal, whose results may not
        be read by the next instruction; s_nop 0 where no filler is left."""
        def gap():
            if fillers:
                fillers.pop(0)()
            else:
                self.emit("s_nop 0")
        self.emit(f"v_exp_f32 {v(T2)}, {v(r)}")
        gap()
        self.emit(f"v_add_f32 {v(T2)}, 1.0, {v(T2)}")
        self.emit(f"v_rcp_f32 {v(T2)}, {v(T2)}")
        gap()
        self.emit(f"v_fma_f32 {v(r)}, {v(T2)}, {v(VM2C)}, {v(CM + rr)}")

    def mask(self, src, dst, rr, e):
        """dst = src if key e of row block rr is allowed, else -inf (KBASE set)."""
        off = (e >> 2) * 8 + (e & 3)
        self.emit(f"v_add_u32 {v(T3)}, {off}, {v(KBASE + rr)}")
        self.emit(f"v_cmp_gt_u32 vcc, {v(14 + rr)}, {v(T3)}")
        self.emit(f"v_cndmask_b32 {v(dst)}, {v(VNINF)}, {v(src)}, vcc")

    def seed_max_unit(self, sbase, u, masked):
        """Max of score pair u into MXA, the scores left as they are (the capped / masked
        values go to T0, T1; softcap and mask use T2, T3)."""
        rr, e = u // 8, 2 * (u % 8)
        x = [sbase + 16 * rr + e, sbase + 16 * rr + e + 1]
        for k in range(2):
            if self.mode == 2:
                self.softcap(x[k], T0 + k, rr)
                x[k] = T0 + k
            if masked:
                self.mask(x[k], T0 + k, rr, e + k)
                x[k] = T0 + k
        self.emit(f"v_max3_f32 {v(MXA + rr)}, {v(MXA + rr)}, {v(x[0])}, {v(x[1])}")

    def mask_elem(self, sbase, g, masked):
        """Softcap (mode 2) and mask of score g of a sub-tile, in place."""
        rr, e = g // 16, g % 16
        r = sbase + 16 * rr + e
        if self.mode == 2:
            self.softcap(r, r, rr)
        if masked:
            self.mask(r, r, rr, e)

    def max_pair(self, sbase, u):
        rr, e = u // 8, 2 * (u % 8)
        r = sbase + 16 * rr + e
        self.emit(f"v_max3_f32 {v(MXA + rr)}, {v(MXA + rr)}, {v(r)}, {v(r + 1)}")

    def gap(self):
        self.emit("s_nop 7")
        self.emit("s_nop 3")

    def exchange_max(self):
        """MXS[rb] = max of MXA[rb] over lanes l and l^32 (the two halves of a row)."""
        self.emit(f"v_mov_b32 {v(T0)}, {v(MXA)}")
        self.emit(f"v_mov_b32 {v(T1)}, {v(MXA)}")
        self.emit(f"v_mov_b32 {v(T2)}, {v(MXA + 1)}")
        self.emit(f"v_mov_b32 {v(T3)}, {v(MXA + 1)}")
        self.emit("s_nop 1")
        self.emit(f"v_permlane32_swap_b32 {v(T0)}, {v(T1)}")
        self.emit(f"v_permlane32_swap_b32 {v(T2)}, {v(T3)}")
        self.emit("s_nop 1")
        self.emit(f"v_max_f32 {v(MXS)}, {v(T0)}, {v(T1)}")
        self.emit(f"v_max_f32 {v(MXS + 1)}, {v(T2)}, {v(T3)}")

    # ------------------------------------------------------------------ tile loads
    def rsrc(self, which, key_sreg):
        """Buffer resource for the tile of K ('k') or V ('v') starting at key key_sreg (< Lk):
        base at that key, records up to the last key (so rows past Lk read as zero)."""
        base, stride, r, key = (40, 44, RSK, KEYK) if which == "k" else (42, 45, RSV, KEYV)
        self.emit(f"s_mov_b32 {s(key)}, {s(key_sreg)}")
        self.emit(f"s_mul_i32 {s(SPAIR)}, {s(key_sreg)}, {s(stride)}")
        self.emit(f"s_mul_hi_u32 {s(SPAIR + 1)}, {s(key_sreg)}, {s(stride)}")
        self.emit(f"s_lshl_b64 {s(SPAIR, 2)}, {s(SPAIR, 2)}, 1")
        self.emit(f"s_add_u32 {s(r)}, {s(base)}, {s(SPAIR)}")
        self.emit(f"s_addc_u32 {s(r + 1)}, {s(base + 1)}, {s(SPAIR + 1)}")
        self.emit(f"s_and_b32 {s(r + 1)}, {s(r + 1)}, 0xffff")
        self.emit(f"s_sub_i32 {s(ST3)}, {s(46)}, {s(key_sreg)}")
        self.emit(f"s_min_i32 {s(ST3)}, {s(ST3)}, 64")
        self.emit(f"s_mul_i32 {s(r + 2)}, {s(ST3)}, {s(stride)}")
        self.emit(f"s_lshl_b32 {s(r + 2)}, {s(r + 2)}, 1")
        self.emit(f"s_mov_b32 {s(r + 3)}, {RSRC_FLAGS}")

    def advance_rsrc(self, which):
        """The resource moves on by one tile; past the last key it holds no records (its
        loads read zeros and fetch nothing)."""
        r, key, step, s2 = (RSK, KEYK, KSTEP, SK2) if which == "k" else (RSV, KEYV, VSTEP, SV2)
        self.emit(f"s_add_u32 {s(key)}, {s(key)}, 64")
        self.emit(f"s_add_u32 {s(r)}, {s(r)}, {s(step)}")
        self.emit(f"s_addc_u32 {s(r + 1)}, {s(r + 1)}, 0")
        self.emit(f"s_sub_i32 {s(ST3)}, {s(46)}, {s(key)}")
        self.emit(f"s_max_i32 {s(ST3)}, {s(ST3)}, 0")
        self.emit(f"s_min_i32 {s(ST3)}, {s(ST3)}, 64")
        self.emit(f"s_mul_i32 {s(r + 2)}, {s(ST3)}, {s(s2)}")

    def load_m0(self, n, buf):
        """M0 for load n (0..3) of this wave: the 1 KiB block (wave + 4 n) of LDS buffer buf."""
        self.emit(f"s_add_u32 m0, {s(SWB)}, {buf * TB + 4096 * n}")

    def load_issue(self, which, n):
        """16 bytes per lane of tile rows (wave + 4 n)*4 + lane/16 into the block at M0."""
        off, r = (KO, RSK) if which == "k" else (VO, RSV)
        self.emit(f"buffer_load_dwordx4 {v(off + n)}, {s(r, 4)}, 0 offen lds")

    def load(self, which, n, buf):
        self.load_m0(n, buf)
        self.emit("s_nop 0")
        self.load_issue(which, n)

    # ------------------------------------------------------------------ one phase
    def tail_ops(self, st, prev):
        """The part of the previous soft phase's pipeline that runs in this phase's first
        steps: exp2 of score 31, packing of pair 15, sums of 30 and 31, then l += the previous
        phase's row sums (and their running max)."""
        sx, px, et, lsub = prev
        keep = (self.et, self.lsub)
        self.et, self.lsub = et, lsub
        if st == 0:
            self.exp_elem(sx, 31)
            self.sum_elem(30)
        elif st == 1:
            self.cvt_pair(px, 15)
            self.sum_elem(31)
        elif st == 2 and lsub != L:
            for rb in range(RB):
                self.emit(f"v_add_f32 {v(L + rb)}, {v(L + rb)}, {v(lsub + rb)}")
        elif st == 3 and lsub != L and not self.bf16:
            for rb in range(RB):
                self.emit(f"v_max_f32 {v(LMX + rb)}, {v(LMX + rb)}, {v(lsub + rb)}")
        self.et, self.lsub = keep
    def phase(self, *, s_next, pv, soft, masked, track, maxonly, kofs, vofs, knofs, vnofs, dma, sx, sy, px, py,
              kt_sreg, tail=None, advance=(), direct=False):
        """Phase X(i): S(i+1) into sy (K at kofs), O += V^T py^T (V at vofs), mask / max /
        P of the scores sx of sub-tile i into px (first key kt_sreg); read-ahead of the next
        phase's first K and V fragments (knofs / vnofs, None: none); tile loads into the
        buffers dma = (K buffer, V buffer) or None.
        track: row maxima and the per-phase check; tail: the previous soft phase (its
        pipeline ends here); advance: groups of scalar instructions spread over the steps;
        direct: the row sums go straight into l (bf16, no rare path in this phase).
        Returns the state a later phase needs to finish this one's pipeline."""
        par = 0 if sx == S_X else 1
        self.et, self.lsub = ET + 4 * par, (LSUB, LSUB2)[par]
        if direct:
            # no rare path and no per-phase guard: the sums go straight into l
            self.lsub = L
        advance = list(advance)
        for st in range(NSTEP):
            is_s, idx, rb = st % 2 == 0, st // 4, (st // 2) % 2
            mark0 = len(self.out)
            dma_now = None
            if dma is not None and st % DMA_EVERY == 0 and st // DMA_EVERY < 8:
                n = st // DMA_EVERY
                if n < 4:
                    dma_now = ("k", n)
                    self.load_m0(n, dma[0])
                elif dma[1] is not None:
                    dma_now = ("v", n - 4)
                    self.load_m0(n - 4, dma[1])
            markr0 = len(self.out)
            if is_s:
                ks = idx
                markr1 = len(self.out)
                if s_next:
                    if rb == 0 and ks + PF < NKS:
                        self.read_k(kofs, ks + PF, (ks + PF) % 4, ("k", ks + PF))
                    markr1 = len(self.out)
                    if ks % 2 == 0 and rb == 0:
                        # one wait per two fragments (each wait takes an issue slot)
                        self.wait_for(("k", ks + 1))
                    if ks:
                        c = v(sy + 16 * rb, 16)
                    else:
                        c = "0" if self.mode == 2 else v(NMB + 16 * rb, 16)
                    self.mfma(v(sy + 16 * rb, 16), v(KF + 4 * (ks % 4), 4), a(128 + (rb * NKS + ks) * 4, 4), c)
                if knofs is not None and rb == 0 and ks >= NKS - PF:
                    g = ks - (NKS - PF)
                    self.read_k(knofs, g, g, ("kn", g))
                if dma_now is not None:
                    self.load_issue(*dma_now)
            else:
                f = idx
                markr1 = len(self.out)
                if pv:
                    if rb == 0 and f + PF < 2 * NDB:
                        self.read_v(vofs, f + PF, (f + PF) % 4, ("v", f + PF))
                    markr1 = len(self.out)
                    if f % 2 == 0 and rb == 0:
                        self.wait_for(("v", f + 1))
                    t, db = f // NDB, f % NDB
                    blk = a((rb * NDB + db) * 16, 16)
                    self.mfma(blk, v(VF + 4 * (f % 4), 4), v(py + (rb * 2 + t) * 4, 4), blk)
                if vnofs is not None and rb == 0 and f >= 2 * NDB - PF:
                    g = f - (2 * NDB - PF)
                    self.read_v(vnofs, g, g, ("vn", g))
            mark1 = len(self.out)
            if tail is not None:
                self.tail_ops(st, tail)
            if soft:
                if st == 0:
                    if track:
                        self.emit(f"v_mov_b32 {v(MXA)}, {v(VNINF)}")
                        self.emit(f"v_mov_b32 {v(MXA + 1)}, {v(VNINF)}")
                    if not maxonly and self.lsub != L:
                        self.emit(f"v_mov_b32 {v(self.lsub)}, 0")
                        self.emit(f"v_mov_b32 {v(self.lsub + 1)}, 0")
                    if masked:
                        self.emit(f"v_add_u32 {v(KBASE)}, {s(kt_sreg)}, {v(12)}")
                        self.emit(f"v_add_u32 {v(KBASE + 1)}, {s(kt_sreg)}, {v(13)}")
                if st == 0 and maxonly:
                    # without the products of V, the scores of the last steps are younger
                    self.emit("s_nop 4")
                # step g: mask score g (odd g: max of the pair); g+1: exp2; g+2: add to the
                # row sum; 2u+3: pack pair u. With a softcap, the exp2 of score g-1 and the
                # sum of g-2 (independent of score g) fill the two slots of the cap's chain.
                fill = []
                if not maxonly:
                    if st >= 1:
                        fill.append(lambda g=st - 1: self.exp_elem(sx, g))
                    if st >= 2:
                        fill.append(lambda g=st - 2: self.sum_elem(g))
                if self.mode == 2:
                    rr_, e_ = st // 16, st % 16
                    reg = sx + 16 * rr_ + e_
                    self.softcap_filled(reg, rr_, fill)
                    if masked:
                        self.mask(reg, reg, rr_, e_)
                else:
                    self.mask_elem(sx, st, masked)
                if track and st % 2 == 1:
                    self.max_pair(sx, st // 2)
                if not maxonly:
                    for f in fill:
                        f()
                    if st >= 3 and st % 2 == 1:
                        self.cvt_pair(px, (st - 3) // 2)
                    if track and st == 16:
                        self.emit(f"v_cmp_gt_f32_e64 {s(SCHK, 2)}, {v(MXA)}, {v(MT)}")
            if advance and 1 <= st <= 28:
                per = -(-len(advance) // (29 - st))
                for _ in range(per):
                    for line in advance.pop(0):
                        self.emit(line)
            # Order of a step: the fragment read-ahead first, then the step's vector and
            # scalar work, then the M0 write of a tile load, the wait, the product and the
            # rest. The reads get the most time to land and the wait comes as late as it
            # can (loop cycles per headline item 310.6K -> 282.1K against reads, wait and
            # product first, measured with timestamps).
            m0w, ra, rest = self.out[mark0:markr0], self.out[markr0:markr1], self.out[markr1:mark1]
            self.out[mark0:] = ra + self.out[mark1:] + m0w + rest
        assert not advance
        if soft and track and not maxonly:
            # any row max past its threshold (reference + slack, or a first unmasked key)?
            ret, rare = self.uniq("ret"), self.uniq("rare")
            self.emit(f"v_cmp_gt_f32_e64 {s(SMASK, 2)}, {v(MXA + 1)}, {v(MT + 1)}")
            self.emit(f"s_or_b64 {s(SMASK, 2)}, {s(SMASK, 2)}, {s(SCHK, 2)}")
            self.emit(f"s_cbranch_scc1 {rare}")
            self.emit(f"{ret}:")
            self.rare.append((rare, ret, sx, sy, px, self.et, self.lsub))
        if soft and maxonly:
            for rb in range(RB):
                self.emit(f"v_max_f32 {v(M + rb)}, {v(M + rb)}, {v(MXA + rb)}")
        return (sx, px, self.et, self.lsub)

    def thresholds(self):
        """From M: MU = reference (0 for a row without one); MT = threshold of the per-phase
        check on scores relative to MU (the slack; -inf without a reference, so that any
        unmasked key trips it); NMB = -MU, the start of the S products; CM (softcap)."""
        for rb in range(RB):
            self.emit(f"v_cmp_eq_f32 vcc, {v(VNINF)}, {v(M + rb)}")
            self.emit(f"v_cndmask_b32_e64 {v(MU + rb)}, {v(M + rb)}, 0, vcc")
            self.emit(f"v_mov_b32 {v(MT + rb)}, {self.slack_bits}")
            self.emit(f"v_cndmask_b32 {v(MT + rb)}, {v(MT + rb)}, {v(VNINF)}, vcc")
            if self.mode == 2:
                self.emit(f"v_sub_f32 {v(CM + rb)}, {s(51)}, {v(MU + rb)}")
            else:
                self.emit(f"v_sub_f32 {v(NMB + 16 * rb)}, 0, {v(MU + rb)}")
                for i in range(1, 16):
                    self.emit(f"v_mov_b32 {v(NMB + 16 * rb + i)}, {v(NMB + 16 * rb)}")

    def shift_scores(self, sbase):
        """Scores of a sub-tile relative to the new reference: minus DELTA (= MU - MUOLD)."""
        for g in range(32):
            r = self.score(sbase, g)
            self.emit(f"v_sub_f32 {v(r)}, {v(r)}, {v(DELTA + g // 16)}")

    def new_reference(self):
        """thresholds() after M changed, with DELTA = MU - MUOLD."""
        for rb in range(RB):
            self.emit(f"v_mov_b32 {v(MUOLD + rb)}, {v(MU + rb)}")
        self.thresholds()
        for rb in range(RB):
            self.emit(f"v_sub_f32 {v(DELTA + rb)}, {v(MU + rb)}, {v(MUOLD + rb)}")
    def flag_addr(self, dst):
        """LDS address of the redo flag (of this item's slot in the persistent form)."""
        self.emit(f"v_mov_b32 {v(dst)}, {FLAG}")
        self.emit(f"v_add_u32 {v(dst)}, {s(56)}, {v(dst)}")
        if self.persistent:
            self.emit(f"v_add_u32 {v(dst)}, {s(SK_FLAG)}, {v(dst)}")

    def set_flag(self):
        self.emit(f"v_mov_b32 {v(T0)}, 1")
        self.flag_addr(T1)
        self.emit(f"ds_write_b32 {v(T1)}, {v(T0)}")
        self.emit("s_waitcnt lgkmcnt(0)")

    def rare_block(self, rare, ret, sx, sy, px, et, lsub):
        """Out of line. Rows whose first unmasked keys arrived take the sub-tile max as their
        reference: the scores of this sub-tile and of the next one (already in sy) move to
        it and P so far is formed again; a row max past a finite reference by more than the
        slack sets the redo flag (and the checks are switched off for the pass)."""
        self.et, self.lsub = et, lsub
        no_risk, back = self.uniq("norisk"), self.uniq("back")
        self.emit(f"{rare}:")
        self.gap()  # the S products of the next sub-tile have just been issued
        self.exchange_max()
        self.emit(f"s_mov_b64 {s(SMASK, 2)}, 0")
        self.emit(f"s_mov_b64 {s(SMASK2, 2)}, 0")
        for rb in range(RB):
            self.emit(f"v_cmp_eq_f32 vcc, {v(VNINF)}, {v(M + rb)}")              # m == -inf
            self.emit(f"v_cmp_neq_f32_e64 {s(SPAIR, 2)}, {v(VNINF)}, {v(MXS + rb)}")
            self.emit(f"s_and_b64 {s(SPAIR, 2)}, {s(SPAIR, 2)}, vcc")            # first
            self.emit(f"s_or_b64 {s(SMASK, 2)}, {s(SMASK, 2)}, {s(SPAIR, 2)}")
            self.emit(f"v_cndmask_b32_e64 {v(M + rb)}, {v(M + rb)}, {v(MXS + rb)}, {s(SPAIR, 2)}")
            self.emit(f"v_mov_b32 {v(T1)}, {self.slack_bits}")
            self.emit(f"v_cmp_lt_f32_e64 {s(SPAIR, 2)}, {v(T1)}, {v(MXS + rb)}")
            self.emit(f"s_andn2_b64 {s(SPAIR, 2)}, {s(SPAIR, 2)}, vcc")          # risk (m was finite)
            self.emit(f"s_or_b64 {s(SMASK2, 2)}, {s(SMASK2, 2)}, {s(SPAIR, 2)}")
        self.emit(f"s_cmp_eq_u64 {s(SMASK2, 2)}, 0")
        self.emit(f"s_cbranch_scc1 {no_risk}")
        self.set_flag()
        # this pass will be run again: no more checks in it
        self.emit(f"v_mov_b32 {v(MT)}, 0x7f800000")
        self.emit(f"v_mov_b32 {v(MT + 1)}, 0x7f800000")
        self.emit(f"s_branch {back}")
        self.emit(f"{no_risk}:")
        self.emit(f"s_cmp_eq_u64 {s(SMASK, 2)}, 0")
        self.emit(f"s_cbranch_scc1 {back}")
        self.new_reference()
        self.shift_scores(sx)
        if self.mode != 2:
            self.shift_scores(sy)   # softcap: the next sub-tile is capped against CM later
        self.emit(f"v_mov_b32 {v(lsub)}, 0")
        self.emit(f"v_mov_b32 {v(lsub + 1)}, 0")
        # everything the pipeline did up to the last step, against the new reference
        for u in range(15):
            self.exp_unit(sx, px, u)
        self.exp_elem(sx, 30)
        self.emit("s_nop 0")
        self.emit(f"{back}:")
        self.emit(f"s_branch {ret}")
    # ------------------------------------------------------------------ a pass
    def advance_groups(self, exact, first):
        """Scalar work that prepares tile j+1 (first=False) or tile 0 (first=True): buffer
        resources of the loads made in its first phase, and which body it takes."""
        out = []

        def grab(fn):
            keep = self.out
            self.out = []
            fn()
            out.append(self.out)
            self.out = keep

        if not first:
            out.append([f"s_add_u32 {s(SJ)}, {s(SJ)}, 1", f"s_add_u32 {s(SKT)}, {s(SKT)}, 64"])
        grab(lambda: self.advance_rsrc("k"))
        if not exact:
            grab(lambda: self.advance_rsrc("v"))
            if self.mode >= 1:
                # plain iff every row has its reference already (kt > s57: a row's first
                # allowed key lies in an earlier tile) and no key of [kt, kt + 64) is masked
                out.append([f"s_add_i32 {s(ST)}, {s(SKT)}, 64",
                            f"s_cmp_le_i32 {s(ST)}, {s(58)}",
                            f"s_cselect_b32 {s(SUNM)}, 1, 0",
                            f"s_cmp_gt_i32 {s(SKT)}, {s(57)}",
                            f"s_cselect_b32 {s(SUNM)}, {s(SUNM)}, 0"])
        return out

    def tile_body(self, exact, c, plain, prev):
        """Both phases of a tile j with j % 3 == c (loads of K(j+2), V(j+1) in the first);
        the second prepares tile j+1."""
        c1, c2 = (c + 1) % 3, (c + 2) % 3
        masked = self.mode >= 1 and not plain
        track = exact or not plain
        # X(2j): S(2j+1) from K(j) rows 32..63; P(2j-1) V(j-1) rows 32..63
        st = self.phase(s_next=True, pv=not exact, soft=True, masked=masked, track=track, maxonly=exact,
                        kofs=kbuf(c, 1), vofs=kbuf(c2, 1), knofs=kbuf(c1, 0),
                        vnofs=None if exact else kbuf(c, 0), dma=(c2, None if exact else 3 + c1), sx=S_X, sy=S_Y, px=P_X,
                        py=P_Y, kt_sreg=SKT, tail=None if exact else prev,
                        direct=self.bf16 and plain and not exact)
        self.relabel()
        self.emit(f"s_add_u32 {s(SKT2)}, {s(SKT)}, 32")
        # X(2j+1): S(2j+2) from K(j+1) rows 0..31; P(2j) V(j) rows 0..31
        st = self.phase(s_next=True, pv=not exact, soft=True, masked=masked, track=track, maxonly=exact,
                        kofs=kbuf(c1, 0), vofs=kbuf(c, 0), knofs=kbuf(c1, 1),
                        vnofs=None if exact else kbuf(c, 1), dma=None, sx=S_Y, sy=S_X, px=P_Y, py=P_X,
                        kt_sreg=SKT2, tail=None if exact else st, advance=self.advance_groups(exact, False))
        self.relabel()
        return st

    def tile(self, exact, c, prev):
        """Tile j (j % 3 == c), in the body its scalar flag selects."""
        if self.mode == 0 or exact:
            return self.tile_body(exact, c, not exact, prev)
        tracked, end = self.uniq("tracked"), self.uniq("tiledone")
        self.emit(f"s_cmp_eq_u32 {s(SUNM)}, 0")
        self.emit(f"s_cbranch_scc1 {tracked}")
        start = list(self.lds)
        st = self.tile_body(exact, c, True, prev)
        self.emit(f"s_branch {end}")
        self.emit(f"{tracked}:")
        self.lds = start
        st2 = self.tile_body(exact, c, False, prev)
        assert st2 == st
        self.emit(f"{end}:")
        return st

    def zero_v5(self):
        """LDS V buffer 5 = 0: it stands for V(-1), read (times P = 0) in the first phase."""
        self.emit(f"v_mbcnt_lo_u32_b32 {v(T0)}, -1, 0")
        self.emit(f"v_mbcnt_hi_u32_b32 {v(T0)}, -1, {v(T0)}")
        self.emit(f"v_lshlrev_b32 {v(T0)}, 4, {v(T0)}")
        self.emit(f"s_lshl_b32 {s(ST)}, {s(53)}, 12")
        self.emit(f"s_add_u32 {s(ST)}, {s(ST)}, {s(56)}")
        self.emit(f"s_add_u32 {s(ST)}, {s(ST)}, {5 * TB}")
        self.emit(f"v_add_u32 {v(T0)}, {s(ST)}, {v(T0)}")
        for i in range(4):
            self.emit(f"ds_write_b128 {v(T0)}, {v(ZERO, 4)} offset:{i * 1024}")

    def prescale_q(self):
        """Q fragments (raw, in S_X..S_Y) pre-scaled (by the score scale in log2 units, or for
        the softcap by the argument factor of its exponential), rounded back to 16 bits, into
        the AGPRs they stay in."""
        e = self.emit
        qscale = v(VCAPK) if self.mode == 2 else s(49)
        for i in range(RB * NKS * 4):
            x = S_X + i
            if self.persistent:
                # the raw fragments arrived in a[QNEXT:]
                x = T3
                e(f"v_accvgpr_read_b32 {v(T3)}, {a(QNEXT + i)}")
            if self.bf16:
                e(f"v_lshlrev_b32 {v(T0)}, 16, {v(x)}")
                e(f"v_and_b32 {v(T1)}, 0xffff0000, {v(x)}")
            else:
                e(f"v_cvt_f32_f16 {v(T0)}, {v(x)}")
                e(f"v_lshrrev_b32 {v(T1)}, 16, {v(x)}")
                e(f"v_cvt_f32_f16 {v(T1)}, {v(T1)}")
            e(f"v_mul_f32 {v(T0)}, {qscale}, {v(T0)}")
            e(f"v_mul_f32 {v(T1)}, {qscale}, {v(T1)}")
            cvt = "v_cvt_pk_bf16_f32" if self.bf16 else "v_cvt_pk_f16_f32"
            e(f"{cvt} {v(T2)}, {v(T0)}, {v(T1)}")
            e(f"v_accvgpr_write_b32 {a(128 + i)}, {v(T2)}")

    def initial_loads(self):
        """K(0) -> buffer 0, V(0) -> buffer 3, K(min(1, n-1)) -> buffer 1."""
        self.rsrc("k", 47)
        for n in range(4):
            self.load("k", n, 0)
        self.rsrc("v", 47)
        for n in range(4):
            self.load("v", n, 3)
        # the resource is read when a load issues: K(1) follows without a wait
        self.advance_rsrc("k")
        for n in range(4):
            self.load("k", n, 1)

    def run_pass(self, exact, first=False):
        tag = "x" if exact else "n"
        self.emit(f"s_mov_b32 {s(SJ)}, 0")
        self.emit(f"s_mov_b32 {s(SKT)}, {s(47)}")
        if exact:
            self.rsrc("k", 47)
            for n in range(4):
                self.load("k", n, 0)
            self.advance_rsrc("k")
            for n in range(4):
                self.load("k", n, 1)
        else:
            if self.persistent:
                # the first attempt finds its first tiles issued at the item change; a second
                # attempt (after a redo) issues them here
                pre = self.uniq("preloaded")
                self.emit(f"s_cmp_eq_u32 {s(SATT)}, 0")
                self.emit(f"s_cbranch_scc1 {pre}")
                self.initial_loads()
                self.emit(f"{pre}:")
            else:
                self.initial_loads()
            self.zero_v5()
            for rb in range(RB):
                self.emit(f"v_mov_b32 {v(LMX + rb)}, 0")
        self.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
        if first:
            # the first attempt only: later ones find Q in the AGPRs already
            done = self.uniq("qready")
            self.emit(f"s_cmp_lg_u32 {s(SATT)}, 0")
            self.emit(f"s_cbranch_scc1 {done}")
            self.prescale_q()
            self.emit(f"{done}:")
        self.emit("s_barrier")
        if not exact:
            # P(-1) = 0, and the pipeline "tail" of sub-tile -1 produces zeros
            for r in range(P_Y, P_Y + 16):
                self.emit(f"v_mov_b32 {v(r)}, 0")
            self.emit(f"v_mov_b32 {v(ET + 6)}, 0")
            self.emit(f"v_mov_b32 {v(S_Y + 31)}, {v(VNINF)}")
            self.emit(f"v_mov_b32 {v(LSUB2)}, 0")
            self.emit(f"v_mov_b32 {v(LSUB2 + 1)}, 0")
        # phase I: S(0) from K(0) rows 0..31; read ahead K(0) rows 32..63 and V(-1) rows 32..63
        self.lds = []
        for g in range(PF):
            self.read_k(kbuf(0, 0), g, g, ("k", g))
        self.phase(s_next=True, pv=False, soft=False, masked=False, track=False, maxonly=exact,
                   kofs=kbuf(0, 0), vofs=None, knofs=kbuf(0, 1), vnofs=None if exact else kbuf(2, 1),
                   dma=None, sx=S_Y, sy=S_X, px=P_Y, py=P_X, kt_sreg=SKT,
                   advance=self.advance_groups(exact, True))
        self.relabel()
        prev = (S_Y, P_Y, ET + 4, LSUB2)
        if not exact:
            # reference max of each row from sub-tile 0 (kept when already larger)
            self.gap()
            self.emit(f"v_mov_b32 {v(MXA)}, {v(VNINF)}")
            self.emit(f"v_mov_b32 {v(MXA + 1)}, {v(VNINF)}")
            if self.mode >= 1:
                self.emit(f"v_add_u32 {v(KBASE)}, {s(SKT)}, {v(12)}")
                self.emit(f"v_add_u32 {v(KBASE + 1)}, {s(SKT)}, {v(13)}")
            for u in range(16):
                self.seed_max_unit(S_X, u, self.mode >= 1)
            self.exchange_max()
            # the sub-tile max is relative to the reference S(0) was formed against
            for rb in range(RB):
                self.emit(f"v_add_f32 {v(T0)}, {v(MXS + rb)}, {v(MU + rb)}")
                self.emit(f"v_max_f32 {v(M + rb)}, {v(M + rb)}, {v(T0)}")
            self.new_reference()
            if self.mode != 2:
                self.shift_scores(S_X)
        loop_state = list(self.lds)
        exits = []
        self.emit(f"L_{tag}tile_%=:")
        for c in range(3):
            assert self.lds == loop_state, (self.lds, loop_state)
            prev = self.tile(exact, c, prev)
            assert self.lds == loop_state, (self.lds, loop_state)
            self.emit("s_waitcnt vmcnt(0)")
            self.emit("s_barrier")
            if c < 2:
                lbl = self.uniq(f"{tag}exit")
                exits.append((lbl, c))
                self.emit(f"s_cmp_ge_u32 {s(SJ)}, {s(48)}")
                self.emit(f"s_cbranch_scc1 {lbl}")
            else:
                self.emit(f"s_cmp_lt_u32 {s(SJ)}, {s(48)}")
                self.emit(f"s_cbranch_scc1 L_{tag}tile_%=")
        done = self.uniq(f"{tag}passdone")
        if not exact:
            # last: P(2n-1) V(n-1) rows 32..63 (first fragments read ahead); the pipeline of
            # sub-tile 2n-1 ends here. V(n-1) sits in buffer 3 + (n-1) % 3.
            for lbl, c in [(None, 2)] + exits:
                if lbl is not None:
                    self.emit(f"{lbl}:")
                self.lds = list(loop_state)
                if self.persistent:
                    self.q_prefetch_next()
                self.phase(s_next=False, pv=True, soft=False, masked=False, track=False, maxonly=False,
                           kofs=None, vofs=kbuf(c, 1), knofs=None, vnofs=None, dma=None, sx=S_X, sy=S_Y,
                           px=P_X, py=P_Y, kt_sreg=SKT, tail=prev)
                self.emit(f"s_branch {done}")
            self.emit(f"{done}:")
            # fp16: a phase's row sums past the slack (P would not fit fp16); bf16: a row
            # sum past 2^100 or infinite (P may exceed the slack in bf16 freely, but O
            # must stay finite): the pass is run again
            ok = self.uniq("sumsok")
            chk = LMX if not self.bf16 else L
            self.emit(f"v_cmp_lt_f32 vcc, {self.sum_limit}, {v(chk)}")
            self.emit(f"s_mov_b64 {s(SMASK, 2)}, vcc")
            self.emit(f"v_cmp_lt_f32 vcc, {self.sum_limit}, {v(chk + 1)}")
            self.emit(f"s_or_b64 {s(SMASK, 2)}, {s(SMASK, 2)}, vcc")
            self.emit(f"s_cbranch_scc0 {ok}")
            self.set_flag()
            self.emit(f"{ok}:")
        else:
            for lbl, c in exits:
                self.emit(f"{lbl}:")
            # the halves of each row exchange their maxima
            self.emit(f"v_mov_b32 {v(MXA)}, {v(M)}")
            self.emit(f"v_mov_b32 {v(MXA + 1)}, {v(M + 1)}")
            self.exchange_max()
            for rb in range(RB):
                self.emit(f"v_mov_b32 {v(M + rb)}, {v(MXS + rb)}")
        self.emit("s_waitcnt lgkmcnt(0)")
        self.lds = []
        self.gap()

    # ------------------------------------------------------------------ persistent form
    def read_record(self, item_sreg):
        """RECV = the 16 dwords of the record of item s[item_sreg]."""
        e = self.emit
        e(f"s_lshl_b32 {s(ST)}, {s(item_sreg)}, 6")
        e(f"s_add_u32 {s(ST)}, {s(ST)}, {s(31)}")
        e(f"v_mov_b32 {v(T0)}, {s(ST)}")
        for i in range(4):
            e(f"ds_read_b128 {v(RECV + 4 * i, 4)}, {v(T0)} offset:{16 * i}")
        e("s_waitcnt lgkmcnt(0)")

    def rec_scalars(self, pairs):
        for dst, dw in pairs:
            self.emit(f"v_readfirstlane_b32 {s(dst)}, {v(RECV + dw)}")
        # an SGPR written by a vector instruction is read by memory instructions only after
        # 5 wait states
        self.emit("s_nop 4")

    def q_prefetch_next(self):
        """While this item's last products run: the raw Q fragments of the next item into
        a[QNEXT:] (first attempt only; nothing after the last item)."""
        e = self.emit
        skip = self.uniq("noqnext")
        e(f"s_cmp_lg_u32 {s(SATT)}, 0")
        e(f"s_cbranch_scc1 {skip}")
        e(f"s_add_u32 {s(ST2)}, {s(SK_ITEM)}, 1")
        e(f"s_cmp_ge_u32 {s(ST2)}, {s(30)}")
        e(f"s_cbranch_scc1 {skip}")
        self.read_record(ST2)
        # row of lane (rb, l32) = min(r0 + wave * 64 + 32 rb + l32, Lq - 1)
        e(f"v_add_u32 {v(T3)}, {v(RECV + 10)}, {v(249)}")
        e(f"v_add_u32 {v(T2)}, -1, {v(RECV + 11)}")
        e(f"v_lshlrev_b32 {v(T1)}, 4, {v(250)}")
        for rb in range(RB):
            e(f"v_add_u32 {v(T0)}, {32 * rb}, {v(T3)}")
            e(f"v_min_i32 {v(T0)}, {v(T0)}, {v(T2)}")
            e(f"v_mov_b32 {v(2 * rb)}, {v(RECV)}")
            e(f"v_mov_b32 {v(2 * rb + 1)}, {v(RECV + 1)}")
            e(f"v_mad_u64_u32 {v(2 * rb, 2)}, {s(SPAIR, 2)}, {v(T0)}, {s(34)}, {v(2 * rb, 2)}")
            e(f"v_add_co_u32 {v(2 * rb)}, vcc, {v(2 * rb)}, {v(T1)}")
            e(f"v_addc_co_u32 {v(2 * rb + 1)}, vcc, 0, {v(2 * rb + 1)}, vcc")
        for rb in range(RB):
            for ks in range(NKS):
                e(f"global_load_dwordx4 {a(QNEXT + (rb * NKS + ks) * 4, 4)}, {v(2 * rb, 2)}, off offset:{ks * 32}")
        e(f"{skip}:")

    def item_kv(self):
        """The record's K / V bases, Lk and first key into the stream's inputs."""
        self.rec_scalars(((40, 6), (41, 7), (42, 8), (43, 9), (46, 12), (47, 13)))

    def item_rest(self):
        """Everything else of the item in RECV: Lq, tiles, sink, the wave's unmasked key range
        and the per-lane rows, key ranges and O / LSE addresses (after the previous item's
        epilogue, which reads the old ones)."""
        e = self.emit
        self.rec_scalars(((54, 11), (48, 14), (52, 15), (ST2, 10)))
        # wave rows [w0, w0 + 64); delta = Lk - Lq
        e(f"s_lshl_b32 {s(ST)}, {s(53)}, 6")
        e(f"s_add_u32 {s(ST)}, {s(ST)}, {s(ST2)}")                 # w0
        e(f"s_sub_i32 {s(ST3)}, {s(46)}, {s(54)}")                  # delta
        # whi = causal ? max(0, min(Lk, w0 + delta + 1)) : Lk
        e(f"s_add_i32 {s(58)}, {s(ST)}, {s(ST3)}")
        e(f"s_add_i32 {s(58)}, {s(58)}, 1")
        e(f"s_min_i32 {s(58)}, {s(58)}, {s(46)}")
        e(f"s_max_i32 {s(58)}, {s(58)}, 0")
        e(f"s_cmp_eq_u32 {s(33)}, 0")
        e(f"s_cselect_b32 {s(58)}, {s(46)}, {s(58)}")
        # wlo = window ? max(0, min(w0 + 63, Lq - 1) + delta - window + 1) : 0
        e(f"s_add_i32 {s(57)}, {s(ST)}, 63")
        e(f"s_add_i32 {s(SPAIR)}, {s(54)}, -1")
        e(f"s_min_i32 {s(57)}, {s(57)}, {s(SPAIR)}")
        e(f"s_add_i32 {s(57)}, {s(57)}, {s(ST3)}")
        e(f"s_sub_i32 {s(57)}, {s(57)}, {s(32)}")
        e(f"s_add_i32 {s(57)}, {s(57)}, 1")
        e(f"s_max_i32 {s(57)}, {s(57)}, 0")
        e(f"s_cmp_gt_i32 {s(32)}, 0")
        e(f"s_cselect_b32 {s(57)}, {s(57)}, 0")
        # per lane: key_lo = window ? row + delta - window + 1 : 0;
        # key_hi = causal ? min(Lk, row + delta + 1) : Lk
        e(f"s_sub_i32 {s(ST)}, {s(ST3)}, {s(32)}")
        e(f"s_add_i32 {s(ST)}, {s(ST)}, 1")                          # delta - window + 1
        e(f"s_add_i32 {s(ST3)}, {s(ST3)}, 1")                        # delta + 1
        e(f"s_cmp_gt_i32 {s(32)}, 0")
        e(f"s_cselect_b64 {s(SMASK, 2)}, -1, 0")
        e(f"s_cmp_lg_u32 {s(33)}, 0")
        e(f"s_cselect_b64 {s(SMASK2, 2)}, -1, 0")
        e(f"v_add_u32 {v(16)}, {s(ST2)}, {v(249)}")
        e(f"v_add_u32 {v(17)}, 32, {v(16)}")
        for rb in range(RB):
            q = v(16 + rb)
            e(f"v_add_u32 {v(T0)}, {s(ST)}, {q}")
            e(f"v_cndmask_b32_e64 {v(T0)}, 0, {v(T0)}, {s(SMASK, 2)}")   # key_lo
            e(f"v_add_u32 {v(T1)}, {s(ST3)}, {q}")
            e(f"v_min_i32 {v(T1)}, {s(46)}, {v(T1)}")
            e(f"v_mov_b32 {v(T2)}, {s(46)}")
            e(f"v_cndmask_b32_e64 {v(T1)}, {v(T2)}, {v(T1)}, {s(SMASK2, 2)}")  # key_hi
            e(f"v_sub_u32 {v(T1)}, {v(T1)}, {v(T0)}")
            e(f"v_max_i32 {v(14 + rb)}, 0, {v(T1)}")                    # key_n
            e(f"v_lshlrev_b32 {v(T2)}, 2, {v(250)}")
            e(f"v_sub_u32 {v(12 + rb)}, {v(T2)}, {v(T0)}")              # 4 hi - key_lo
            # O row address: O base + row * O stride + 8 hi; LSE: LSE base + 4 row
            e(f"v_mov_b32 {v(4 + 2 * rb)}, {v(RECV + 2)}")
            e(f"v_mov_b32 {v(5 + 2 * rb)}, {v(RECV + 3)}")
            e(f"v_mad_u64_u32 {v(4 + 2 * rb, 2)}, {s(SPAIR, 2)}, {q}, {s(35)}, {v(4 + 2 * rb, 2)}")
            e(f"v_lshlrev_b32 {v(T2)}, 3, {v(250)}")
            e(f"v_add_co_u32 {v(4 + 2 * rb)}, vcc, {v(4 + 2 * rb)}, {v(T2)}")
            e(f"v_addc_co_u32 {v(5 + 2 * rb)}, vcc, 0, {v(5 + 2 * rb)}, vcc")
            e(f"v_mov_b32 {v(8 + 2 * rb)}, {v(RECV + 4)}")
            e(f"v_mov_b32 {v(9 + 2 * rb)}, {v(RECV + 5)}")
            e(f"v_mad_u64_u32 {v(8 + 2 * rb, 2)}, {s(SPAIR, 2)}, {q}, 4, {v(8 + 2 * rb, 2)}")

    def clear_flag(self):
        """Wave 0 sets this item's redo-flag slot to 0 (before the pass's first barrier)."""
        skip = self.uniq("noclear")
        self.emit(f"s_cmp_lg_u32 {s(53)}, 0")
        self.emit(f"s_cbranch_scc1 {skip}")
        self.flag_addr(T1)
        self.emit(f"ds_write_b32 {v(T1)}, {v(ZERO)}")
        self.emit("s_waitcnt lgkmcnt(0)")
        self.emit(f"{skip}:")

    def setup(self):
        """Constants of the stream: masks' -inf, softcap factors, LDS addresses, load offsets."""
        e = self.emit
        e(f"v_mov_b32 {v(VNINF)}, 0xff800000")
        e(f"v_mul_f32 {v(VM2C)}, -2.0, {s(51)}")
        e(f"v_mov_b32 {v(VCAPK)}, 0x4038aa3b")
        e(f"v_mul_f32 {v(VCAPK)}, {s(50)}, {v(VCAPK)}")
        e(f"s_lshl_b32 {s(SWB)}, {s(53)}, 10")
        e(f"s_add_u32 {s(SWB)}, {s(SWB)}, {s(56)}")
        e(f"s_lshl_b32 {s(SKROW)}, {s(44)}, 5")
        e(f"s_lshl_b32 {s(SVROW)}, {s(45)}, 5")
        e(f"s_lshl_b32 {s(SK2)}, {s(44)}, 1")
        e(f"s_lshl_b32 {s(SV2)}, {s(45)}, 1")
        e(f"s_lshl_b32 {s(KSTEP)}, {s(44)}, 7")
        e(f"s_lshl_b32 {s(VSTEP)}, {s(45)}, 7")
        # per-lane LDS read addresses (swizzle applied) and load offsets
        for ks in range(NKS):
            e(f"v_xor_b32 {v(KR + ks)}, {ks << 5}, {v(21)}")
            e(f"v_add_u32 {v(KR + ks)}, {s(56)}, {v(KR + ks)}")
        for db in range(NDB):
            e(f"v_xor_b32 {v(VR + db)}, {db << 6}, {v(22)}")
            e(f"v_add_u32 {v(VR + db)}, {s(56)}, {v(VR + db)}")
            e(f"v_add_u32 {v(VR + db)}, {3 * TB}, {v(VR + db)}")
        for n in range(4):
            e(f"s_mul_i32 {s(ST3)}, {s(SKROW)}, {n}")
            e(f"v_add_u32 {v(KO + n)}, {s(ST3)}, {v(19)}")
            e(f"s_mul_i32 {s(ST3)}, {s(SVROW)}, {n}")
            e(f"v_add_u32 {v(VO + n)}, {s(ST3)}, {v(20)}")
        for r in range(ZERO, ZERO + 4):
            e(f"v_mov_b32 {v(r)}, 0")

    def attempts(self):
        """One item: the pass, and if its check tripped, the exact row maxima and the pass
        again; ends with every wave past a barrier after the last pass."""
        e = self.emit
        e(f"s_mov_b32 {s(SATT)}, 0")
        for rb in range(RB):
            e(f"v_mov_b32 {v(M + rb)}, {v(VNINF)}")
        e("L_attempt_%=:")
        self.thresholds()
        for rb in range(RB):
            e(f"v_mov_b32 {v(L + rb)}, 0")
        e("s_nop 1")
        for blk in range(RB * NDB):
            self.mfma(a(blk * 16, 16), v(ZERO, 4), v(ZERO, 4), "0")
        self.run_pass(exact=False, first=True)
        # redo? (read after every wave has finished writing it)
        done = "L_done_%="
        e("s_barrier")
        e(f"s_cmp_lg_u32 {s(SATT)}, 0")
        e(f"s_cbranch_scc1 {done}")
        self.flag_addr(T1)
        e(f"ds_read_b32 {v(T0)}, {v(T1)}")
        e("s_waitcnt lgkmcnt(0)")
        e(f"v_readfirstlane_b32 {s(ST)}, {v(T0)}")
        e(f"s_cmp_eq_u32 {s(ST)}, 0")
        e(f"s_cbranch_scc1 {done}")
        # exact row max first, then the pass again against it
        e(f"s_mov_b32 {s(SATT)}, 1")
        for rb in range(RB):
            e(f"v_mov_b32 {v(M + rb)}, {v(VNINF)}")
        self.thresholds()
        self.run_pass(exact=True)
        e("s_barrier")
        e("s_branch L_attempt_%=")
        e(f"{done}:")

    def build_persistent(self):
        e = self.emit
        self.setup()
        e(f"s_mov_b32 {s(SK_ITEM)}, 0")
        e(f"s_mov_b32 {s(SK_FLAG)}, 0")
        # item 0: Q (raw) into a[QNEXT:], its first tiles, its per-lane values
        e(f"s_mov_b32 {s(SATT)}, 0")
        e(f"s_sub_u32 {s(SK_ITEM)}, 0, 1")
        self.q_prefetch_next()
        e(f"s_mov_b32 {s(SK_ITEM)}, 0")
        self.read_record(SK_ITEM)
        self.item_kv()
        self.initial_loads()
        self.item_rest()
        e("L_item_%=:")
        self.clear_flag()
        self.attempts()
        # every wave is past the barrier after this item's last LDS read: the next item's
        # first tiles go into the buffers now, ahead of this item's epilogue
        last = self.uniq("lastitem")
        e(f"s_add_u32 {s(ST2)}, {s(SK_ITEM)}, 1")
        e(f"s_cmp_ge_u32 {s(ST2)}, {s(30)}")
        e(f"s_cbranch_scc1 {last}")
        self.read_record(ST2)
        self.item_kv()
        self.initial_loads()
        e(f"{last}:")
        self.epilogue()
        e(f"s_add_u32 {s(SK_ITEM)}, {s(SK_ITEM)}, 1")
        e(f"s_cmp_ge_u32 {s(SK_ITEM)}, {s(30)}")
        e("s_cbranch_scc1 L_end_%=")
        self.item_rest()
        e(f"s_xor_b32 {s(SK_FLAG)}, {s(SK_FLAG)}, 4")
        e("s_branch L_item_%=")
        for blk in self.rare:
            self.rare_block(*blk)
        e("L_end_%=:")
        return self.out

    # ------------------------------------------------------------------ whole stream
    def build(self):
        e = self.emit
        self.setup()
        # Q fragments (raw; scaled into AGPRs once the first pass's tile loads are issued)
        for rb in range(RB):
            for ks in range(NKS):
                e(f"global_load_dwordx4 {v(S_X + (rb * NKS + ks) * 4, 4)}, {v(2 * rb, 2)}, off offset:{ks * 32}")
        # redo flag = 0 (wave 0), ordered before any write of 1 by the first barrier
        self.clear_flag()
        self.attempts()
        self.epilogue()
        e("s_branch L_end_%=")
        for blk in self.rare:
            self.rare_block(*blk)
        e("L_end_%=:")
        return self.out

    def epilogue(self):
        e = self.emit
        e(f"v_mov_b32 {v(T0)}, {v(L)}")
        e(f"v_mov_b32 {v(T1)}, {v(L)}")
        e(f"v_mov_b32 {v(T2)}, {v(L + 1)}")
        e(f"v_mov_b32 {v(T3)}, {v(L + 1)}")
        e("s_nop 1")
        e(f"v_permlane32_swap_b32 {v(T0)}, {v(T1)}")
        e(f"v_permlane32_swap_b32 {v(T2)}, {v(T3)}")
        e("s_nop 1")
        e(f"v_add_f32 {v(LT)}, {v(T0)}, {v(T1)}")
        e(f"v_add_f32 {v(LT + 1)}, {v(T2)}, {v(T3)}")
        for rb in range(RB):
            # The sink (s52: the head's sink logit in log2 units, -inf for none) joins the
            # denominator: M = max(MU, sink) (sink alone for a row with no allowed key),
            # l' = l 2^(MU - M) + 2^(sink - M), O = o 2^(MU - M) / l', LSE = M + log2 l'.
            # Without a sink M = MU, the factor is 2^0 = 1 and l' = l exactly.
            e(f"v_mov_b32 {v(T3)}, {s(52)}")
            e(f"v_max_f32 {v(T0)}, {v(T3)}, {v(MU + rb)}")
            e(f"v_cmp_lt_f32 vcc, 0, {v(LT + rb)}")
            e(f"v_cndmask_b32 {v(T0)}, {v(T3)}, {v(T0)}, vcc")
            e(f"v_sub_f32 {v(T1)}, {v(MU + rb)}, {v(T0)}")
            e(f"v_exp_f32 {v(T1)}, {v(T1)}")
            e(f"v_sub_f32 {v(T2)}, {v(T3)}, {v(T0)}")
            e(f"v_exp_f32 {v(T2)}, {v(T2)}")
            e("s_nop 0")
            e(f"v_cndmask_b32 {v(T1)}, 0, {v(T1)}, vcc")
            e(f"v_fma_f32 {v(LT + rb)}, {v(LT + rb)}, {v(T1)}, {v(T2)}")
            e(f"v_mov_b32 {v(MU + rb)}, {v(T0)}")
            # factor / l' (0 for a row with no weight at all)
            e(f"v_rcp_f32 {v(INV + rb)}, {v(LT + rb)}")
            e("s_nop 0")
            e(f"v_mul_f32 {v(INV + rb)}, {v(INV + rb)}, {v(T1)}")
            e(f"v_cmp_lt_f32 vcc, 0, {v(LT + rb)}")
            e(f"v_cndmask_b32 {v(INV + rb)}, 0, {v(INV + rb)}, vcc")
        for rb in range(RB):
            skip = self.uniq("nostore")
            e(f"v_cmp_gt_i32 vcc, {s(54)}, {v(16 + rb)}")
            e(f"s_and_saveexec_b64 {s(SEXEC, 2)}, vcc")
            e(f"s_cbranch_execz {skip}")
            for db in range(NDB):
                for g4 in range(4):
                    base = (rb * NDB + db) * 16 + g4 * 4
                    for k in range(4):
                        e(f"v_accvgpr_read_b32 {v(EP + k)}, {a(base + k)}")
                    for k in range(4):
                        e(f"v_mul_f32 {v(EP + k)}, {v(EP + k)}, {v(INV + rb)}")
                    cvt = "v_cvt_pk_bf16_f32" if self.bf16 else "v_cvt_pk_f16_f32"
                    e(f"{cvt} {v(EP + 4)}, {v(EP)}, {v(EP + 1)}")
                    e(f"{cvt} {v(EP + 5)}, {v(EP + 2)}, {v(EP + 3)}")
                    e(f"global_store_dwordx2 {v(4 + 2 * rb, 2)}, {v(EP + 4, 2)}, off offset:{db * 64 + g4 * 16}")
            e(f"{skip}:")
            e(f"s_mov_b64 exec, {s(SEXEC, 2)}")
        nolse = self.uniq("nolse")
        e(f"s_cmp_eq_u32 {s(55)}, 0")
        e(f"s_cbranch_scc1 {nolse}")
        for rb in range(RB):
            skip = self.uniq("nolserow")
            # LSE = ln2 (m + log2 l), -inf for a row with no allowed key; lanes 0..31 store
            e(f"v_log_f32 {v(T0)}, {v(LT + rb)}")
            e("s_nop 0")
            e(f"v_add_f32 {v(T0)}, {v(MU + rb)}, {v(T0)}")
            e(f"v_mul_f32 {v(T0)}, {LN2}, {v(T0)}")
            e(f"v_cmp_lt_f32 vcc, 0, {v(LT + rb)}")
            e(f"v_cndmask_b32 {v(T0)}, {v(VNINF)}, {v(T0)}, vcc")
            e(f"v_cmp_gt_i32 vcc, {s(54)}, {v(16 + rb)}")
            e(f"v_mbcnt_lo_u32_b32 {v(T1)}, -1, 0")
            e(f"v_mbcnt_hi_u32_b32 {v(T1)}, -1, {v(T1)}")
            e(f"v_cmp_gt_u32_e64 {s(SPAIR, 2)}, 32, {v(T1)}")
            e(f"s_and_b64 vcc, vcc, {s(SPAIR, 2)}")
            e(f"s_and_saveexec_b64 {s(SEXEC, 2)}, vcc")
            e(f"s_cbranch_execz {skip}")
            e(f"global_store_dword {v(8 + 2 * rb, 2)}, {v(T0)}, off")
            e(f"{skip}:")
            e(f"s_mov_b64 exec, {s(SEXEC, 2)}")
        e(f"{nolse}:")


def render(lines):
    return "\n".join('"' + ln + '\\n\\t"' for ln in lines) + "\n"


def clobbers(persistent=False):
    regs = [f'"v{i}"' for i in range(24, NVGPR)] + [f'"a{i}"' for i in range(256 if persistent else 192)]
    regs += [f'"s{i}"' for i in range(NSGPR_LO, NSGPR_HI)]
    if persistent:
        # the item's own inputs are computed inside the statement from the item table
        regs += [f'"v{i}"' for i in range(18)]
        regs += [f'"s{i}"' for i in (40, 41, 42, 43, 46, 47, 48, 52, 54, 57, 58, SK_ITEM, SK_FLAG)]
    # m0 is written for the LDS-DMA loads; exec is written around the row-masked stores and
    # restored before the statement ends
    regs += ['"vcc"', '"scc"', '"m0"', '"memory"']
    return ", ".join(regs)


def main(out_dir):
    os.makedirs(out_dir, exist_ok=True)
    for bf16 in (True, False):
        for mode in (0, 1, 2):
            for persistent in (False, True):
                g = Gen(bf16, mode, persistent)
                lines = g.build_persistent() if persistent else g.build()
                name = f"prefill_r2{'p' if persistent else ''}_{'bf16' if bf16 else 'f16'}_m{mode}.inc"
                with open(os.path.join(out_dir, name), "w") as f:
                    f.write(f"// generated by gen_prefill_r2.py: {len(lines)} lines\n")
                    f.write(render(lines))
    with open(os.path.join(out_dir, "prefill_r2_clobbers.inc"), "w") as f:
        f.write("// generated by gen_prefill_r2.py\n")
        f.write("#define ATTN_R2_CLOBBERS " + clobbers() + "\n")
        f.write("#define ATTN_R2P_CLOBBERS " + clobbers(True) + "\n")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else ".")
