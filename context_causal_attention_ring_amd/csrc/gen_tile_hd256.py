#!/usr/bin/env python3
"""Writes tile_hd256.inc: the instruction block of one 32-key tile of the
fused ring + current attention kernel at HD = 256 (a wave owns two 32-row
blocks; the accumulator O^T is 2 x 8 tiles of 32 x 32 fp32 in AGPRs).

Tiles run in pairs (K and V slots t mod 4).  One block, in order:
  1. S^T = K Q^T of tile v: 32 MFMAs.  The operands of the first two
     k-steps were read into KPRE ahead (by the block before, or before the
     loop), so the MFMAs start at once; the others are read from LDS two
     k-steps ahead; the first two V operands of the P.V below are read at
     the end.  Every two k-steps one LDS-DMA copy of the next tiles is
     issued (8 per block: the wave's rows of one K tile and one V tile), so
     the vector memory pipe drains them in the MFMAs' shadow rather than
     stalling the wave.  The walkers' step to the next tile (copy offsets,
     key bound, and the two counters the code around the block keeps:
     tiles before the next cut one, tiles before a region change) is scalar
     ops in the same shadow.
  2. Only when the tile is cut by a key bound (the first counter has run
     out): the tile's bound, then the scores of keys at or past each row's
     bound become -inf.
  3. O^T += V^T P^T of tile v-1: 32 MFMAs.  After each MFMA an even share
     (by issue cost) of tile v's online softmax is issued.  ASM blocks (bf16
     output): one FMA + exp2 per score against the running max as it
     stands, the row sums, their compensated fold (read from one register
     set, written to the other: even and odd tiles alternate), the bf16
     packing of the probabilities into the next P.V operands, and a test of
     each lane's tile sum against a bound.  F32 blocks (fp32 output): first
     the row max (two in-lane max3 chains, one v_permlane32_swap exchange
     with lane ^ 32) and the running-max vote, then the same sums; P.V takes
     each probability as two bf16 operands hi + lo (four MFMAs per step),
     packed late because the register file holds one hi/lo set.  The even
     tile of a pair reads the odd tile's KPRE here.
  4. ASM blocks, when a lane's tile sum passes its bound: if some
     probability may exceed 2^tau (the first tile; a row's max grew by more
     than tau) compute the tile's scores again from its K slot, mask them
     again, and run the F32 blocks' softmax (vote, rescale factors, exact
     new max where voted); either way treat the tile as significant: add
     the difference between its bf16-rounded and fp32 row sums to dq (the
     output is normalised by l + dq) and raise the bound.
  5. Odd tile only (the end of the pair): wait for this wave's copies, meet
     the other waves at the pair's barrier, and read the next pair's first
     KPRE, left in flight: the scalar code between blocks hides its latency.
The block is a single asm statement so that the softmax stays in the MFMAs'
shadow (as separate C++ it was sunk past the tile's barrier).  The scores
live in clobbered VGPRs v[204:235] and the operand ring in v[244:255]; both
are dead outside the block.

Hazards respected inside the block (gfx950): a VALU op never reads the
result of a transcendental in the next slot; two wait states between a VALU
write and v_permlane32_swap, and between an SGPR write and its use as a lane
mask; MFMA results are read by VALU only after a later MFMA and an s_nop;
a v_dot2 result is read by another VALU op only after DOT_WAIT wait states
(checked by check_dot_hazards on every block written).
Code after the block must leave the last MFMAs' operands alone for a while
(the compiler cannot see them); a CPU test checks the compiled kernel.

Usage: python gen_tile_hd256.py            (rewrites the .inc)
       python gen_tile_hd256.py --check    (exit 1 if the .inc is stale)
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "tile_hd256.inc")

NKS = 16           # 16-wide k-steps of QK^T (HD / 16)
NDB = 8            # 32-wide d blocks of the output (HD / 32)
NPS = 2            # 16-key steps of P.V per 32-key tile
NT = NPS * NDB     # P.V steps; each issues one MFMA per row block
NRB = 2            # 32-row blocks per wave
Q0 = 44            # Q^T operands (pinned): row block rb, k-step k -> v[Q0 + 64 rb + 4 k : +3]
PB = (172, 188)    # bf16 probabilities (pinned), two buffers: [rb][ks] -> v[PB + 8 rb + 4 ks : +3]
S0 = 204           # scores (clobbered): row block rb, key slot i -> v[S0 + 16 rb + i]
KPRE = 236         # K operands of k-steps 0 and 1 (pinned), read ahead: v[KPRE + 4 k : +3]
RING0 = 244        # operand ring (clobbered): group j -> v[RING0 + 4j : RING0 + 4j + 3]
KPRE_STEP = 2      # P.V step of an even tile after which the odd tile's KPRE is read

# READ_NOTE: an LDS read issued right behind an MFMA costs the wave little;
# issued after VALU work in an MFMA's shadow it stalls the next MFMA (a
# loop of MFMAs with one transposing V read and five VALU issue units each
# ran at 38 cycles per MFMA with the reads behind the MFMA, 43 with them
# after the VALU ops, on gfx950).  Every LDS read of the block goes out
# right behind an MFMA.

# Issue cost of one instruction, in units of one full-rate VALU op (measured
# on gfx950: v_exp_f32 is half rate; SALU and s_nop issue in about a cycle).
COST = {"valu": 1.0, "trans": 2.0, "dot": 2.0, "salu": 0.5, "nop": 0.5}


def grp(j, half=None):
    b = RING0 + 4 * (j % 3)
    if half is None:
        return f"v[{b}:{b + 3}]"
    return f"v[{b + 2 * half}:{b + 2 * half + 1}]"


def s(rb, i):
    return f"v{S0 + 16 * rb + i}"


def qop(rb, k):
    b = Q0 + 64 * rb + 4 * k
    return f"v[{b}:{b + 3}]"


def pbop(buf, rb, ks):
    b = PB[buf] + 8 * rb + 4 * ks
    return f"v[{b}:{b + 3}]"


def pbreg(buf, rb, j):
    """VGPR of pair j (keys 2j, 2j + 1) of row block rb in buffer buf."""
    return f"v{PB[buf] + 8 * rb + j}"


def stile(rb):
    return f"v[{S0 + 16 * rb}:{S0 + 16 * rb + 15}]"


# K step k uses ring group k % 3; V step t uses group (t + 1) % 3, so that
# the first two V operands can be read while the last K operands are in use.
def kgroup(k):
    return k % 3


def vgroup(t):
    return (t + 1) % 3


def kread(k):
    return f"ds_read_b128 {grp(kgroup(k))}, %[ka{k % 8}] offset:%[ko{k // 8}]"


def vreads(t):
    """Two transposing reads (keys 0-7 and 8-15 of the step) of V operand t."""
    ks, db = divmod(t, NDB)
    g = vgroup(t)
    return [f"ds_read_b64_tr_b16 {grp(g, h)}, %[va{db % 4}] offset:%[vo{ks}{db // 4}{h}]"
            for h in (0, 1)]


def kop(k):
    """K operand of k-step k: the first two were read ahead into KPRE."""
    return f"%[kp{k}]" if k < 2 else grp(kgroup(k))


def kpre_reads():
    """The first two K operands of the next tile, into KPRE (slot at kpo)."""
    return [f"ds_read_b128 %[kp{k}], %[ka{k}] offset:%[kpo]" for k in range(2)]


def dma_setup(i):
    """M0 (the LDS destination) and the scalar offset of copy i, set right
    after copy i - 1 went out (LDS-DMA reads M0 when issued, and needs one
    wait state after an SALU write of M0, which the k-steps in between
    give).  Copy i < 4 moves rows of a K tile, i >= 4 rows of a V tile.
    Instruction j = 2 a + b of wave w moves rows 2 w + 8 a + 16 b and the
    next one.  Rows 16 apart share their swizzle, so lane offset a
    (precomputed, %[d<kind>a] / %[d<kind>b]) serves both b; the 16 rows of
    b = 1 go into the scalar offset next to the tile's first byte."""
    kind, j = ("k", i) if i < 4 else ("v", i - 4)
    out = [f"s_add_u32 m0, %[m0b], %[m{kind}{j}]"]
    if j & 1:
        out.append(f"s_add_u32 %[st], %[off{kind}], %[rs16]")
    return out


def dma_issue(i):
    """Copy i (see dma_setup): 16 bytes per lane into LDS at M0."""
    kind, j = ("k", i) if i < 4 else ("v", i - 4)
    a, b = j >> 1, j & 1
    soff = "%[st]" if b else f"%[off{kind}]"
    return [f"buffer_load_dwordx4 %[d{kind}{'b' if a else 'a'}], %[desc{kind}], {soff} offen lds"]


def walk_ops():
    """The tile's scalar bookkeeping, one group in the shadow of the QK^T
    MFMAs: the bound walker's key bound wlim moves on to the next tile by
    dlim (-32 in a shard visit, +32 in the current tiles); nm, the tiles
    left before the next one a key bound cuts (set by the code around the
    block whenever the bound walker enters a region), and tn, the tiles left
    before some walker enters its next region, drop by one.  This tile is
    cut when nm has gone negative (mask_test); the code after the block
    takes the walkers into their next regions when tn reaches 0.  The copy
    offsets move on after the block's last copy (copy_step_ops)."""
    return ["s_add_i32 %[wlim], %[wlim], %[dlim]", "s_sub_i32 %[nm], %[nm], 1",
            "s_sub_u32 %[tn], %[tn], 1"]


def mask_test(label):
    """Branch to label when a key bound cuts this tile (after walk_ops)."""
    return ["s_cmp_lt_i32 %[nm], 0", f"s_cbranch_scc1 {label}"]


def bound_ops():
    """The cut tile's key bound, all scalar, on the mask's own path (wlim
    has already moved on by dlim): lm = 1 for the current tiles (region wk
    >= P), lc = the bound, wt = this tile's wlim: lc = wt in a visit (keys
    left), 1 - wt for the current tiles (wt = the tile's first position),
    -32 past the walk (vv >= tt, with lm = 0: every key masked)."""
    return ["s_sub_i32 %[wt], %[wlim], %[dlim]",
            "s_cmp_ge_i32 %[wk], %[np]", "s_cselect_b32 %[lm], 1, 0",
            "s_sub_i32 %[lc], 1, %[wt]",
            "s_cmp_eq_u32 %[lm], 0", "s_cselect_b32 %[lc], %[wt], %[lc]",
            "s_cmp_ge_i32 %[vv], %[tt]", "s_cselect_b32 %[lm], 0, %[lm]",
            "s_cselect_b32 %[lc], -32, %[lc]"]


def copy_step_ops():
    """After the block's last copy: the K and V copy walkers' tile offsets
    move on by one tile."""
    return ["s_add_u32 %[offk], %[offk], %[tstr]", "s_add_u32 %[offv], %[offv], %[tstr]"]


def qk_part(extra=()):
    """S^T = K Q^T with the block's copies and scalar bookkeeping; `extra`
    VALU ops (independent of the scores) are spread over the k-steps, two
    per step."""
    # KPRE was read by the block before (or before the loop): wait for it.
    out = ["s_nop 1", "s_waitcnt lgkmcnt(0)"] + dma_setup(0)
    extra = list(extra)
    per = -(-len(extra) // NKS) if extra else 0
    pending = []  # LDS reads in flight, in issue order
    for k in range(NKS):
        if k >= 2:  # this step's K operand (read two steps ahead) must be in
            out.append(f"s_waitcnt lgkmcnt({len(pending) - 1 - pending.index(k)})")
            pending = pending[pending.index(k) + 1:]
        for rb in range(NRB):
            c = "0" if k == 0 else stile(rb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {stile(rb)}, {kop(k)}, {qop(rb, k)}, {c}")
            if rb == 0:  # LDS reads go out right behind an MFMA (see READ_NOTE)
                if k + 2 < NKS:
                    out.append(kread(k + 2))
                    pending.append(k + 2)
                else:
                    out += vreads(k + 2 - NKS)
                    pending += ["v", "v"]
        if k % 2 == 1:  # one copy of the next tiles per two k-steps
            out += dma_issue(k // 2)
            if k == NKS - 1:
                out += copy_step_ops()
            else:
                out += dma_setup(k // 2 + 1)
        elif k == 0:  # the walkers' scalar step
            out += walk_ops()
        out += extra[k * per:(k + 1) * per]
    return out


SIG_SHIFT = -4  # a tile is significant when its sum exceeds 2^SIG_SHIFT of the running sum


def sig_ops(buf):
    """bf16 output, a significant tile (a lane's tile sum r is above its
    bound: 2^SIG_SHIFT of the lane's running sum, at most 2^tau): the
    tile's bf16-rounded probabilities (buffer buf, just packed) are summed
    (one v_dot2 against (1, 1) per pair of keys) and their difference from
    the fp32 tile sum r is added to dq.  The output is normalised by
    l + dq, so for every significant tile numerator and denominator weight
    each key identically; each other tile holds at most 2^SIG_SHIFT of the
    row's weight, so the bf16 rounding of its weights (2^-9 each, random
    sign) moves the output little.  Then bnd = min(2^SIG_SHIFT l, 2^tau).
    The bound only grows in the common path (l does), so a stale bound is
    conservative.  a and b are scratch.  A v_dot2 result is read by another
    VALU instruction only after DOT_WAIT more instructions (the hardware
    does not wait for it): the bound update and an s_nop sit between."""
    chains = []
    for rb in range(NRB):
        st = [f"v_dot2_f32_bf16 %[b{rb}], {pbreg(buf, rb, 0)}, %[one2], 0"]
        st += [f"v_dot2_f32_bf16 %[b{rb}], {pbreg(buf, rb, j)}, %[one2], %[b{rb}]"
               for j in range(1, 8)]
        chains.append(st)
    out = [op for pair in zip(*chains) for op in pair]
    out += [f"v_ldexp_f32 %[a{rb}], %[lo{rb}], {SIG_SHIFT}" for rb in range(NRB)]
    out += [f"v_min_f32 %[bnd{rb}], %[pbnd], %[a{rb}]" for rb in range(NRB)]
    out += [f"s_nop {DOT_WAIT - 1}"]
    out += [f"v_sub_f32 %[b{rb}], %[b{rb}], %[r{rb}]" for rb in range(NRB)]
    out += [f"v_add_f32 %[dq{rb}], %[dq{rb}], %[b{rb}]" for rb in range(NRB)]
    return out


# Wait states after a v_dot2 writes a VGPR before another (non-dot) VALU
# instruction may read it; back-to-back v_dot2 accumulating into the same
# register are forwarded.
DOT_WAIT = 4


SCC_READERS = ("s_cselect", "s_cbranch_scc", "s_cmov", "s_addc", "s_subb")
SCC_WRITERS = ("s_cmp", "s_add_", "s_sub_", "s_and_", "s_or_", "s_xor_", "s_min_", "s_max_",
               "s_lshl", "s_lshr", "s_ashr", "s_bfe", "s_not", "s_abs", "s_andn2", "s_orn2",
               "s_nand", "s_nor", "s_xnor", "s_bcnt", "s_absdiff", "s_addc", "s_subb")


def check_scc(lines):
    """Raise unless every instruction that reads SCC finds, as the nearest
    SCC writer before it (a label ends the search: a branch target starts
    its own sequence), a compare: no scalar op placed between a compare and
    its selects (the copies' M0 setup, the walkers' step) may clobber SCC."""
    last = None
    for ln in lines:
        op = ln.split(None, 1)[0] if ln.strip() else ""
        if op.endswith(":"):
            last = None
            continue
        if op.startswith(SCC_READERS) and last is not None and not last.startswith("s_cmp"):
            raise AssertionError(f"{ln!r} reads SCC last written by {last!r}")
        if op.startswith(SCC_WRITERS):
            last = ln


def scc_atomic(ops):
    """Merge each SALU compare with the ops that read its SCC into one op
    (lines joined by newlines), so that spreading the ops over MFMA gaps
    never puts a gap's scalar ops between them; emit with split_ops."""
    out = []
    for kind, text in ops:
        if out and text.startswith(SCC_READERS) and out[-1][1].split("\n")[0].startswith("s_cmp"):
            out[-1] = (out[-1][0], out[-1][1] + "\n" + text)
        else:
            out.append((kind, text))
    return out


def split_ops(texts):
    """The lines of a gap's ops (undoing scc_atomic's joins)."""
    return [ln for text in texts for ln in text.split("\n")]


def check_dot_hazards(lines):
    """Raise if an instruction other than v_dot2 reads a VGPR a v_dot2
    wrote fewer than DOT_WAIT wait states before (s_nop n counts n + 1;
    labels and branches end the window)."""
    import re
    pending = []  # (register text, wait states since the write)
    for ln in lines:
        op = ln.split(None, 1)[0] if ln.strip() else ""
        if op.endswith(":") or op.startswith(("s_branch", "s_cbranch")):
            pending = []
            continue
        args = ln.split(None, 1)[1] if " " in ln else ""
        dst, srcs = (args.split(",", 1) + [""])[:2] if args else ("", "")
        if not op.startswith("v_dot2"):
            for reg, _ in pending:
                if re.search(re.escape(reg) + r"(?![\w\]])", srcs if op.startswith("v_") else args):
                    raise AssertionError(f"{ln!r} reads {reg} too soon after a v_dot2")
        n = int(args) + 1 if op == "s_nop" else 1
        pending = [(r, w + n) for r, w in pending if w + n < DOT_WAIT]
        if op.startswith("v_dot2"):
            pending = [(r, w) for r, w in pending if r != dst.strip()] + [(dst.strip(), 0)]


def pack_f32(rb, j, direct, src=s):
    """fp32 output: split the probabilities of keys 2j, 2j + 1 of row block
    rb into hi = the bf16 truncation (exact: the upper half of the fp32
    word) and lo = bf16(p - hi), so that hi + lo holds p to about 2^-16
    relative and the P.V MFMAs on both carry no bf16 rounding of the
    weights.  direct: write the hi and lo operands at once (their buffer is
    no longer read); else leave hi packed in the odd score register and lo
    in the even one for a later move (src: the score registers).  a0 and b0
    are scratch."""
    i0, i1 = src(rb, 2 * j), src(rb, 2 * j + 1)
    hi, lo = (pbreg(0, rb, j), pbreg(1, rb, j)) if direct else (i1, i0)
    return [("valu", f"v_and_b32 %[a0], %[hmask], {i0}"),
            ("valu", f"v_and_b32 %[b0], %[hmask], {i1}"),
            ("valu", f"v_sub_f32 {i0}, {i0}, %[a0]"),
            ("valu", f"v_sub_f32 {i1}, {i1}, %[b0]"),
            ("valu", f"v_cvt_pk_bf16_f32 {lo}, {i0}, {i1}"),
            ("valu", f"v_perm_b32 {hi}, %[b0], %[a0], %[psel]")]


def mask_part(src=s):
    """Keys at or past the row's bound -> -inf, only on a cut tile (the cut
    counter nm has run below 0; src: the score registers, (rb, i) -> name).
    The bound of row block rb is lc (a visit's keys left, lm = 0) or
    pos_rb + lc (current tiles, lm = 1: lc = 1 - first key's position).
    Lane half h holds keys 8 (i / 4) + 4 h + i % 4 of the tile; with lim =
    bound - 4 h, key slot i is kept iff 8 (i / 4) + i % 4 < lim."""
    return ["s_cmp_ge_i32 %[nm], 0", "s_cbranch_scc1 1f"] + mask_body(src) + ["1:"]


def mask_body(src=s):
    """mask_part without its test: the tile's bound (bound_ops), the per-row
    bounds, then the compares."""
    out = bound_ops()
    out += ["v_mbcnt_lo_u32_b32 %[a0], -1, 0", "v_mbcnt_hi_u32_b32 %[a0], -1, %[a0]",
           "v_lshrrev_b32 %[a0], 5, %[a0]", "v_lshlrev_b32 %[a0], 2, %[a0]",  # 4 h
           "s_cmp_eq_u32 %[lm], 0", "s_cbranch_scc0 2f"]
    out += [f"v_sub_u32 %[th{rb}], %[lc], %[a0]" for rb in range(NRB)] + ["s_branch 3f", "2:"]
    out += [f"v_sub_u32 %[th{rb}], %[pos{rb}], %[a0]" for rb in range(NRB)]
    out += [f"v_add_u32 %[th{rb}], %[lc], %[th{rb}]" for rb in range(NRB)]
    out += ["3:", "s_nop 7", "s_nop 7"]
    for rb in range(NRB):
        for i in range(16):
            c = 8 * (i // 4) + i % 4
            out.append(f"v_sub_u32 %[a0], {c}, %[th{rb}]")    # < 0 iff kept
            out.append("v_ashrrev_i32 %[a0], 31, %[a0]")      # all ones iff kept
            out.append(f"v_bfi_b32 {src(rb, i)}, %[a0], {src(rb, i)}, %[ninf]")
    return out


def softmax_ops(pout, pack=True, src=s):
    """The online softmax of tile v as (kind, text) in dependency order
    (pack: the bf16 packing of the probabilities into buffer pout; src: the
    score registers, (rb, i) -> name, overwritten by the probabilities)."""
    ops = [("nop", "s_nop 4")]  # the last score MFMAs' results (after one more MFMA)
    for rb in range(NRB):  # threshold for the lazy rescale: mlog + tau
        ops.append(("valu", f"v_add_f32 %[th{rb}], %[tau], %[ml{rb}]"))
    # In-lane max of the 16 scores of each row: two max3 chains per row block.
    chains = [((0, 1, 2), (3, 4, 5)), ((6, 7), (8, 9)), ((10, 11), (12, 13)), ((14, 15), None)]
    for ca, cb in chains:
        for rb in range(NRB):
            for name, c in (("a", ca), ("b", cb)):
                if c is None:
                    continue
                regs = [src(rb, i) for i in c]
                if len(c) == 2:
                    regs = [f"%[{name}{rb}]"] + regs
                ops.append(("valu", f"v_max3_f32 %[{name}{rb}], {', '.join(regs)}"))
    # The two halves of a row live in lanes l and l ^ 32: the in-lane max
    # goes into both swap operands, the halves are exchanged, max taken.
    for rb in range(NRB):
        ops.append(("valu", f"v_max_f32 %[b{rb}], %[a{rb}], %[b{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_mov_b32 %[a{rb}], %[b{rb}]"))
    ops.append(("nop", "s_nop 1"))
    for rb in range(NRB):
        ops.append(("valu", f"v_permlane32_swap_b32 %[a{rb}], %[b{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_max_f32 %[a{rb}], %[a{rb}], %[b{rb}]"))
    for rb in range(NRB):  # to log2 units; the scale is positive, so max commutes
        ops.append(("valu", f"v_mul_f32 %[a{rb}], %[c2], %[a{rb}]"))
    # Lazy running max: rows whose max grew by more than tau vote; if any row
    # of the block voted, every row of it takes the exact new max.
    for rb in range(NRB):
        ops.append(("valu", f"v_cmp_gt_f32_e64 %[c{rb}], %[a{rb}], %[th{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_max_f32 %[b{rb}], %[ml{rb}], %[a{rb}]"))
    # c{rb}: all ones if some row of the block voted; bit rb of resc the same
    for rb in range(NRB):
        ops.append(("salu", f"s_cmp_lg_u64 %[c{rb}], 0"))
        ops.append(("salu", f"s_cselect_b64 %[c{rb}], -1, 0"))
        ops.append(("salu", f"s_cselect_b32 %[v{rb}], {1 << rb}, 0"))
    ops.append(("salu", "s_or_b32 %[resc], %[v0], %[v1]"))
    ops.append(("nop", "s_nop 1"))
    for rb in range(NRB):  # m_new
        ops.append(("valu", f"v_cndmask_b32_e64 %[b{rb}], %[ml{rb}], %[b{rb}], %[c{rb}]"))
    # the running max starts at -FLT_MAX (finite), so m_new is finite and a
    # row that has seen only masked keys gets exp2(-inf) = 0
    for rb in range(NRB):
        ops.append(("valu", f"v_mov_b32 %[a{rb}], %[b{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_sub_f32 %[al{rb}], %[ml{rb}], %[a{rb}]"))
    for rb in range(NRB):
        ops.append(("trans", f"v_exp_f32 %[al{rb}], %[al{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_mov_b32 %[ml{rb}], %[b{rb}]"))
    # One FMA + exp2 per score; each probability is added to the tile's row
    # sum r after the next FMA (a transcendental's result is not read in the
    # next slot), and each pair of keys is packed to bf16 once both are
    # summed.  The tile sum is formed first and then folded into l (below):
    # added one by one to the running sum, the many tiny probabilities of a
    # peaky row would be rounded away against it.
    streams = []
    for rb in range(NRB):
        st = []
        for i in range(16):
            st.append(("valu", f"v_fma_f32 {src(rb, i)}, {src(rb, i)}, %[c2], -%[a{rb}]"))
            if i == 2:
                st.append(("valu", f"v_add_f32 %[r{rb}], {src(rb, 0)}, {src(rb, 1)}"))
            elif i > 2:
                st.append(("valu", f"v_add_f32 %[r{rb}], %[r{rb}], {src(rb, i - 1)}"))
            if pack and i >= 2 and i % 2 == 0:
                j = i // 2 - 1
                st.append(("valu", f"v_cvt_pk_bf16_f32 {pbreg(pout, rb, j)}, {src(rb, 2 * j)}, "
                                   f"{src(rb, 2 * j + 1)}"))
            st.append(("trans", f"v_exp_f32 {src(rb, i)}, {src(rb, i)}"))
        streams.append(st)
    for k in range(max(len(x) for x in streams)):
        for st in streams:
            if k < len(st):
                ops.append(st[k])
    for rb in range(NRB):
        ops.append(("valu", f"v_add_f32 %[r{rb}], %[r{rb}], {src(rb, 15)}"))
    # l = l * alpha + r, compensated (Kahan): lk keeps what the rounding of
    # each fold dropped, so millions of tiny tile sums do not drift.  The
    # sums are read from li / lki and written to lo / lko (two register
    # sets used by even and odd tiles in turn), so a slow path finds the
    # sums before this tile's fold untouched.
    for rb in range(NRB):
        ops.append(("valu", f"v_mul_f32 %[a{rb}], %[li{rb}], %[al{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_fma_f32 %[b{rb}], -%[lki{rb}], %[al{rb}], %[r{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_add_f32 %[lo{rb}], %[a{rb}], %[b{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_sub_f32 %[lko{rb}], %[lo{rb}], %[a{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_sub_f32 %[lko{rb}], %[lko{rb}], %[b{rb}]"))
    if pack:
        for rb in range(NRB):
            ops.append(("valu", f"v_cvt_pk_bf16_f32 {pbreg(pout, rb, 7)}, {src(rb, 14)}, "
                                f"{src(rb, 15)}"))
    return ops


def softmax_ops_stale(pout, src=s, dst=s):
    """The common case of tile v's online softmax (bf16 output): every score
    is taken against the running max as it stands (it starts at -FLT_MAX,
    so a row that has seen no key gets +inf probabilities and the slow
    path), the tile's row sums r and the bf16 packing as in softmax_ops,
    and lo = li + r compensated (alpha = 1).  Valid while every
    probability is at most 2^tau, which r <= 2^tau (pbnd) proves: otherwise
    (a row's max grew by more than tau, or the first tile) the block's
    slow path recomputes the tile with softmax_ops, from li as it was.
    src holds the scores, dst gets the probabilities ((rb, i) -> name); with
    dst = src they replace the scores."""
    ops = [("nop", "s_nop 4"), ("salu", "s_mov_b32 %[resc], 0")]
    streams = []
    for rb in range(NRB):
        st = []
        for i in range(16):
            st.append(("valu", f"v_fma_f32 {dst(rb, i)}, {src(rb, i)}, %[c2], -%[ml{rb}]"))
            if i == 2:
                st.append(("valu", f"v_add_f32 %[r{rb}], {dst(rb, 0)}, {dst(rb, 1)}"))
            elif i > 2:
                st.append(("valu", f"v_add_f32 %[r{rb}], %[r{rb}], {dst(rb, i - 1)}"))
            if i >= 2 and i % 2 == 0:
                j = i // 2 - 1
                st.append(("valu", f"v_cvt_pk_bf16_f32 {pbreg(pout, rb, j)}, {dst(rb, 2 * j)}, "
                                   f"{dst(rb, 2 * j + 1)}"))
            st.append(("trans", f"v_exp_f32 {dst(rb, i)}, {dst(rb, i)}"))
        streams.append(st)
    main = []
    for k in range(max(len(x) for x in streams)):
        for st in streams:
            if k < len(st):
                main.append(st[k])
    ops += main
    for rb in range(NRB):
        ops.append(("valu", f"v_add_f32 %[r{rb}], %[r{rb}], {dst(rb, 15)}"))
    for rb in range(NRB):  # y = r - lki; lo = li + y; lko = (lo - li) - y
        ops.append(("valu", f"v_sub_f32 %[a{rb}], %[r{rb}], %[lki{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_add_f32 %[lo{rb}], %[li{rb}], %[a{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_sub_f32 %[lko{rb}], %[lo{rb}], %[li{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_sub_f32 %[lko{rb}], %[lko{rb}], %[a{rb}]"))
    for rb in range(NRB):
        ops.append(("valu", f"v_cvt_pk_bf16_f32 {pbreg(pout, rb, 7)}, {dst(rb, 14)}, {dst(rb, 15)}"))
    # some probability of the lane may exceed 2^tau, or the tile is
    # significant: bnd <= 2^tau (see sig_ops)
    for rb in range(NRB):
        ops.append(("valu", f"v_cmp_gt_f32_e64 %[c{rb}], %[r{rb}], %[bnd{rb}]"))
    ops.append(("salu", "s_or_b64 %[any], %[c0], %[c1]"))
    return ops


def qk_again():
    """S^T = K Q^T of this tile once more, every K operand read from LDS
    (the slow path; the ring's last readers, P.V MFMAs, are long done)."""
    out = [kread(0), kread(1)]
    for k in range(NKS):
        if k + 2 < NKS:
            out.append(kread(k + 2))
        out.append(f"s_waitcnt lgkmcnt({min(2, NKS - 1 - k)})")
        for rb in range(NRB):
            c = "0" if k == 0 else stile(rb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {stile(rb)}, {grp(kgroup(k))}, {qop(rb, k)}, {c}")
    return out + ["s_nop 15", "s_nop 15"]  # the scores are read by VALU next


def assign(ops, ngaps, weights=None):
    """Split the ops into ngaps consecutive groups of even cumulative cost
    (or of cost in proportion to weights, one per gap)."""
    total = sum(COST[k] for k, _ in ops)
    per = total / ngaps
    w = weights or [1.0] * ngaps
    bounds, run = [], 0.0
    for x in w:  # cumulative cost at the end of each gap
        run += x
        bounds.append(total * run / sum(w))
    gaps = [[] for _ in range(ngaps)]
    acc, g = 0.0, 0
    for kind, text in ops:
        while g < ngaps - 1 and acc + COST[kind] / 2 > bounds[g]:
            g += 1
        gaps[g].append(text)
        acc += COST[kind]
    return gaps, per


def pv_part(pin, lazy=True):
    """P.V of the previous tile with this tile's softmax.  Variant P1 is the
    even tile of a pair: it reads the odd tile's KPRE at step KPRE_STEP
    (that K landed before the previous pair's barrier).  Variant P0, the odd
    tile, ends the pair: wait for this wave's copies, meet the other waves
    at the barrier, then read the next pair's first KPRE, left in flight
    for the next block to wait on."""
    even = pin == 1
    ops = softmax_ops_stale(1 - pin) if lazy else softmax_ops(1 - pin)
    gaps, per = assign(ops, NRB * NT)
    out = []
    for t in range(NT):
        ks, db = divmod(t, NDB)
        wait = 2 if t + 1 < NT else 0
        if even and t == KPRE_STEP + 1:  # the KPRE reads went out before step t+1's V reads
            wait = 4
        out.append(f"s_waitcnt lgkmcnt({wait})")
        for rb in range(NRB):
            out.append(f"v_mfma_f32_32x32x16_bf16 %[acc{rb}{db}], {grp(vgroup(t))}, "
                       f"{pbop(pin, rb, ks)}, %[acc{rb}{db}]")
            if rb == 0:  # LDS reads right behind the MFMA, before the VALU ops
                if even and t == KPRE_STEP:
                    out += kpre_reads()
                if t + 2 < NT:
                    out += vreads(t + 2)
            out += gaps[NRB * t + rb]
    tail = [] if even else ["s_waitcnt vmcnt(0)", "s_barrier"] + kpre_reads()
    if not lazy:
        return out + tail, per
    # Some lane's tile sum passed its bound (label 8): if some probability
    # may exceed 2^tau the slow path (label 5) recomputes the
    # scores, masks them again if the tile is cut, and runs the full softmax
    # (running-max vote, rescale factors, dq rescaled with them); either
    # way the tile is then treated as significant (sig_ops).  The odd
    # tile's barrier waits for both: after the barrier the other waves may
    # refill this tile's K slot.
    out += ["s_cmp_lg_u64 %[any], 0", "s_cbranch_scc1 8f"] + tail + ["s_branch 9f"]
    out += ["7:"] + mask_body() + ["s_branch 6b"]  # the mask, out of the common path
    out += ["8:"] + [f"v_cmp_gt_f32_e64 %[c{rb}], %[r{rb}], %[pbnd]" for rb in range(NRB)]
    out += ["s_nop 1", "s_or_b64 %[any], %[c0], %[c1]", "s_cmp_lg_u64 %[any], 0",
            "s_cbranch_scc1 5f"]
    out += sig_ops(1 - pin) + tail + ["s_branch 9f"]
    out += ["5:", "s_nop 15", "s_nop 15"]
    out += qk_again() + mask_part() + [text for _, text in softmax_ops(1 - pin)]
    out += [f"v_mul_f32 %[dq{rb}], %[dq{rb}], %[al{rb}]" for rb in range(NRB)]
    out += sig_ops(1 - pin)
    return out + tail + ["9:"], per


# fp32 output, P.V step t: hi rb0, hi rb1, lo rb0, lo rb1 (MFMA 4 t + u).
# The last reader of the 16-key step ks = 0 operands is MFMA 4 * NDB - 1;
# its operands may be overwritten from the gap after MFMA F32_KS0_FREE on.
F32_KS0_FREE = 4 * NDB - 1 + 4


def pv_part_f32(even):
    """fp32 output: O^T += V^T (P_hi + P_lo)^T of tile v-1 with tile v's
    exact-max softmax (vote, rescale factors) in the MFMAs' shadow.  The
    probabilities are single-buffered (the register file holds no second
    hi/lo pair): the packing of the step-0 operands waits until the MFMAs
    reading them are done, and the step-1 operands are packed into the
    score registers and moved into place after the last MFMA."""
    nm = 2 * NRB * NT
    soft = softmax_ops(0, pack=False)
    late = [op for rb in range(NRB) for j in range(4, 8) for op in pack_f32(rb, j, False)]
    direct = [op for rb in range(NRB) for j in range(4) for op in pack_f32(rb, j, True)]
    ca = sum(COST[k] for k, _ in soft + late)
    cd = sum(COST[k] for k, _ in direct)
    g1 = max(F32_KS0_FREE + 1, round(nm * ca / (ca + cd)))
    ga, per = assign(soft + late, g1)
    gd, _ = assign(direct, nm - g1)
    gaps = ga + gd
    out = []
    for t in range(NT):
        ks, db = divmod(t, NDB)
        wait = 2 if t + 1 < NT else 0
        if even and t == KPRE_STEP + 1:
            wait = 4
        out.append(f"s_waitcnt lgkmcnt({wait})")
        for u in range(2 * NRB):
            buf, rb = divmod(u, NRB)
            out.append(f"v_mfma_f32_32x32x16_bf16 %[acc{rb}{db}], {grp(vgroup(t))}, "
                       f"{pbop(buf, rb, ks)}, %[acc{rb}{db}]")
            if u == 0:  # LDS reads right behind the MFMA, before the VALU ops
                if even and t == KPRE_STEP:
                    out += kpre_reads()
                if t + 2 < NT:
                    out += vreads(t + 2)
            out += gaps[2 * NRB * t + u]
    # the step-1 operands: the last MFMAs read them while they run
    out += ["s_nop 15", "s_nop 15"]
    for rb in range(NRB):
        for j in range(4, 8):
            out.append(f"v_mov_b32 {pbreg(0, rb, j)}, {s(rb, 2 * j + 1)}")
            out.append(f"v_mov_b32 {pbreg(1, rb, j)}, {s(rb, 2 * j)}")
    tail = [] if even else ["s_waitcnt vmcnt(0)", "s_barrier"] + kpre_reads()
    return out + tail, per


def macro(name, lines, sep="\\n\\t"):
    out = [f"#define {name} \\"]
    for ln in lines:
        out.append(f'  "{ln}{sep}" \\')
    out.append('  ""')
    return out


def operand_list(name, items):
    out = [f"#define {name} \\"]
    for i, it in enumerate(items):
        out.append(f"  {it}{',' if i + 1 < len(items) else ''} \\")
    out.append("")
    return out


ROW_B = 512  # bytes of one K or V row in LDS (HD = 256 bf16)


def offset_operands():
    """The block's LDS offsets (immediates, from the slot offsets KOFF, VOFF,
    MK, MV of the asm statement's scope) and the copy lane offsets: K
    k-step s at ka[s % 8] + ko<s / 8>; V step (ks, db), half h at va[db %
    4] + vo<ks><db / 4><h> (16 rows per ks, 8 rows per h, d blocks 4..7 at
    +256); copy j = 2 a + b to the rows 8 a + 16 b past the wave's first."""
    ops = ['[ko0] "i"(KOFF)', '[ko1] "i"(KOFF + 256)']
    ops += [f'[vo{ks}{hi}{h}] "i"(VOFF + {16 * ROW_B * ks + 256 * hi + 8 * ROW_B * h})'
            for ks in range(NPS) for hi in (0, 1) for h in (0, 1)]
    ops += [f'[mk{j}] "i"(MK + {ROW_B * (8 * (j >> 1) + 16 * (j & 1))})' for j in range(4)]
    ops += [f'[mv{j}] "i"(MV + {ROW_B * (8 * (j >> 1) + 16 * (j & 1))})' for j in range(4)]
    ops += ['[dka] "v"(dl.ka)', '[dkb] "v"(dl.kb)', '[dva] "v"(dl.va)', '[dvb] "v"(dl.vb)']
    return ops


def render():
    out = ["// Generated by gen_tile_hd256.py -- edit the generator, not this file.",
           "// One 32-key tile at HD = 256: S^T = K Q^T, the optional key-bound mask,",
           "// and O^T += V^T P^T of the previous tile with this tile's online softmax",
           "// in its shadow.  Variant P<b> reads the bf16 probabilities from buffer b",
           "// and writes the new ones to buffer 1 - b.  ASM blocks (bf16 output) take",
           "// the scores against the running max as it stands and fall back to a slow",
           "// path when a probability may exceed 2^tau; F32 blocks (fp32 output) keep",
           "// the exact running max.  Operands are bound by the asm statement in",
           "// ring_attn_fused.hip."]
    per = None
    for lazy, name in ((True, "ASM"), (False, "F32")):
        for pin in (0, 1):
            if lazy:
                pv, per = pv_part(pin, True)
                # the mask (rare) is out of line, branched to
                body = qk_part() + mask_test("7f") + ["6:"] + pv
            else:
                pv, per = pv_part_f32(pin == 1)
                body = qk_part() + mask_part() + pv
            out.append(f"// P.V block of variant {name}_P{pin}: about {per:.1f} full-rate VALU issue"
                       " slots of softmax work per MFMA.")
            check_dot_hazards(body)
            check_scc(body)
            out += macro(f"RA_TILE_HD256_{name}_P{pin}", body)
    q = [f'[q{rb}_{k}] "{{{qop(rb, k)}}}"(q[{rb}][{k}])' for rb in range(NRB) for k in range(NKS)]
    out += operand_list("RA_TILE_HD256_Q_OPERANDS", q)
    kp = [f'[kp{k}] "+{{v[{KPRE + 4 * k}:{KPRE + 4 * k + 3}]}}"(kpre[{k}])' for k in range(2)]
    out += operand_list("RA_TILE_HD256_KPRE_OPERANDS", kp)
    acc = [f'[acc{rb}{db}] "+a"(acc[{rb}][{db}])' for rb in range(NRB) for db in range(NDB)]
    out += operand_list("RA_TILE_HD256_ACC_OPERANDS", acc)
    out += operand_list("RA_TILE_HD256_OFFSET_OPERANDS", offset_operands())
    # probability buffers: p0 at PB[0], p1 at PB[1].  bf16 output: one is
    # read (the previous tile's), the other written; fp32 output: hi in p0,
    # lo in p1, both read and rewritten.
    for buf in (0, 1):
        regs = [(pbop(buf, rb, ks), f"p{buf}[{rb}][{ks}]") for rb in range(NRB)
                for ks in range(NPS)]
        out += operand_list(f"RA_TILE_HD256_PB_IN{buf}", [f'"{{{r}}}"({c})' for r, c in regs])
        out += operand_list(f"RA_TILE_HD256_PB_OUT{buf}", [f'"=&{{{r}}}"({c})' for r, c in regs])
        out += operand_list(f"RA_TILE_HD256_PB_RW{buf}", [f'"+{{{r}}}"({c})' for r, c in regs])
    clob = [f'"v{r}"' for r in list(range(S0, S0 + 32)) + list(range(RING0, RING0 + 12))]
    out += operand_list("RA_TILE_HD256_CLOBBERS", clob)
    return "\n".join(out) + "\n"


def main():
    text = render()
    if "--check" in sys.argv:
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        if cur != text:
            print(f"{OUT} is stale: run {os.path.basename(__file__)}", file=sys.stderr)
            return 1
        return 0
    with open(OUT, "w") as f:
        f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
