#!/usr/bin/env python3
"""Writes tile_hd128.inc and tile_hd64.inc: the instruction block of one
step of the fused ring + current attention kernel at HD = 128 and HD = 64
with bf16 output (a wave owns two 32-row blocks; the accumulator O^T is
2 x HD/32 tiles of 32 x 32 fp32 in AGPRs).

A 32-key tile takes HD/4 MFMAs per wave (HD/8 for S^T = K Q^T, HD/8 for
O^T += V^T P^T), while its online softmax is 32 scores per lane at any
HD.  Hidden behind the P.V MFMAs alone, as the HD = 256 block does, the
softmax would need about twice (HD = 128) or four times (HD = 64) the
VALU issue slots those MFMAs leave.  So the block works on three tiles at
once: block u computes the scores of tile u, the softmax of tile u-1 and
the P.V of tile u-2, and spreads the softmax over all of its MFMAs.  The
scores live in two buffers by tile parity, and the common softmax writes
its exponentials to temporaries, so tile u-1's raw scores are still there
for its slow path: no second S^T = K Q^T is needed.

Tiles run in pairs (K and V slots t mod 4).  Block u (E = u mod 2):
  1. HD/8 MFMAs S^T = K Q^T of tile u into score buffer E.  The first two
     K operands were read into KPRE ahead, the others are read from LDS
     two k-steps ahead.  One LDS-DMA copy per two k-steps: the wave's rows
     of K tile u + 2 and of V tile u (HD/64 instructions each).
  2. HD/8 MFMAs O^T += V^T P^T of tile u-2 (probability buffer E).  The
     even block reads the odd tile's KPRE here.
  Behind every MFMA goes a share (by issue cost; an S^T MFMA's share is
  qk_weight of a P.V MFMA's) of tile u-1's common-case softmax: scores of
  buffer 1 - E against the running max as it stands, exponentials into
  temporaries, the row sums and their compensated fold, the bf16
  probabilities into buffer 1 - E, and a test of each lane's tile sum
  against its bound.  The walkers' step to the next tile shares the same
  shadow.
  3. When a lane's tile sum passed its bound: if some probability may exceed
     2^tau, the full softmax (running-max vote, rescale factors, exact new
     max where voted) on tile u-1's intact scores; either way the tile is
     significant (its bf16-rounded minus fp32 row sums go to dq, the bound
     rises).
  4. When tile u is cut by a key bound: its scores at or past each row's
     bound become -inf (the next block's softmax reads them).
  5. Odd u (the end of the pair): wait for this wave's copies, meet the
     other waves at the pair's barrier, read the next tile's KPRE and leave
     it in flight.

The walk runs two blocks more than it has tiles (their scores are masked),
so the last tile's P.V comes out of the final block.

Usage: python gen_tile_pipe.py            (rewrites both .inc files)
       python gen_tile_pipe.py --check    (exit 1 if one is stale)
"""
import contextlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import gen_tile_hd256 as base  # noqa: E402  (softmax, mask, walker and hazard helpers)

NPS = 2            # 16-key steps of P.V per 32-key tile
NRB = base.NRB     # 32-row blocks per wave
# The register map of the geometry being written (see Geometry and regmap):
Q0 = 44            # Q^T operands (pinned): row block rb, k-step k -> v[Q0 + 4 NKS rb + 4 k : +3]
S0 = (108, 140)    # score buffers (pinned): buffer b, row block rb, key slot i -> v[S0[b] + 16 rb + i]
T0 = 204           # exponentials (clobbered): row block rb, key slot i -> v[T0 + 4 rb + i % 4]
PB = base.PB       # bf16 probabilities (pinned), two buffers, as at HD = 256
KPRE = base.KPRE   # K operands of k-steps 0 and 1 (pinned), read ahead; None: read in the block
RING0 = base.RING0  # operand ring (clobbered)
KPRE_STEP = 2      # P.V step of an even block after which the next tile's KPRE is read
# HD = 128: the HD = 256 map (one wave per SIMD, 512 registers).  HD = 64:
# two workgroups per CU, so a wave has 256 registers, 64 of them the
# accumulator's AGPRs: everything pinned or clobbered fits v[44:191], and
# the first two K operands are read at the start of each block instead of
# ahead (the other wave on the SIMD covers their latency).
REGMAPS = {
    128: dict(Q0=44, S0=(108, 140), T0=204, PB=base.PB, KPRE=base.KPRE, RING0=base.RING0),
    64: dict(Q0=44, S0=(76, 108), T0=172, PB=(140, 156), KPRE=None, RING0=180),
}
# Softmax share of an MFMA gap in the S^T half relative to the P.V half: the
# S^T half also carries the copies and the walkers' scalar step (HD = 128:
# 0.7 measured 0.2-1.5 % faster than an even split on gfx950, 1.3 slower).
QK_WEIGHT = {128: 0.7, 64: 0.7}


class Geometry:
    """The block's shape at head dim hd."""

    def __init__(self, hd):
        self.hd = hd
        self.nks = hd // 16            # 16-wide k-steps of QK^T
        self.ndb = hd // 32            # 32-wide d blocks of the output
        self.nt = NPS * self.ndb       # P.V steps; each issues one MFMA per row block
        self.nm = 2 * NRB * self.nks   # MFMAs per block (nt = nks)
        self.row_b = 2 * hd            # bytes of one K or V row in LDS
        self.ncopy = self.row_b // 128  # copy instructions per operand and wave (a KiB each)
        self.qk_weight = QK_WEIGHT[hd]
        self.name = f"RA_TILE_HD{hd}"
        self.out = os.path.join(HERE, f"tile_hd{hd}.inc")
        self.regs = REGMAPS[hd]
        r = self.regs
        assert self.nt == self.nks and 2 * self.ncopy == self.nks // 2
        assert r["Q0"] + 4 * self.nks * NRB <= r["S0"][0] and r["S0"][1] + 32 <= r["PB"][0]
        assert r["PB"][1] + 16 <= r["T0"] and r["PB"][0] + 16 <= r["PB"][1]
        top = r["T0"] + 4 * NRB
        if r["KPRE"] is not None:
            assert top <= r["KPRE"]
            top = r["KPRE"] + 8
        assert top <= r["RING0"] and r["RING0"] + 12 <= 256
        self.top = r["RING0"] + 12  # VGPRs the blocks pin or clobber end here


@contextlib.contextmanager
def regmap(g):
    """Geometry g's register map in force: the helpers of this module and
    of gen_tile_hd256 read these constants when they are called."""
    mine = {k: globals()[k] for k in g.regs}
    theirs = (base.PB, base.RING0)
    globals().update(g.regs)
    base.PB, base.RING0 = g.regs["PB"], g.regs["RING0"]
    try:
        yield
    finally:
        globals().update(mine)
        base.PB, base.RING0 = theirs


def sreg(buf):
    """Score register of buffer buf as a function (rb, i) -> name."""
    return lambda rb, i: f"v{S0[buf] + 16 * rb + i}"


def treg(rb, i):
    """Exponential of key slot i of row block rb: four rotating registers
    per row block (a pair is packed two slots after its second member is
    written, so slot i's register is free again by slot i + 4)."""
    return f"v{T0 + 4 * rb + i % 4}"


def stile(buf, rb):
    b = S0[buf] + 16 * rb
    return f"v[{b}:{b + 15}]"


def qop(g, rb, k):
    b = Q0 + 4 * g.nks * rb + 4 * k
    return f"v[{b}:{b + 3}]"


# K step k uses ring group k % 3 and V step t group (t + nks) % 3: the
# first two V operands, read during the last two K steps, go to the groups
# those steps do not use.
def kgroup(k):
    return k % 3


def vgroup(g, t):
    return (t + g.nks) % 3


def kread(k):
    return f"ds_read_b128 {base.grp(kgroup(k))}, %[ka{k}] offset:%[ko]"


def kop(k):
    """K operand of k-step k: the first two were read ahead into KPRE (when
    the map has it)."""
    return f"%[kp{k}]" if k < 2 and KPRE is not None else base.grp(kgroup(k))


def block_start(g):
    """The block's first instructions and the LDS reads they leave in
    flight: without KPRE the first two K operands are read here."""
    out = ["s_nop 1", "s_waitcnt lgkmcnt(0)"]
    pending = []
    if KPRE is None:
        out += [kread(0), kread(1)]
        pending = [("k", 0), ("k", 1)]
    return out + dma_setup(g, 0), pending


def kpre_reads():
    """The next tile's KPRE reads (none without KPRE)."""
    return base.kpre_reads() if KPRE is not None else []


def vreads(g, t):
    """Two transposing reads (keys 0-7 and 8-15 of the step) of V operand t."""
    ks, db = divmod(t, g.ndb)
    return [f"ds_read_b64_tr_b16 {base.grp(vgroup(g, t), h)}, %[va{db}] offset:%[vo{ks}{h}]"
            for h in (0, 1)]


def copy_of(g, i):
    """Copy i of the block: (operand, b).  Copies 0 .. ncopy-1 move rows of
    the K tile, the next ncopy rows of the V tile; copy b of an operand
    moves the wave's 1024 / row_b rows at 16 b past its first row."""
    return ("k", i) if i < g.ncopy else ("v", i - g.ncopy)


def dma_setup(g, i):
    """M0 (the LDS destination) and the scalar offset of copy i, set right
    after copy i - 1 went out (LDS-DMA reads M0 when issued, and needs one
    wait state after an SALU write of M0, which the k-steps in between
    give).  Rows 16 apart share their swizzle, so one precomputed lane
    offset per operand (%[dk] / %[dv]) serves every b; the 16 b rows go
    into the scalar offset next to the tile's first byte."""
    kind, b = copy_of(g, i)
    out = [f"s_add_u32 m0, %[m0b], %[m{kind}{b}]"]
    if b:
        assert b == 1
        out.append(f"s_add_u32 %[st], %[off{kind}], %[rs16]")
    return out


def dma_issue(g, i):
    """Copy i (see dma_setup): 16 bytes per lane into LDS at M0."""
    kind, b = copy_of(g, i)
    soff = "%[st]" if b else f"%[off{kind}]"
    return [f"buffer_load_dwordx4 %[d{kind}], %[desc{kind}], {soff} offen lds"]


def softmax_common(sr, pout):
    """Tile u-1's common-case softmax (see base.softmax_ops_stale) on score
    buffer sr, exponentials into the temporaries.  Its scores are a block
    old, so the wait for score MFMAs the HD = 256 list opens with is
    dropped."""
    ops = base.softmax_ops_stale(pout, src=sreg(sr), dst=treg)
    assert ops[0] == ("nop", "s_nop 4")
    return ops[1:]


def block(g, E):
    """Block u with u mod 2 = E at geometry g."""
    sw, sr = E, 1 - E    # scores written (tile u) / read by the softmax (tile u-1)
    pin, pout = E, 1 - E  # probabilities read by P.V (tile u-2) / written (tile u-1)
    even = E == 0
    half = g.nm // 2
    gaps, per = base.assign(softmax_common(sr, pout), g.nm,
                            [g.qk_weight] * half + [1.0] * half)
    out, pending = block_start(g)  # pending: LDS reads in flight, in issue order

    def wait_for(tag):
        """Wait until the read tagged tag (and every one before it) is in."""
        nonlocal pending
        i = pending.index(tag)
        out.append(f"s_waitcnt lgkmcnt({len(pending) - 1 - i})")
        pending = pending[i + 1:]

    m = 0
    for k in range(g.nks):
        if k >= 2 or KPRE is None:  # this step's K operand must be in
            wait_for(("k", k))
        for rb in range(NRB):
            c = "0" if k == 0 else stile(sw, rb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {stile(sw, rb)}, {kop(k)}, {qop(g, rb, k)}, "
                       f"{c}")
            if rb == 0:  # LDS reads go out right behind an MFMA (see base.READ_NOTE)
                if k + 2 < g.nks:
                    out.append(kread(k + 2))
                    pending.append(("k", k + 2))
                else:
                    out += vreads(g, k + 2 - g.nks)
                    pending += [("v", k + 2 - g.nks, h) for h in (0, 1)]
            out += gaps[m]
            m += 1
        if k % 2 == 1:  # one copy of the next tiles per two k-steps
            out += dma_issue(g, k // 2)
            out += base.copy_step_ops() if k == g.nks - 1 else dma_setup(g, k // 2 + 1)
        if k == 0:  # the walkers' scalar step, in the first k-step's shadow
            out += base.walk_ops()
    for t in range(g.nt):
        ks, db = divmod(t, g.ndb)
        wait_for(("v", t, 1))
        for rb in range(NRB):
            out.append(f"v_mfma_f32_32x32x16_bf16 %[acc{rb}{db}], {base.grp(vgroup(g, t))}, "
                       f"{base.pbop(pin, rb, ks)}, %[acc{rb}{db}]")
            if rb == 0:
                if even and t == KPRE_STEP and KPRE is not None:
                    out += base.kpre_reads()
                    pending += [("kp", 0), ("kp", 1)]
                if t + 2 < g.nt:
                    out += vreads(g, t + 2)
                    pending += [("v", t + 2, h) for h in (0, 1)]
            out += gaps[m]
            m += 1
    assert m == g.nm
    tail = [] if even else ["s_waitcnt vmcnt(0)", "s_barrier"] + kpre_reads()
    # Common path: no lane's tile sum passed its bound and tile u is not cut.
    out += ["s_cmp_lg_u64 %[any], 0", "s_cbranch_scc1 8f", "10:"] + base.mask_test("7f")
    out += ["11:"] + tail + ["s_branch 9f"]
    # tile u cut by a key bound: mask its scores, for the next block
    out += ["7:"] + base.mask_body(sreg(sw)) + ["s_branch 11b"]
    # Some lane's tile sum passed its bound: if some probability may
    # exceed 2^tau, the full softmax on the intact scores (5); either way
    # the tile is significant.  Then back to the mask test.
    out += ["8:"] + [f"v_cmp_gt_f32_e64 %[c{rb}], %[r{rb}], %[pbnd]" for rb in range(NRB)]
    out += ["s_nop 1", "s_or_b64 %[any], %[c0], %[c1]", "s_cmp_lg_u64 %[any], 0",
            "s_cbranch_scc1 5f"]
    out += base.sig_ops(pout) + ["s_branch 10b"]
    out += ["5:"] + [text for _, text in base.softmax_ops(pout, src=sreg(sr))]
    out += [f"v_mul_f32 %[dq{rb}], %[dq{rb}], %[al{rb}]" for rb in range(NRB)]
    out += base.sig_ops(pout) + ["s_branch 10b", "9:"]
    return out, per


def block_f32(g, E):
    """Block u with u mod 2 = E at geometry g, fp32 output: the exact-max
    softmax of tile u-1 (running-max vote, rescale factors; in place on its
    scores, there is no slow path) and O^T += V^T (P_hi + P_lo)^T of tile
    u-2, four MFMAs per step (hi and lo of each row block).  As in the
    HD = 256 fp32 block the probabilities are single-buffered: the step-0
    hi/lo operands of tile u-1 are packed once the MFMAs reading tile u-2's
    are done, the step-1 ones into the score registers (free once the
    softmax has read them) and moved into place after the last MFMA."""
    sw, sr = E, 1 - E
    even = E == 0
    src = sreg(sr)
    nqk = NRB * g.nks
    nm = nqk + 2 * NRB * g.nt
    soft = base.softmax_ops(0, pack=False, src=src)
    assert soft[0] == ("nop", "s_nop 4")  # the scores are a block old
    soft = soft[1:]
    late = [op for rb in range(NRB) for j in range(4, 8)
            for op in base.pack_f32(rb, j, False, src)]
    direct = [op for rb in range(NRB) for j in range(4)
              for op in base.pack_f32(rb, j, True, src)]
    # the last reader of the step-0 operands is P.V MFMA 4 ndb - 1; they may
    # be overwritten from the gap four MFMAs after it
    ks0_free = nqk + 2 * NRB * g.ndb - 1 + 4
    w = [g.qk_weight] * nqk + [1.0] * (nm - nqk)
    ca = sum(base.COST[k] for k, _ in soft + late)
    cd = sum(base.COST[k] for k, _ in direct)
    g1 = max(ks0_free + 1, round(nm * ca / (ca + cd)))
    # the vote's compare-and-select chains stay whole: the S^T half's gaps
    # are followed by the copies' and walkers' scalar ops, which write SCC
    ga, per = base.assign(base.scc_atomic(soft + late), g1, w[:g1])
    gd, _ = base.assign(direct, nm - g1, w[g1:])
    gaps = [base.split_ops(gap) for gap in ga + gd]
    out, pending = block_start(g)

    def wait_for(tag):
        nonlocal pending
        i = pending.index(tag)
        out.append(f"s_waitcnt lgkmcnt({len(pending) - 1 - i})")
        pending = pending[i + 1:]

    m = 0
    for k in range(g.nks):
        if k >= 2 or KPRE is None:
            wait_for(("k", k))
        for rb in range(NRB):
            c = "0" if k == 0 else stile(sw, rb)
            out.append(f"v_mfma_f32_32x32x16_bf16 {stile(sw, rb)}, {kop(k)}, {qop(g, rb, k)}, "
                       f"{c}")
            if rb == 0:
                if k + 2 < g.nks:
                    out.append(kread(k + 2))
                    pending.append(("k", k + 2))
                else:
                    out += vreads(g, k + 2 - g.nks)
                    pending += [("v", k + 2 - g.nks, h) for h in (0, 1)]
            out += gaps[m]
            m += 1
        if k % 2 == 1:
            out += dma_issue(g, k // 2)
            out += base.copy_step_ops() if k == g.nks - 1 else dma_setup(g, k // 2 + 1)
        if k == 0:
            out += base.walk_ops()
    for t in range(g.nt):
        ks, db = divmod(t, g.ndb)
        wait_for(("v", t, 1))
        for u in range(2 * NRB):
            buf, rb = divmod(u, NRB)
            out.append(f"v_mfma_f32_32x32x16_bf16 %[acc{rb}{db}], {base.grp(vgroup(g, t))}, "
                       f"{base.pbop(buf, rb, ks)}, %[acc{rb}{db}]")
            if u == 0:
                if even and t == KPRE_STEP and KPRE is not None:
                    out += base.kpre_reads()
                    pending += [("kp", 0), ("kp", 1)]
                if t + 2 < g.nt:
                    out += vreads(g, t + 2)
                    pending += [("v", t + 2, h) for h in (0, 1)]
            out += gaps[m]
            m += 1
    assert m == nm
    # the step-1 operands: the last MFMAs read them while they run
    out += ["s_nop 15", "s_nop 15"]
    for rb in range(NRB):
        for j in range(4, 8):
            out.append(f"v_mov_b32 {base.pbreg(0, rb, j)}, {src(rb, 2 * j + 1)}")
            out.append(f"v_mov_b32 {base.pbreg(1, rb, j)}, {src(rb, 2 * j)}")
    tail = [] if even else ["s_waitcnt vmcnt(0)", "s_barrier"] + kpre_reads()
    out += base.mask_test("7f") + ["11:"] + tail + ["s_branch 9f"]
    out += ["7:"] + base.mask_body(sreg(sw)) + ["s_branch 11b", "9:"]
    return out, per


def offset_operands(g):
    """The block's LDS offsets (immediates, from the slot offsets KOFF, VOFF,
    MK, MV of the asm statement's scope) and the copy lane offsets: K
    k-step s at ka[s] + ko; V step (ks, db), half h at va[db] + vo<ks><h>
    (16 rows per ks, 8 rows per h); copy b to the rows 16 b past the wave's
    first."""
    ops = ['[ko] "i"(KOFF)']
    ops += [f'[vo{ks}{h}] "i"(VOFF + {16 * g.row_b * ks + 8 * g.row_b * h})'
            for ks in range(NPS) for h in (0, 1)]
    ops += [f'[mk{b}] "i"(MK + {16 * g.row_b * b})' for b in range(g.ncopy)]
    ops += [f'[mv{b}] "i"(MV + {16 * g.row_b * b})' for b in range(g.ncopy)]
    ops += ['[dk] "v"(dl.ka)', '[dv] "v"(dl.va)']
    return ops


def render(g):
    with regmap(g):
        return render_map(g)


def render_map(g):
    out = [f"// Generated by gen_tile_pipe.py -- edit the generator, not this file.",
           f"// One step of the HD = {g.hd} tile loop: S^T = K Q^T of tile u,",
           "// the online softmax of tile u-1 and O^T += V^T P^T of tile u-2, the",
           "// softmax spread over all the block's MFMAs.  Variant E<e> is block u",
           "// with u mod 2 = e: it writes score buffer e, reads score buffer 1 - e,",
           "// reads probability buffer e and writes buffer 1 - e.  Variant F32_E<e>",
           "// (fp32 output) takes the exact-max softmax and hi + lo probabilities",
           "// (P.V MFMAs for both), single-buffered in the two probability buffers",
           "// (hi, lo).  Operands are bound by the asm statement in",
           "// ring_attn_fused.hip."]
    for f32 in (False, True):
        for E in (0, 1):
            body, per = block_f32(g, E) if f32 else block(g, E)
            name = f"F32_E{E}" if f32 else f"E{E}"
            out.append(f"// Block {name}: about {per:.1f} full-rate VALU issue slots of softmax"
                       " work per MFMA.")
            base.check_dot_hazards(body)
            base.check_scc(body)
            out += base.macro(f"{g.name}_{name}", body)
    q = [f'[q{rb}_{k}] "{{{qop(g, rb, k)}}}"(q[{rb}][{k}])' for rb in range(NRB)
         for k in range(g.nks)]
    out += base.operand_list(f"{g.name}_Q_OPERANDS", q)
    if KPRE is not None:
        kp = [f'[kp{k}] "+{{v[{KPRE + 4 * k}:{KPRE + 4 * k + 3}]}}"(kpre[{k}])' for k in range(2)]
    else:  # no K operands read ahead: a placeholder the asm statement binds
        kp = ['[kpd] "+s"(kpd)']
    out += base.operand_list(f"{g.name}_KPRE_OPERANDS", kp)
    acc = [f'[acc{rb}{db}] "+a"(acc[{rb}][{db}])' for rb in range(NRB) for db in range(g.ndb)]
    out += base.operand_list(f"{g.name}_ACC_OPERANDS", acc)
    out += base.operand_list(f"{g.name}_OFFSET_OPERANDS", offset_operands(g))
    # score buffers: the one written (tile u) is an output, the one the
    # softmax reads (tile u-1) is rewritten by the slow path
    for buf in (0, 1):
        regs = [(stile(buf, rb), f"sc[{buf}][{rb}]") for rb in range(NRB)]
        out += base.operand_list(f"{g.name}_S_OUT{buf}", [f'"=&{{{r}}}"({c})' for r, c in regs])
        out += base.operand_list(f"{g.name}_S_RW{buf}", [f'"+{{{r}}}"({c})' for r, c in regs])
    for buf in (0, 1):
        regs = [(base.pbop(buf, rb, ks), f"p{buf}[{rb}][{ks}]") for rb in range(NRB)
                for ks in range(NPS)]
        out += base.operand_list(f"{g.name}_PB_IN{buf}", [f'"{{{r}}}"({c})' for r, c in regs])
        out += base.operand_list(f"{g.name}_PB_OUT{buf}", [f'"=&{{{r}}}"({c})' for r, c in regs])
        out += base.operand_list(f"{g.name}_PB_RW{buf}", [f'"+{{{r}}}"({c})' for r, c in regs])
    clob = [f'"v{r}"' for r in list(range(T0, T0 + 4 * NRB)) + list(range(RING0, RING0 + 12))]
    out += base.operand_list(f"{g.name}_CLOBBERS", clob)
    return "\n".join(out) + "\n"


GEOMETRIES = [Geometry(128), Geometry(64)]


def main():
    stale = 0
    for g in GEOMETRIES:
        text = render(g)
        if "--check" in sys.argv:
            cur = open(g.out).read() if os.path.exists(g.out) else ""
            if cur != text:
                print(f"{g.out} is stale: run {os.path.basename(__file__)}", file=sys.stderr)
                stale = 1
            continue
        with open(g.out, "w") as f:
            f.write(text)
    return stale


if __name__ == "__main__":
    sys.exit(main())
