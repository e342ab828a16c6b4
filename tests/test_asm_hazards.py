"""Static checks of the compiled fused kernel around its hand-scheduled blocks.

The HD = 256, 128 and 64 tile blocks are single inline-asm statements,
so the compiler's hazard checks do not see the MFMAs inside them.  An MFMA
reads its A and B
operands while it runs and writes its result at the end, so compiler code
that follows a block must not, before those MFMAs are done, write a
register the block's last two MFMAs read or touch a register they write.
Inside the block this holds by construction; this test checks the
compiler's side on the device assembly of the kernel as it is built: the
first WINDOW instructions after every tile block (up to the next asm
statement) do none of that unless two s_nop 15 (32 wait states) come
first.  A block may also leave LDS reads of
the next tile's first K operands (KPRE) in flight, so no compiler
instruction between two blocks may touch those registers.

The LDS-DMA copies set M0 (their LDS destination) inside asm statements
that declare it clobbered, which the compiler honours but warns may be
undefined behaviour.  So that this can never matter, no instruction the
compiler emits in any fused kernel may use M0 at all: neither name it nor
be one of the instructions that read it implicitly.
"""
import importlib.util
import os
import re
import shutil
import tempfile

import pytest

from context_causal_attention_ring_amd import build

_spec = importlib.util.spec_from_file_location("gen_tile_hd256",
                                               os.path.join(build.CSRC, "gen_tile_hd256.py"))
gen = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(gen)
KPRE = {("v", r) for r in range(gen.KPRE, gen.KPRE + 8)}

WINDOW = 40  # instructions; each takes at least a cycle, an MFMA's operands are read well within
HAS_HIPCC = any(p and os.path.exists(p) for p in
                (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"))


def regs(text):
    out = set()
    for kind, a, b in re.findall(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {(kind, r) for r in range(int(a), int(b) + 1)}
    for kind, a in re.findall(r"\b([va])(\d+)\b", text):
        out.add((kind, int(a)))
    return out


def tile_blocks(lines):
    """(start, index after the block, last two MFMAs) for every big inline-asm
    block.  A block with a slow path (label 8, reached by a branch after the
    P.V MFMAs) leaves by two ways: the common one right after those MFMAs,
    and the slow path, whose last MFMAs are followed by two s_nop 15 and the
    softmax reading their results; the MFMAs that matter are the common
    path's last ones."""
    start = None
    for i, line in enumerate(lines):
        if ";;#ASMSTART" in line:
            start = i
        elif ";;#ASMEND" in line and start is not None and i - start > 300:
            body = [x.strip() for x in lines[start:i]]
            if "8:" in body:
                body = body[:body.index("8:")]
            mfma = [x for x in body if x.startswith("v_mfma")]
            yield start, i + 1, mfma[-2:]


def compiler_code(lines):
    """Instructions outside inline asm (labels and comments dropped)."""
    inside = False
    for line in lines:
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif not inside:
            ins = line.split(";")[0].strip()
            if ins and not ins.startswith(".") and not ins.endswith(":"):
                yield ins


def hazards_after(lines, at, mfmas):
    src, dst = set(), set()
    for m in mfmas:
        ops = m.split(None, 1)[1].split(", ")
        dst |= regs(ops[0])
        src |= regs(ops[1]) | regs(ops[2])
    found, n, nops = [], 0, 0
    for line in lines[at:at + 10 * WINDOW]:
        if ";;#ASMSTART" in line:  # the next block: its ring refills are LDS reads, as inside
            break                  # a block, landing long after an MFMA has read its operands
        ins = line.split(";")[0].strip()
        if not ins or ins.startswith("."):
            continue
        n += 1
        if n > WINDOW:
            break
        if ins.startswith("s_nop 15"):
            nops += 1
            if nops >= 2:
                break
        parts = ins.split(None, 1)
        if len(parts) < 2:
            continue
        writes = regs(parts[1].split(",")[0]) if parts[0].startswith(
            ("v_", "ds_read", "scratch_load", "global_load", "buffer_load")) else set()
        if writes & (src | dst) or regs(parts[1]) & dst:
            found.append(ins)
    return found


@pytest.mark.skipif(not HAS_HIPCC, reason="needs hipcc to assemble the kernel")
@pytest.mark.parametrize("extra", [(), ("-DRA_SYNC_EVERY_TILE",)], ids=["product", "checking"])
def test_no_compiler_code_races_the_last_mfmas_of_a_tile_block(extra):
    with tempfile.TemporaryDirectory() as tmp:
        asm = open(build.assemble(out=os.path.join(tmp, "fused.s"), extra=extra)).read()
    # every head dim (256, 128, 64) with bf16 and fp32 output
    kernels = re.findall(r"^(_ZN2ra\S*fused_kernel\S*):", asm, re.M)
    assert len(kernels) == 6
    for name in kernels:
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))]
        lines = body.splitlines()
        blocks = list(tile_blocks(lines))
        assert len(blocks) == 4, name  # the loop is unrolled over the four slots
        for _, at, mfmas in blocks:
            assert len(mfmas) == 2
            bad = hazards_after(lines, at, mfmas)
            assert not bad, f"{name}: compiler code after a tile block: {bad}"
        # from the first block to the last (the tile loop), KPRE is the blocks' own
        first, last = blocks[0][0], blocks[-1][1]
        touch = [ins for ins in compiler_code(lines[first:last]) if regs(ins) & KPRE]
        assert not touch, f"{name}: compiler code touches the KPRE registers: {touch[:4]}"


# Instructions that read or write M0 without naming it (gfx9 family).
IMPLICIT_M0 = ("s_movrel", "v_movrel", "s_sendmsg", "ds_gws", "ds_append", "ds_consume",
               "ds_ordered", "ds_read_addtid", "ds_write_addtid", "v_interp", "s_set_gpr_idx")


def m0_users(code):
    """Compiler instructions that use M0: naming it, reading it implicitly,
    or an LDS-DMA load (`... lds`, whose LDS address M0 holds)."""
    return [ins for ins in code
            if re.search(r"\bm0\b", ins) or re.search(r"\blds\s*$", ins)
            or ins.split(None, 1)[0].startswith(IMPLICIT_M0)]


@pytest.mark.skipif(not HAS_HIPCC, reason="needs hipcc to assemble the kernel")
@pytest.mark.parametrize("extra", [(), ("-DRA_SYNC_EVERY_TILE",)], ids=["product", "checking"])
def test_compiler_code_never_uses_m0(extra):
    with tempfile.TemporaryDirectory() as tmp:
        asm = open(build.assemble(out=os.path.join(tmp, "fused.s"), extra=extra)).read()
    kernels = re.findall(r"^(_ZN2ra\S*fused_kernel\S*):", asm, re.M)
    assert len(kernels) == 6  # HD 64, 128, 256 x bf16 / fp32 output
    for name in kernels:
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))]
        bad = m0_users(compiler_code(body.splitlines()))
        assert not bad, f"{name}: compiler code uses M0: {bad[:4]}"


def scratch_use(asm):
    """(kernel, private segment bytes, VGPR spills) of every fused kernel."""
    out = []
    for name, body in re.findall(r"\.amdhsa_kernel (\S*fused_kernel\S*)(.*?)\.end_amdhsa_kernel",
                                 asm, re.S):
        seg = int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", body).group(1))
        out.append((name, seg))
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)]
    return out, spills


@pytest.mark.skipif(not HAS_HIPCC, reason="needs hipcc to assemble the kernel")
@pytest.mark.parametrize("extra", [(), ("-DRA_SYNC_EVERY_TILE",)], ids=["product", "checking"])
def test_fused_kernels_use_no_scratch(extra):
    """Every register of the fused kernels is spoken for during the walk, so
    a value the compiler keeps live across it spills to scratch memory; none
    may (values needed after the walk are derived again there)."""
    with tempfile.TemporaryDirectory() as tmp:
        asm = open(build.assemble(out=os.path.join(tmp, "fused.s"), extra=extra)).read()
    segs, spills = scratch_use(asm)
    assert len(segs) == 6
    assert all(seg == 0 for _, seg in segs), segs
    assert spills and all(n == 0 for n in spills), spills


@pytest.mark.skipif(not HAS_HIPCC, reason="needs hipcc to assemble the kernel")
def test_hd64_kernels_fit_two_workgroups_per_cu():
    """At HD = 64 two workgroups share a CU: each wave may hold 256 of the
    SIMD's 512 registers per lane (VGPRs and AGPRs together) and each
    workgroup half the LDS."""
    with tempfile.TemporaryDirectory() as tmp:
        asm = open(build.assemble(out=os.path.join(tmp, "fused.s"), extra=())).read()
    found = 0
    for name, body in re.findall(r"\.amdhsa_kernel (\S*fused_kernel\S*)(.*?)\.end_amdhsa_kernel",
                                 asm, re.S):
        if "fused_kernelILi64E" not in name:
            continue
        found += 1
        regs_ = int(re.search(r"\.amdhsa_next_free_vgpr\s+(\d+)", body).group(1))
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size\s+(\d+)", body).group(1))
        assert regs_ <= 256 and lds <= 80 * 1024, (name, regs_, lds)
    assert found == 2


def test_m0_check_has_teeth():
    """The M0 check flags explicit and implicit users, and passes plain code."""
    assert m0_users(["s_mov_b32 m0, s4", "s_sendmsg sendmsg(MSG_INTERRUPT)",
                     "buffer_load_dword v1, v2, s[4:7], 0 offen lds",
                     "v_readlane_b32 s0, v1, m0"]) == [
        "s_mov_b32 m0, s4", "s_sendmsg sendmsg(MSG_INTERRUPT)",
        "buffer_load_dword v1, v2, s[4:7], 0 offen lds", "v_readlane_b32 s0, v1, m0"]
    assert m0_users(["v_add_f32 v1, v2, v3", "s_add_u32 s0, s1, s2",
                     "v_readlane_b32 s0, v1, 5", "ds_read_b128 v[0:3], v4"]) == []


def test_scc_check_has_teeth():
    """The generators' SCC check (run on every block they write) flags a
    scalar op that clobbers SCC between a compare and its select, and
    passes the compare-select pair alone."""
    gen.check_scc(["s_cmp_eq_u32 s0, 0", "s_cselect_b32 s1, 1, 0", "s_cbranch_scc1 7f"])
    with pytest.raises(AssertionError):
        gen.check_scc(["s_cmp_eq_u32 s0, 0", "s_add_u32 m0, s2, s3", "s_cselect_b32 s1, 1, 0"])
    merged = gen.scc_atomic([("salu", "s_cmp_lg_u64 s[0:1], 0"), ("salu", "s_cselect_b64 s[0:1], -1, 0"),
                             ("valu", "v_add_f32 v0, v1, v2")])
    assert len(merged) == 2 and gen.split_ops([m[1] for m in merged]) == [
        "s_cmp_lg_u64 s[0:1], 0", "s_cselect_b64 s[0:1], -1, 0", "v_add_f32 v0, v1, v2"]
