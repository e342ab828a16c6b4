"""Seeded random configurations on the GPU against the oracle, every real
row: head dims, GQA groups, shard counts, stripe units, first shards, cache
lengths (none, short, unaligned), head/tail pieces at arbitrary chunk
positions, pad rows, pad current tokens, split counts and both output
dtypes, drawn together so that combinations the hand-written cases do not
name are covered too.  RINGATTN_RANDOM_CASES=N runs N configurations of the
same draw instead of the default 24 (a wider sweep).

A second draw takes long walks: caches of up to 40000 tokens in up to 64
shards, up to 1400 chunk rows (several row tiles per KV head), splits up to
16.  Those are checked on sampled rows (the ends of each piece, the real/pad
edge and seeded random rows); RINGATTN_RANDOM_LARGE_CASES=N runs N of them
instead of the default 6.

A third set takes configurations of the first draw with the strided cache
write of a random number of the chunk's tokens inside the attention launch
(split or not): bit for bit what the write followed by the attention
gives, the cache against the oracle's write, the attention against the
oracle; RINGATTN_RANDOM_WRITE_CASES=N runs N of them instead of the
default 8.

A fourth set runs the two-launch comparator on configurations of the first
draw: the cache-only and current-only launches against the oracle's
one-region attention, their LSE merge against the merge's definition on
the same partials, and with fp32 partials the merged result against the
full attention; RINGATTN_RANDOM_PARTIAL_CASES=N runs N of them instead of
the default 8."""
import os

import numpy as np
import pytest
import torch

import context_causal_attention_ring_amd as ra
import oracle
import workloads
from helpers import Case, bits, sample_rows
from test_gpu_parity import (SENTINEL, TOL_BF16, TOL_F32, TOL_LSE, check_pads_untouched,
                             compare, peaky_bf16_tol, run_partial, run_split)

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("RINGATTN_RANDOM_CASES", "24"))
N_LARGE = int(os.environ.get("RINGATTN_RANDOM_LARGE_CASES", "6"))
N_WRITE = int(os.environ.get("RINGATTN_RANDOM_WRITE_CASES", "8"))
N_PARTIAL = int(os.environ.get("RINGATTN_RANDOM_PARTIAL_CASES", "8"))


def draw(i, large=False):
    """Configuration i, a pure function of i (numpy's seeded generator);
    large: the long-walk draw."""
    g = np.random.default_rng((5000 if large else 1000) + i)
    hd = int(g.choice([64, 128, 256]))
    nkv = int(g.choice([1, 2] if large else [1, 2, 3, 4]))
    group = int(g.choice([1, 4, 8, 16] if large else [1, 2, 3, 4, 8, 16]))
    while nkv * group > (32 if large else 16):
        group //= 2
    P = int(g.choice([1, 2, 3, 8, 13, 64])) if large else int(g.integers(1, 10))
    interleave = int(g.choice([1, 1, 4, 16, 64] if large else [1, 1, 1, 2, 7, 16]))
    max_cache, max_rows, max_gap = (40000, 700, 2000) if large else (2500, 120, 200)
    cache_len = 0 if g.random() < (0.1 if large else 0.2) else int(g.integers(1, max_cache))
    head_rows = int(g.integers(0, max_rows))
    tail_rows = int(g.integers(0 if head_rows else 1, max_rows))
    head_pos = int(g.integers(0, max_gap))
    tail_pos = head_pos + head_rows + int(g.integers(0, max_gap))
    q_rows = head_rows + tail_rows
    # pads only at the end of the rows: a partly real tail needs a full head
    real_rows = int(g.integers(0, q_rows + 1)) if g.random() < 0.5 else q_rows
    if real_rows > head_rows:
        real_rows = max(real_rows, head_rows)
    last = -1
    if real_rows:
        last = head_pos + min(real_rows, head_rows) - 1 if head_rows else -1
        if real_rows > head_rows:
            last = max(last, tail_pos + real_rows - head_rows - 1)
    cur_len = max(last + 1, 1) + int(g.integers(0, 40))
    cur_real = max(last + 1, 0) + int(g.integers(0, cur_len - max(last + 1, 0) + 1))
    cap = max(oracle.shard_lengths(cache_len, P, interleave) + [1])
    name, seed = (f"large{i}", 6000 + i) if large else (f"rand{i}", 2000 + i)
    w = workloads.custom(name, seed=seed, nq=nkv * group, nkv=nkv, hd=hd, cache_len=cache_len,
                         P=P, head_rows=head_rows, tail_rows=tail_rows,
                         real_rows=real_rows, shard_cap=cap, interleave=interleave,
                         head_pos=head_pos, tail_pos=tail_pos, cur_len=cur_len,
                         cur_real=cur_real)
    splits = int(g.choice([1, 2, 4, 7, 16] if large else [1, 1, 1, 2, 3, 5]))
    fp32 = bool(g.random() < 0.3)
    ring_start = int(g.integers(0, P))
    return w, splits, fp32, ring_start


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration_matches_oracle(i):
    w, splits, fp32, ring_start = draw(i)
    print(f"[gpu] random config {i}: NQ={w.nq} NKV={w.nkv} HD={w.hd} L={w.cache_len} P={w.P} "
          f"I={w.interleave} start={ring_start} head={w.head_rows}@{w.head_pos} "
          f"tail={w.tail_rows}@{w.tail_start} real={w.real_rows} cur={w.n_cur}/{w.n_cur_real} "
          f"splits={splits} fp32={fp32}", flush=True)
    case = Case(w).to_device()
    out, lse = run_split(case, splits, out_fp32=fp32, ring_start=ring_start)
    if w.real_rows:
        compare(case, out, lse, list(range(w.real_rows)), TOL_F32 if fp32 else TOL_BF16)
    check_pads_untouched(case, out, lse)


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_long_walk_matches_oracle(i):
    w, splits, fp32, ring_start = draw(i, large=True)
    print(f"[gpu] long-walk config {i}: NQ={w.nq} NKV={w.nkv} HD={w.hd} L={w.cache_len} "
          f"P={w.P} I={w.interleave} start={ring_start} head={w.head_rows}@{w.head_pos} "
          f"tail={w.tail_rows}@{w.tail_start} real={w.real_rows} cur={w.n_cur}/{w.n_cur_real} "
          f"splits={splits} fp32={fp32}", flush=True)
    case = Case(w).to_device()
    out, lse = run_split(case, splits, out_fp32=fp32, ring_start=ring_start)
    if w.real_rows:
        compare(case, out, lse, sample_rows(w, 48, seed=i), TOL_F32 if fp32 else TOL_BF16)
    check_pads_untouched(case, out, lse)


def write_run(case, n_tokens, splits, fp32, ring_start, fused):
    """The attention with the write of n_tokens chunk tokens inside its
    launch (fused), or kv_cache_write and then the attention, on fresh
    device copies of the case."""
    w = case.w
    case.to_device()
    d = case.d
    C, NQ, HD = w.q_rows, w.nq, w.hd
    out = torch.full((C, NQ, HD), SENTINEL, device="cuda",
                     dtype=torch.float32 if fp32 else torch.bfloat16)
    lse = torch.full((NQ, C), SENTINEL, device="cuda", dtype=torch.float32)
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, out_fp32=fp32,
                        head_pos=w.head_pos, tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, ring_start)
    nbytes = ra.ra_split_workspace_bytes(dims, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None
    args = (d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"], w.cache_len, w.P, layout)
    if fused and splits == 1:
        ra.ring_attn_prefill_write(*args, n_tokens, out, lse, dims)
    elif fused:
        ra.ring_attn_prefill_split_write(*args, splits, ws, n_tokens, out, lse, dims)
    else:
        ra.kv_cache_write(d["k_cur"], d["v_cur"], n_tokens, d["k_cache"], d["v_cache"],
                          w.cache_len, w.P, layout, dims)
        ra.ring_attn_prefill_split(*args, splits, ws, out, lse, dims)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), d["k_cache"].cpu(), d["v_cache"].cpu()


def draw_write(i):
    """Write configuration i: a configuration of the first draw (its own
    seeds), the number of chunk tokens to write, and shard room for them."""
    w, splits, fp32, ring_start = draw(3000 + i)
    g = np.random.default_rng(9000 + i)
    # every sixth configuration writes nothing (the attention alone)
    n_tokens = 0 if i % 6 == 5 else int(g.integers(0, w.n_cur_real + 1))
    cap = max(oracle.shard_lengths(w.cache_len + n_tokens, w.P, w.interleave) + [1])
    w = workloads.with_fields(w, name=f"write{i}", shard_cap=cap + int(g.integers(0, 3)))
    return w, splits, fp32, ring_start, n_tokens


@pytest.mark.parametrize("i", range(N_WRITE))
def test_random_fused_write_matches_write_then_attention(i):
    w, splits, fp32, ring_start, n_tokens = draw_write(i)
    print(f"[gpu] write config {i}: NQ={w.nq} NKV={w.nkv} HD={w.hd} L={w.cache_len} P={w.P} "
          f"I={w.interleave} start={ring_start} cap={w.shard_cap} head={w.head_rows}@{w.head_pos} "
          f"tail={w.tail_rows}@{w.tail_start} real={w.real_rows} cur={w.n_cur}/{w.n_cur_real} "
          f"n_tokens={n_tokens} splits={splits} fp32={fp32}", flush=True)
    case = Case(w)
    out, lse, kc, vc = write_run(case, n_tokens, splits, fp32, ring_start, fused=True)
    out2, lse2, kc2, vc2 = write_run(case, n_tokens, splits, fp32, ring_start, fused=False)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    kc_ref, vc_ref = oracle.kv_cache_write_ref(bits(case.kc), bits(case.vc), bits(case.t["k_cur"]),
                                               bits(case.t["v_cur"]), n_tokens, w.cache_len, w.P,
                                               w.interleave)
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)
    assert np.array_equal(bits(kc2), kc_ref) and np.array_equal(bits(vc2), vc_ref)
    if w.real_rows:
        compare(case, out, lse, list(range(w.real_rows)), TOL_F32 if fp32 else TOL_BF16)
    check_pads_untouched(case, out, lse)


@pytest.mark.parametrize("i", range(N_PARTIAL))
def test_random_partials_and_merge(i):
    w, _, parts_fp32, ring_start = draw(6000 + i)
    out_fp32 = bool(np.random.default_rng(11000 + i).random() < 0.5)
    print(f"[gpu] partial config {i}: NQ={w.nq} NKV={w.nkv} HD={w.hd} L={w.cache_len} P={w.P} "
          f"I={w.interleave} start={ring_start} head={w.head_rows}@{w.head_pos} "
          f"tail={w.tail_rows}@{w.tail_start} real={w.real_rows} cur={w.n_cur}/{w.n_cur_real} "
          f"parts_fp32={parts_fp32} out_fp32={out_fp32}", flush=True)
    case = Case(w).to_device()
    o1, l1, _ = run_partial(case, ra.RA_REGION_CACHE, parts_fp32, ring_start)
    o2, l2, _ = run_partial(case, ra.RA_REGION_CURRENT, parts_fp32, ring_start)
    out = torch.full((w.q_rows, w.nq, w.hd), SENTINEL, device="cuda",
                     dtype=torch.float32 if out_fp32 else torch.bfloat16)
    lse = torch.full((w.nq, w.q_rows), SENTINEL, device="cuda", dtype=torch.float32)
    ra.merge_attn_states(o1, l1, o2, l2, out, lse, ra.make_dims(
        case.d["q"], case.d["k_cur"], w.shard_cap, real_rows=w.real_rows,
        head_rows=w.head_rows, out_fp32=out_fp32))
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    check_pads_untouched(case, out, lse)
    if not w.real_rows:
        return
    rows = list(range(w.real_rows))
    t = case.t
    args = (t["q"].float().numpy(), t["k_cache_tok"].float().numpy(),
            t["v_cache_tok"].float().numpy(), t["k_cur"].float().numpy(),
            t["v_cur"].float().numpy(), rows, w.scale)
    tol = TOL_F32 if parts_fp32 else TOL_BF16
    parts = []
    for o, l, only in ((o1, l1, dict(current=False)), (o2, l2, dict(cache=False))):
        r, rl = oracle.attention_rows(*args, positions=w.positions, **only)
        o, l = o.cpu().double().numpy()[rows], l.cpu().double().numpy()[:, rows]
        fin = np.isfinite(rl)
        print(f"    partial {only} max|d out|={np.abs(o - r).max():.3e} (<= {tol})", flush=True)
        assert np.abs(o - r).max() <= tol
        assert (np.isneginf(l) == ~fin).all()
        if fin.any():
            assert np.abs(l[fin] - rl[fin]).max() <= TOL_LSE
        parts += [o, l]
    # the merge kernel against the merge's definition on these very partials:
    # what is left is the output's own rounding (reading of the bf16 bar for
    # outputs of 2 and more, as for the peaky inputs)
    om, lm = oracle.two_pass_merge(*parts)
    d = np.abs(out.double().numpy()[rows] - om)
    bar = TOL_F32 if out_fp32 else peaky_bf16_tol(om)
    print(f"    merge of the partials max|d out|={d.max():.3e} max|d|/bar={np.max(d / bar):.3f}",
          flush=True)
    assert (d <= bar).all()
    assert np.abs(lse.double().numpy()[:, rows] - lm).max() <= TOL_LSE
    if parts_fp32:  # and the whole against the oracle's full attention
        compare(case, out, lse, rows, TOL_F32 if out_fp32 else TOL_BF16)


def test_random_configurations_are_varied():
    """The draws cover what they claim (a check of the generators, on the CPU
    side of the same file; the default counts whatever the environment asks)."""
    ws = [draw(i) for i in range(24)]
    assert {w.hd for w, *_ in ws} == {64, 128, 256}
    assert any(w.cache_len == 0 for w, *_ in ws) and any(w.cache_len % 32 for w, *_ in ws)
    assert any(s > 1 for _, s, _, _ in ws) and any(f for _, _, f, _ in ws)
    assert any(w.real_rows < w.q_rows for w, *_ in ws)
    assert any(w.interleave > 1 for w, *_ in ws) and any(r > 0 for *_, r in ws)
    assert any(w.n_cur_real < w.n_cur for w, *_ in ws)
    large = [draw(i, large=True) for i in range(6)]
    assert any(w.cache_len > 10000 for w, *_ in large) and any(s > 1 for _, s, _, _ in large)
    assert any(w.real_rows * (w.nq // w.nkv) > 256 for w, *_ in large)
    writes = [draw_write(i) for i in range(8)]
    assert any(n == 0 for *_, n in writes) and any(0 < n for *_, n in writes)
    assert any(s > 1 for _, s, *_ in writes) and any(s == 1 and n > 0 for _, s, _, _, n in writes)
