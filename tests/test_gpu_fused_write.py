"""ring_attn_prefill_write on the GPU: the attention and the strided cache
write in one launch must give, bit for bit, what kv_cache_write and
ring_attn_prefill give one after the other; the cache against the oracle's
stripe map, the attention against the oracle."""
import numpy as np
import pytest
import torch

import context_causal_attention_ring_amd as ra
import oracle
import workloads
from helpers import Case, bits, sample_rows
from test_gpu_parity import SENTINEL, TOL_BF16, TOL_F32, compare, small

pytestmark = pytest.mark.gpu


def fused_write(case, n_tokens, out_fp32=False):
    """One ring_attn_prefill_write launch on fresh device copies of the case."""
    w = case.w
    case.to_device()
    d = case.d
    C, NQ, HD = w.q_rows, w.nq, w.hd
    out = torch.full((C, NQ, HD), SENTINEL, device="cuda",
                     dtype=torch.float32 if out_fp32 else torch.bfloat16)
    lse = torch.full((NQ, C), SENTINEL, device="cuda", dtype=torch.float32)
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, out_fp32=out_fp32,
                        head_pos=w.head_pos, tail_pos=w.tail_start)
    print(f"[gpu] ring_attn_prefill_write {w.name} C={C} L={w.cache_len} P={w.P} "
          f"I={w.interleave} cur={w.n_cur} n_tokens={n_tokens} real={w.real_rows}", flush=True)
    ra.ring_attn_prefill_write(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                               w.cache_len, w.P, ra.StripeLayout(w.interleave, 0), n_tokens,
                               out, lse, dims)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), d["k_cache"].cpu(), d["v_cache"].cpu()


def separate(case, n_tokens, out_fp32=False):
    """kv_cache_write, then ring_attn_prefill, on fresh device copies."""
    w = case.w
    case.to_device()
    d = case.d
    C, NQ, HD = w.q_rows, w.nq, w.hd
    out = torch.full((C, NQ, HD), SENTINEL, device="cuda",
                     dtype=torch.float32 if out_fp32 else torch.bfloat16)
    lse = torch.full((NQ, C), SENTINEL, device="cuda", dtype=torch.float32)
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, out_fp32=out_fp32,
                        head_pos=w.head_pos, tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, 0)
    ra.kv_cache_write(d["k_cur"], d["v_cur"], n_tokens, d["k_cache"], d["v_cache"], w.cache_len,
                      w.P, layout, dims)
    if w.real_rows:
        ra.ring_attn_prefill(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                             w.cache_len, w.P, layout, out, lse, dims)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), d["k_cache"].cpu(), d["v_cache"].cpu()


CASES = [
    (workloads.CONFIGS["tiny"], None),
    (small("w-interleave", nq=8, nkv=2, hd=128, cache_len=1000, P=3, real_rows=200,
           interleave=16), None),
    (small("w-nocache", nq=4, nkv=1, hd=256, cache_len=0, P=2, real_rows=96), None),
    (workloads.CONFIGS["tiny_rank1of2"], None),
    (workloads.CONFIGS["32k"], None),
    (workloads.CONFIGS["32k_rank3of8"], None),
    (workloads.CONFIGS["tiny"], 0),         # attention only
    (small("w-partial", nq=4, nkv=2, hd=64, cache_len=77, P=4, real_rows=50), 17),
]


@pytest.mark.parametrize("w,n", CASES, ids=[f"{w.name}-n{n}" for w, n in CASES])
def test_fused_write_matches_write_then_prefill(w, n):
    n_tokens = w.n_cur_real if n is None else n
    case = Case(w)
    out, lse, kc, vc = fused_write(case, n_tokens)
    out2, lse2, kc2, vc2 = separate(case, n_tokens)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    kc_ref, vc_ref = oracle.kv_cache_write_ref(bits(case.kc), bits(case.vc), bits(case.t["k_cur"]),
                                               bits(case.t["v_cur"]), n_tokens, w.cache_len, w.P,
                                               w.interleave)
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)
    assert np.array_equal(bits(kc2), kc_ref) and np.array_equal(bits(vc2), vc_ref)
    compare(case, out, lse, sample_rows(w, 8, seed=w.seed + 7), TOL_BF16)


def test_fused_write_fp32_output():
    w = workloads.CONFIGS["tiny"]
    case = Case(w)
    out, lse, kc, vc = fused_write(case, w.n_cur_real, out_fp32=True)
    out2, lse2, _, _ = separate(case, w.n_cur_real, out_fp32=True)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    compare(case, out, lse, sample_rows(w, 8, seed=3), TOL_F32)


def test_fused_write_without_real_rows_still_writes():
    """real_rows = 0: no attention launch, the write alone."""
    w = small("w-norows", nq=4, nkv=1, hd=64, cache_len=40, P=2, real_rows=0)
    w = workloads.with_fields(w, shard_cap=max(oracle.shard_lengths(w.cache_len + w.n_cur, w.P,
                                                                     w.interleave)))
    case = Case(w)
    n = w.n_cur
    _, _, kc, vc = fused_write(case, n)
    kc_ref, vc_ref = oracle.kv_cache_write_ref(bits(case.kc), bits(case.vc), bits(case.t["k_cur"]),
                                               bits(case.t["v_cur"]), n, w.cache_len, w.P,
                                               w.interleave)
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)


def split_run(case, n_tokens, splits, fused):
    """The split walk with the write inside its launch (fused) or as its own
    launch before it, on fresh device copies."""
    w = case.w
    case.to_device()
    d = case.d
    C, NQ, HD = w.q_rows, w.nq, w.hd
    out = torch.full((C, NQ, HD), SENTINEL, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((NQ, C), SENTINEL, device="cuda", dtype=torch.float32)
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, head_pos=w.head_pos,
                        tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, 0)
    ws = torch.empty(ra.ra_split_workspace_bytes(dims, splits), dtype=torch.uint8, device="cuda")
    print(f"[gpu] split {'write' if fused else 'then prefill'} {w.name} splits={splits} "
          f"n_tokens={n_tokens}", flush=True)
    if fused:
        ra.ring_attn_prefill_split_write(d["q"], d["k_cache"], d["v_cache"], d["k_cur"],
                                         d["v_cur"], w.cache_len, w.P, layout, splits, ws,
                                         n_tokens, out, lse, dims)
    else:
        ra.kv_cache_write(d["k_cur"], d["v_cur"], n_tokens, d["k_cache"], d["v_cache"],
                          w.cache_len, w.P, layout, dims)
        ra.ring_attn_prefill_split(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                                   w.cache_len, w.P, layout, splits, ws, out, lse, dims)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), d["k_cache"].cpu(), d["v_cache"].cpu()


SPLIT_CASES = [
    (workloads.CONFIGS["32k_rank3of8"], 4),
    (small("w-split", nq=8, nkv=2, hd=256, cache_len=700, P=3, real_rows=180, interleave=4), 3),
    (workloads.CONFIGS["tiny"], 16),
]


@pytest.mark.parametrize("w,splits", SPLIT_CASES, ids=[f"{w.name}-s{s}" for w, s in SPLIT_CASES])
def test_split_write_matches_write_then_split(w, splits):
    n_tokens = w.n_cur_real
    case = Case(w)
    out, lse, kc, vc = split_run(case, n_tokens, splits, fused=True)
    out2, lse2, _, _ = split_run(case, n_tokens, splits, fused=False)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    kc_ref, vc_ref = oracle.kv_cache_write_ref(bits(case.kc), bits(case.vc), bits(case.t["k_cur"]),
                                               bits(case.t["v_cur"]), n_tokens, w.cache_len, w.P,
                                               w.interleave)
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)
    compare(case, out, lse, sample_rows(w, 8, seed=w.seed + 11), TOL_BF16)
