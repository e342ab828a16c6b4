"""The no-allocation split entry point against the split entry point with a
caller workspace: the same kernels on the same inputs, so the results must
be bit-identical; two calls in a row, the second smaller than the first (the
library's workspace keeps the first call's partials, which must not leak
into the second), and the second also against the oracle; then a run of
seeded random configurations, one call after another on the same
workspace, each bit-identical to the caller-workspace call and within the
bar of the oracle."""
import numpy as np
import pytest
import torch

import context_causal_attention_ring_amd as ra
import workloads
from helpers import Case
from test_gpu_parity import (FULL_CASES, SENTINEL, TOL_BF16, TOL_F32, check_pads_untouched,
                             compare)
from test_gpu_random_configs import draw

pytestmark = pytest.mark.gpu


def both(case, splits, out_fp32, ring_start=0):
    """(noalloc out, lse), (workspace out, lse) for one case."""
    w, d = case.w, case.d
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, out_fp32=out_fp32,
                        head_pos=w.head_pos, tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, ring_start)
    dt = torch.float32 if out_fp32 else torch.bfloat16
    res = []
    for noalloc in (True, False):
        out = torch.full((w.q_rows, w.nq, w.hd), SENTINEL, device="cuda", dtype=dt)
        lse = torch.full((w.nq, w.q_rows), SENTINEL, device="cuda", dtype=torch.float32)
        print(f"[gpu] split{'_noalloc' if noalloc else ''} {w.name} splits={splits} "
              f"fp32={out_fp32}", flush=True)
        if noalloc:
            ra.ring_attn_prefill_split_noalloc(d["q"], d["k_cache"], d["v_cache"], d["k_cur"],
                                               d["v_cur"], w.cache_len, w.P, layout, splits, out,
                                               lse, dims)
        else:
            ws = torch.empty(ra.ra_split_workspace_bytes(dims, splits), dtype=torch.uint8,
                             device="cuda")
            ra.ring_attn_prefill_split(d["q"], d["k_cache"], d["v_cache"], d["k_cur"],
                                       d["v_cur"], w.cache_len, w.P, layout, splits, ws, out,
                                       lse, dims)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    return res


def test_noalloc_split_matches_workspace_split_twice():
    big = Case(workloads.CONFIGS["32k_rank3of8"]).to_device()    # 4 splits: 64.25 MiB
    (o1, l1), (o2, l2) = both(big, 4, False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    small = Case(FULL_CASES[2]).to_device()                      # 7 splits, fp32 output
    (o1, l1), (o2, l2) = both(small, 7, True)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    compare(small, o1, l1, list(range(small.w.real_rows)), TOL_F32)
    check_pads_untouched(small, o1, l1)


def test_noalloc_split_random_sequence():
    """Twelve seeded random configurations (splits 2 to 16), one after
    another: each call finds the previous call's partials in the workspace."""
    for i in range(12):
        w, _, fp32, ring_start = draw(8000 + i)
        splits = int(np.random.default_rng(12000 + i).choice([2, 3, 5, 16]))
        print(f"[gpu] noalloc random {i}: NQ={w.nq} NKV={w.nkv} HD={w.hd} L={w.cache_len} "
              f"P={w.P} I={w.interleave} start={ring_start} real={w.real_rows} "
              f"splits={splits} fp32={fp32}", flush=True)
        case = Case(w).to_device()
        (o1, l1), (o2, l2) = both(case, splits, fp32, ring_start)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        if w.real_rows:
            compare(case, o1, l1, list(range(w.real_rows)), TOL_F32 if fp32 else TOL_BF16)
        check_pads_untouched(case, o1, l1)
