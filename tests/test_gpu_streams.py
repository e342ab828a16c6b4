"""Independent calls on several streams at once.  Outside the no-allocation
entry point the library keeps no device state between calls, so work
launched concurrently on different streams (default priority) must give,
bit for bit, what the same calls give one after another on one stream."""
import pytest
import torch

import context_causal_attention_ring_amd as ra
import workloads
from helpers import Case
from test_gpu_parity import SENTINEL, small
from test_gpu_random_configs import draw

pytestmark = pytest.mark.gpu


def launch(case, kind, splits, fp32, stream):
    """Queue one call of `kind` on `stream` (nothing waits for it) on the
    case's device inputs; returns the device tensors it writes."""
    w, d = case.w, case.d
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, out_fp32=fp32,
                        head_pos=w.head_pos, tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, 0)
    with torch.cuda.stream(stream):
        out = torch.full((w.q_rows, w.nq, w.hd), SENTINEL, device="cuda",
                         dtype=torch.float32 if fp32 else torch.bfloat16)
        lse = torch.full((w.nq, w.q_rows), SENTINEL, device="cuda", dtype=torch.float32)
        nbytes = ra.ra_split_workspace_bytes(dims, splits)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"], w.cache_len, w.P, layout)
    if kind == "prefill":
        ra.ring_attn_prefill(*args, out, lse, dims, stream=stream)
    elif kind == "split":
        ra.ring_attn_prefill_split(*args, splits, ws, out, lse, dims, stream=stream)
    elif kind == "write":
        ra.ring_attn_prefill_split_write(*args, splits, ws, w.n_cur_real, out, lse, dims,
                                         stream=stream)
    else:
        raise ValueError(kind)
    return out, lse, d["k_cache"], d["v_cache"]


def calls():
    return [
        (Case(workloads.CONFIGS["32k_rank3of8"]), "split", 4, False),
        (Case(workloads.CONFIGS["tiny"]), "write", 1, False),
        (Case(draw(2, large=True)[0]), "split", 16, False),
        (Case(small("streams-hd64-fp32", hd=64, cache_len=1500, P=5, real_rows=300)),
         "prefill", 1, True),
        (Case(workloads.CONFIGS["tiny_rank1of2"]), "write", 3, True),
        (Case(small("streams-hd128", hd=128, cache_len=900, P=3, real_rows=250)),
         "prefill", 1, False),
    ]


def test_concurrent_streams_match_one_after_another():
    todo = calls()
    default = torch.cuda.current_stream()
    alone = []
    for case, kind, splits, fp32 in todo:
        print(f"[gpu] one stream: {case.w.name} {kind} splits={splits} fp32={fp32}", flush=True)
        case.to_device()
        res = launch(case, kind, splits, fp32, default)
        torch.cuda.synchronize()
        alone.append([t.cpu() for t in res])
    for case, *_ in todo:  # fresh device copies (a write call changes the caches),
        case.to_device()   # complete before any of the streams reads them
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    print(f"[gpu] {len(todo)} calls over {len(streams)} streams", flush=True)
    queued = [launch(case, kind, splits, fp32, streams[i % len(streams)])
              for i, (case, kind, splits, fp32) in enumerate(todo)]
    torch.cuda.synchronize()
    for (case, kind, _, _), a, b in zip(todo, alone, queued):
        for x, y in zip(a, b):
            y = y.cpu()
            assert x.dtype == y.dtype and x.shape == y.shape
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), (case.w.name, kind)
