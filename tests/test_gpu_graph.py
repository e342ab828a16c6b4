"""HIP graph capture of the library's calls (torch.cuda.graph).  A call is
kernel launches on the caller's stream with plain pointers and sizes, and
nothing else that goes on the stream (no allocation, no memset), so a
captured call replays against whatever its buffers hold at replay time.
The graph here holds the no-allocation split walk and the attention with
the strided cache write inside its launch; it is replayed several times,
with eager work between replays (new query values, output buffers
overwritten), and every replay must equal, bit for bit, the eager calls on
the same buffer contents."""
import pytest
import torch

import context_causal_attention_ring_amd as ra
import workloads
from helpers import Case
from test_gpu_parity import SENTINEL

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    w = workloads.CONFIGS["32k_rank3of8"]
    case = Case(w).to_device()
    d = case.d
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, head_pos=w.head_pos,
                        tail_pos=w.tail_start)
    layout = ra.StripeLayout(w.interleave, 0)
    shape_o, shape_l = (w.q_rows, w.nq, w.hd), (w.nq, w.q_rows)
    bufs = [torch.empty(shape_o, device="cuda", dtype=torch.bfloat16),
            torch.empty(shape_l, device="cuda", dtype=torch.float32),
            torch.empty(shape_o, device="cuda", dtype=torch.bfloat16),
            torch.empty(shape_l, device="cuda", dtype=torch.float32)]

    def calls():
        ra.ring_attn_prefill_split_noalloc(d["q"], d["k_cache"], d["v_cache"], d["k_cur"],
                                           d["v_cur"], w.cache_len, w.P, layout, 4, bufs[0],
                                           bufs[1], dims)
        # rewrites the same cache slots with the same values on every call
        ra.ring_attn_prefill_write(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                                   w.cache_len, w.P, layout, w.n_cur_real, bufs[2], bufs[3], dims)

    def clobber():
        for b in bufs:
            b.fill_(SENTINEL)

    q0 = d["q"].clone()
    q1 = q0.clone()
    q1[:w.real_rows] = q0[:w.real_rows] * 0.5
    eager = []
    for q in (q0, q1):
        print(f"[gpu] eager {w.name} (q scaled by {1.0 if q is q0 else 0.5})", flush=True)
        d["q"].copy_(q)
        clobber()
        calls()
        torch.cuda.synchronize()
        eager.append([b.cpu() for b in bufs])
    assert not torch.equal(eager[0][0], eager[1][0])  # the two inputs differ

    # warm up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print(f"[gpu] capturing {w.name}", flush=True)
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for rep in range(4):
        k = rep % 2
        d["q"].copy_((q0, q1)[k])  # eager work between the replays
        clobber()
        torch.cuda.synchronize()
        print(f"[gpu] replay {rep} (inputs {k})", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for x, b in zip(eager[k], bufs):
            assert torch.equal(x.view(torch.uint8), b.cpu().view(torch.uint8)), rep
