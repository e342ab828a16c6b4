#!/usr/bin/env python3
"""Benchmark of the fused ring + current attention step on one MI355X.

A step is the whole hot path over one 4k-token chunk at 32k context:
the strided KV-cache write of the chunk's 4096 current tokens into the P=8
striped shards, then the single fused launch that visits the 28672 cached
tokens (8 shard visits) and the causal current chunk (NQ=32, NKV=2, HD=256,
bf16 in, fp32 accumulation, bf16 out + fp32 LSE).  Inputs are seeded N(0,1)
bf16 draws (no dataset or trained weights are involved on this path) and are
resident in HBM before timing; the cache is striped by the library's own
strided write, as earlier chunks would have left it.

Prints ONE JSON line.  ``value`` is TFLOP/s of algorithmic work
4*HD*NQ*sum_rows(cache_len + i + 1) per step time; ``roofline`` relates the
fused kernel's own duration (HIP events on its launch stream) to the bf16
dense MFMA peak; ``cpu_baseline`` times the fp64 oracle on a bounded sample
of rows of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "fused ring attention TFLOP/s + % bf16 MFMA peak; ms/chunk at 32k ctx"
WARMUP_S = 0.1                 # default warm-up: at least this long (and at least 5 steps)


def alg_flops(w):
    """QK^T + PV flops over visible (row, key) pairs of the real rows: a row
    at chunk position p sees the cache and current tokens 0..p."""
    pos = w.positions[:w.real_rows]
    pairs = w.real_rows * w.cache_len + sum(p + 1 for p in pos)
    return 4 * w.hd * w.nq * pairs


def alg_bytes(w, with_write):
    """Q + visible K/V once + out + LSE (+ the write's read and write)."""
    row = w.nkv * w.hd * 2
    cur_seen = max(w.positions[:w.real_rows]) + 1 if w.real_rows else 0
    b = w.real_rows * w.nq * w.hd * 2 * 2 + w.real_rows * w.nq * 4
    b += 2 * (w.cache_len + cur_seen) * row
    if with_write:
        b += 2 * 2 * w.n_cur_real * row
    return b


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "ring_attn_fused_32k_hbm_traffic.md")
FUSED_SOURCES = [os.path.join(ROOT, "context_causal_attention_ring_amd", "csrc", f)
                 for f in ("ring_attn_fused.hip", "tile_hd256.inc", "tile_hd128.inc",
                           "tile_hd64.inc")]


def peak_sclk_mhz():
    """The device's peak engine clock as HIP reports it (attribute 5, kHz), or
    None if the runtime cannot be asked.  The clock under load is lower."""
    import ctypes
    import context_causal_attention_ring_amd as ra
    try:  # the HIP runtime the library itself is linked against
        get = ctypes.CDLL(ra.LIB_PATH).hipDeviceGetAttribute
    except (OSError, AttributeError):
        return None
    val = ctypes.c_int(0)
    if get(ctypes.byref(val), 5, torch_device_index()) == 0 and val.value > 0:
        return round(val.value / 1000)
    return None


def torch_device_index():
    import torch
    return torch.cuda.current_device()


def fused_source_sha():
    """sha256 over the fused kernel's sources (the kernel and its generated
    tile block), comments and blank space left out: a comment edit does not
    change the kernel the counters were taken on.  (No string literal in
    these sources holds a comment marker.)"""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in FUSED_SOURCES:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_SUMMARY):
    """HBM bytes per fused launch from the committed rocprofv3 counter summary,
    or None when it was taken on a different kernel source (or is absent)."""
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
    if rec is None:
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == fused_source_sha() else None


def setup(w, device, out_fp32=False):
    import torch
    import context_causal_attention_ring_amd as ra
    import workloads
    t = workloads.generate(w)
    C = w.q_rows
    d = dict(q=t["q"].to(device), k_cur=t["k_cur"].to(device), v_cur=t["v_cur"].to(device))
    shape = (w.P, w.shard_cap, w.nkv, w.hd)
    d["k_cache"] = torch.full(shape, float("nan"), device=device, dtype=torch.bfloat16)
    d["v_cache"] = torch.full(shape, float("nan"), device=device, dtype=torch.bfloat16)
    layout = ra.StripeLayout(w.interleave, 0)
    dims = ra.make_dims(d["q"], d["k_cur"], w.shard_cap, real_rows=w.real_rows,
                        head_rows=w.head_rows, scale=w.scale, head_pos=w.head_pos,
                        tail_pos=w.tail_start, out_fp32=out_fp32)
    if w.cache_len:
        k_tok = t["k_cache_tok"].to(device)
        v_tok = t["v_cache_tok"].to(device)
        ra.kv_cache_write(k_tok, v_tok, w.cache_len, d["k_cache"], d["v_cache"], 0, w.P, layout,
                          dims)
        torch.cuda.synchronize()
        del k_tok, v_tok
    d["out"] = torch.empty(C, w.nq, w.hd, device=device,
                           dtype=torch.float32 if out_fp32 else torch.bfloat16)
    d["lse"] = torch.empty(w.nq, C, device=device, dtype=torch.float32)
    return t, d, layout, dims


def cpu_baseline(w, t, budget_s=12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of rows
    (budget_s of oracle time; None: every real row)."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    args = [t[k].float().numpy() for k in ("q", "k_cache_tok", "v_cache_tok", "k_cur", "v_cur")]
    rng = np.random.default_rng(0)
    order = rng.permutation(w.real_rows).tolist()
    done, flops, elapsed, blk = 0, 0, 0.0, 8
    while done < len(order) and (budget_s is None or elapsed < budget_s):
        rows = order[done:done + blk]
        t0 = time.perf_counter()
        oracle.attention_rows(*args, rows, w.scale, positions=w.positions)
        elapsed += time.perf_counter() - t0
        flops += sum(4 * w.hd * w.nq * (w.cache_len + w.positions[i] + 1) for i in rows)
        done += len(rows)
        blk = min(64, blk * 2)
    try:
        host_cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cpus = os.cpu_count()
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "host_cpus": host_cpus, "host_cpus_total": os.cpu_count(),
            "sample": f"fp64 oracle on {done} random real rows of the {w.name} chunk "
                      f"(all {w.nq} heads, {w.cache_len} cached + causal keys), "
                      f"{elapsed:.1f} s; TFLOP/s of the same algorithmic count; cores = the "
                      f"BLAS threads the oracle's matrix products ran on"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 5, and as many "
                         "more as fill 100 ms, so that the clock has settled on short steps)")
    ap.add_argument("--config", default="32k", help="workload name (default: 32k)")
    ap.add_argument("--head-dim", type=int, default=0, choices=(0, 64, 128, 256),
                    help="run the workload's shape at this head dim (0: the workload's own)")
    ap.add_argument("--splits", type=int, default=0,
                    help="cut each row's key walk into this many segments (partials merged by "
                         "LSE); 0 (default): the library's suggestion for this GPU")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-fp32", action="store_true",
                    help="time the fp32-output mode (hi + lo probabilities in P.V)")
    ap.add_argument("--no-two-launch", action="store_true",
                    help="skip timing the two-launch comparator (cache-only + current-only + merge)")
    ap.add_argument("--traffic", default=TRAFFIC_SUMMARY,
                    help="rocprofv3 summary holding the measured HBM bytes per fused launch")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for counter calibration)")
    ap.add_argument("--separate-write", action="store_true",
                    help="time kv_cache_write as its own launch before the attention "
                         "(default without a split: the write inside the attention launch)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="only time the oracle on the host (no GPU needed) and print its line")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the CPU baseline's sample; 0: every real "
                         "row of the workload")
    args = ap.parse_args()
    budget = args.cpu_budget if args.cpu_budget > 0 else None

    if args.cpu_only:
        import workloads
        w = workloads.CONFIGS[args.config]
        line = {"config": {"workload": w.name}, "cpu_baseline": cpu_baseline(
            w, workloads.generate(w), budget)}
        print(json.dumps(line), flush=True)
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build computes one rank's share of the ring "
              f"on a single MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2

    import torch
    import context_causal_attention_ring_amd as ra
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return 0

    w = workloads.CONFIGS[args.config]
    if args.head_dim and args.head_dim != w.hd:
        w = workloads.with_fields(w, name=f"{w.name}_hd{args.head_dim}", hd=args.head_dim)
    t, d, layout, dims = setup(w, dev, args.out_fp32)
    stream = torch.cuda.current_stream()
    if args.splits == 0:
        args.splits = ra.ra_split_suggest(dims, torch.cuda.get_device_properties(dev)
                                          .multi_processor_count)
    ws_bytes = ra.ra_split_workspace_bytes(dims, args.splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    # The step: the chunk's strided cache write and the attention.  Without a
    # split the write runs inside the attention launch (ring_attn_prefill_write);
    # a split walk, whose segments all end together, keeps kv_cache_write as
    # its own launch before it (measured: the copy at the end of every
    # segment costs the split launch more than the separate launch does), as
    # does --separate-write.
    fused_write = args.splits == 1 and not args.separate_write

    def step(ev=None):
        if fused_write:
            if ev is not None:
                ev[0].record(stream)
            ra.ring_attn_prefill_split_write(d["q"], d["k_cache"], d["v_cache"], d["k_cur"],
                                             d["v_cur"], w.cache_len, w.P, layout, args.splits,
                                             ws, w.n_cur_real, d["out"], d["lse"], dims)
            if ev is not None:
                ev[1].record(stream)
            return
        ra.kv_cache_write(d["k_cur"], d["v_cur"], w.n_cur_real, d["k_cache"], d["v_cache"],
                          w.cache_len, w.P, layout, dims)
        if ev is not None:
            ev[0].record(stream)
        ra.ring_attn_prefill_split(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                                   w.cache_len, w.P, layout, args.splits, ws, d["out"], d["lse"],
                                   dims)
        if ev is not None:
            ev[1].record(stream)

    # Warm-up.  The engine clock settles over the first ~10 ms of load, which
    # a few steps of a short workload (a rank share: 0.4 ms) do not cover.
    n_warm = args.warmup if args.warmup is not None else 5
    for _ in range(n_warm):
        step()
    torch.cuda.synchronize()
    if args.warmup is None:
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < WARMUP_S:
            for _ in range(5):
                step()
            n_warm += 5
            torch.cuda.synchronize()
    args.warmup = n_warm
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_ms_avg = sum(kern_ms) / len(kern_ms)
    kern_sorted = sorted(kern_ms)
    kern_ms_median = kern_sorted[len(kern_sorted) // 2]
    ms_per_step = total_s * 1e3 / args.steps

    # The removed two-launch variant as a comparator: cache-only launch,
    # current-only launch, LSE merge (same write before it).
    two = None
    if not args.no_two_launch:
        C = w.q_rows  # partials in the model dtype (bf16) with fp32 LSEs, merged in fp32
        parts = (torch.empty(C, w.nq, w.hd, device=dev, dtype=torch.bfloat16),
                 torch.empty(w.nq, C, device=dev),
                 torch.empty(C, w.nq, w.hd, device=dev, dtype=torch.bfloat16),
                 torch.empty(w.nq, C, device=dev))

        def step2():
            ra.kv_cache_write(d["k_cur"], d["v_cur"], w.n_cur_real, d["k_cache"], d["v_cache"],
                              w.cache_len, w.P, layout, dims)
            ra.two_launch_prefill(d["q"], d["k_cache"], d["v_cache"], d["k_cur"], d["v_cur"],
                                  w.cache_len, w.P, layout, d["out"], d["lse"], dims, parts)
        for _ in range(args.warmup):
            step2()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            step2()
        torch.cuda.synchronize()
        ms2 = (time.perf_counter() - t1) * 1e3 / args.steps
        del parts
        two = {"ms_per_step": round(ms2, 4), "fused_time_reduction": None}

    # Cold-cache view: evict the Infinity Cache with a 512 MiB write before each step.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(min(args.steps, 10)):
        scratch.fill_(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        cold.append(a.elapsed_time(b))
    del scratch

    F = alg_flops(w)
    value = F / (ms_per_step * 1e-3) / 1e12
    achieved = F / (kern_ms_avg * 1e-3) / 1e12
    traffic = measured_traffic(args.traffic) if w.name == "32k" and not args.out_fp32 else None
    props = torch.cuda.get_device_properties(dev)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "out_dtype": "fp32" if args.out_fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: fused ring+current prefill of one {w.q_rows}-row "
                               f"chunk share (head {w.head_rows} rows at chunk position "
                               f"{w.head_pos} + tail {w.tail_rows} at {w.tail_start}, "
                               f"{w.n_cur} current tokens) over "
                               f"{w.cache_len} cached tokens in P={w.P} striped shards, "
                               f"NQ={w.nq} NKV={w.nkv} HD={w.hd}, plus the strided "
                               f"kv_cache_write of the chunk",
                   "cache_len": w.cache_len, "P": w.P, "q_rows": w.q_rows,
                   "real_rows": w.real_rows, "nq": w.nq, "nkv": w.nkv, "hd": w.hd,
                   "splits": args.splits, "flop_per_step": F,
                   "write": "in the fused launch" if fused_write else "kv_cache_write launch"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_chunk": round(ms_per_step, 4),
        "ms_per_step_cold_median": round(sorted(cold)[len(cold) // 2], 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": f"ring_attn_fused_kernel<{w.hd}>",
                     "kernel_ms_avg": round(kern_ms_avg, 4),
                     "kernel_ms_median": round(kern_ms_median, 4),
                     "kernel_ms_min": round(kern_sorted[0], 4)},
        "device": {"name": props.name, "arch": props.gcnArchName.split(":")[0],
                   "cus": props.multi_processor_count, "peak_sclk_mhz": peak_sclk_mhz()},
    }
    if two is not None:
        two["fused_time_reduction"] = round(1 - ms_per_step / two["ms_per_step"], 4)
        res["two_launch"] = two
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, t, budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
