"""Shared test plumbing: seeded inputs -> striped device tensors, and the
oracle's view of the same bits.  Striping for the device inputs uses the
oracle's map (test code may call the oracle; the library never does)."""
import numpy as np
import torch

import oracle
import workloads

NAN_BF16 = 0x7FC0


def bits(t):
    """bf16 torch tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def f64(t):
    """bf16 torch tensor -> numpy float32 holding the same values exactly
    (every bf16 value is a float32 value); the oracle widens to fp64."""
    return t.float().numpy()


def striped_cache(tok, P, interleave, cap, fill=NAN_BF16):
    """Token-order bf16 [L, NKV, HD] -> striped bf16 [P, cap, NKV, HD];
    unused slots hold `fill` (a bf16 bit pattern, NaN by default)."""
    return from_bits(oracle.stripe(bits(tok), P, interleave, cap, fill=np.uint16(fill)))


class Case:
    """Inputs of one workload on the CPU (token order) and on the device."""

    def __init__(self, w, fill=NAN_BF16, device="cuda"):
        self.w = w
        self.t = workloads.generate(w)
        self.kc = striped_cache(self.t["k_cache_tok"], w.P, w.interleave, w.shard_cap, fill)
        self.vc = striped_cache(self.t["v_cache_tok"], w.P, w.interleave, w.shard_cap, fill)
        self.device = device
        self.d = None

    def to_device(self):
        dev = self.device
        self.d = dict(q=self.t["q"].to(dev), k_cur=self.t["k_cur"].to(dev),
                      v_cur=self.t["v_cur"].to(dev), k_cache=self.kc.to(dev),
                      v_cache=self.vc.to(dev))
        return self

    def oracle_rows(self, rows):
        t, w = self.t, self.w
        return oracle.attention_rows(f64(t["q"]), f64(t["k_cache_tok"]), f64(t["v_cache_tok"]),
                                     f64(t["k_cur"]), f64(t["v_cur"]), rows, w.scale,
                                     positions=w.positions)


def sample_rows(w, n_random, seed=0):
    """Rows for sampled parity at full size: first/last rows of the head and
    tail sequences, the real/pad boundary, and seeded random real rows."""
    real = w.real_rows
    fixed = {0, 1, w.head_rows - 1, w.head_rows, w.head_rows + 1, real - 1, real - 2}
    fixed = {r for r in fixed if 0 <= r < real}
    rng = np.random.default_rng(seed)
    rand = set(rng.choice(real, size=min(n_random, real), replace=False).tolist())
    return sorted(fixed | rand)
