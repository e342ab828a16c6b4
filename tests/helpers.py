"""Shared test plumbing: seeded inputs -> striped device tensors, and the
oracle's view of the same bits.  Striping for the device inputs uses the
oracle's map (test code may call the oracle; the library never does)."""
import math

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


# ------------------------------------------------------------ needle inputs
# One KV head, 16 query heads, HD = 256, 16 chunk tokens: row r = 16 t + h
# of the chunk has q = ALPHA * e_r, and its own "needle" cache token n_r
# holds k = BETA * e_r and a random v = w_r; every other key and value (the
# cache's other tokens and the whole current chunk) is zero.  Row r then
# scores s = scale * ALPHA * BETA on its needle and 0 on each of its other
# n_vis(r) - 1 visible keys, so the softmax definition gives in closed form
#   out_r = (e^s w_r + sum_{r' != r} w_r') / (e^s + n_vis(r) - 1)
#   lse_r = ln(e^s + n_vis(r) - 1),  n_vis(r) = cache_len + t + 1.
# Any misplaced read of the cache (wrong slot, past the shard) changes it.

NEEDLE_T, NEEDLE_G, NEEDLE_HD = 16, 16, 256
NEEDLE_ALPHA = NEEDLE_BETA = 16.0


def needle_positions(cache_len, seed=0):
    """256 distinct cache tokens: the last 128 and 128 spread from token 0,
    dealt to the rows in a seeded order."""
    n = NEEDLE_T * NEEDLE_G
    assert cache_len >= n
    tail = list(range(cache_len - n // 2, cache_len))
    spread = [k * ((cache_len - n // 2) // (n // 2)) for k in range(n // 2)]
    pos = np.array(spread + tail, dtype=np.int64)
    assert len(set(pos.tolist())) == n
    return np.random.default_rng(seed).permutation(pos)


def needle_values(seed=0):
    """w_r: [256, HD] bf16 values (seeded normal draws)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(NEEDLE_T * NEEDLE_G, NEEDLE_HD, generator=g).to(torch.bfloat16)


def needle_q():
    q = torch.zeros(NEEDLE_T, NEEDLE_G, NEEDLE_HD)
    r = torch.arange(NEEDLE_T * NEEDLE_G)
    q.view(-1, NEEDLE_HD)[r, r] = NEEDLE_ALPHA
    return q.to(torch.bfloat16)


def needle_expected(cache_len, w, scale, pos0=0):
    """Closed form above, fp64: out [T, G, HD], lse [G, T]; chunk token t at
    chunk position pos0 + t (it sees current tokens 0..pos0 + t)."""
    w = w.double().numpy()
    s = scale * NEEDLE_ALPHA * NEEDLE_BETA
    es = math.exp(s)
    total = w.sum(axis=0)
    out = np.zeros((NEEDLE_T, NEEDLE_G, NEEDLE_HD))
    lse = np.zeros((NEEDLE_G, NEEDLE_T))
    for t in range(NEEDLE_T):
        n_vis = cache_len + pos0 + t + 1
        for h in range(NEEDLE_G):
            r = t * NEEDLE_G + h
            out[t, h] = (es * w[r] + (total - w[r])) / (es + n_vis - 1)
            lse[h, t] = math.log(es + n_vis - 1)
    return out, lse
