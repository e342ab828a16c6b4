"""Seeded synthetic inputs for fused ring + current attention.

Shared by the tests, the bench and the smoke check.  This module draws
numbers and lays out token-order tensors only; it holds none of the method's
arithmetic (no striping, no attention).  The workload shape follows the
vLLM tpu-inference pull request "PCP: in-kernel ring cache phase, fused with
the current phase", Performance section: NQ=32 query heads, NKV=2 KV heads,
head dim 256, bf16, 4k-token chunks, 8 context-parallel ranks, contexts
8k..1M.  There is no dataset or trained model on the pages' path, so the
activations are N(0, 1) draws rounded to bf16.

Recipe (per named config): ``torch.Generator().manual_seed(seed)`` draws, in
this order, ``q [C, NQ, HD]``, ``k_cache_tok [L, NKV, HD]``,
``v_cache_tok [L, NKV, HD]``, ``k_cur [C, NKV, HD]``, ``v_cur [C, NKV, HD]``
as float32 ``randn`` rounded to bf16 (round-to-nearest-even).  ``k_mult``
multiplies both key tensors after rounding (a power of two, so exact).
Rows ``>= real_rows`` of ``q``, ``k_cur`` and ``v_cur`` are pads and are set
to NaN.
"""
from dataclasses import dataclass, replace
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    nq: int
    nkv: int
    hd: int
    cache_len: int          # L, tokens already cached (striped over P shards)
    P: int                  # number of cache shards (ring rounds)
    head_rows: int          # chunk rows of the head sequence
    tail_rows: int          # chunk rows of the tail sequence (padded)
    real_rows: int          # rows [0, real_rows) are real, the rest are pads
    shard_cap: int          # slots allocated per shard (room for this chunk)
    k_mult: float = 1.0
    interleave: int = 1

    @property
    def q_rows(self):
        return self.head_rows + self.tail_rows

    @property
    def scale(self):
        return self.hd ** -0.5


# Named configurations.  shard_cap is the per-shard room for the cache plus
# the chunk's own write: the largest shard after cache_len + real_rows tokens.
CONFIGS = {
    "tiny": Workload("tiny", 0, 4, 1, 64, 512, 2, 64, 64, 128, 320),
    "8k": Workload("8k", 1, 32, 2, 256, 4096, 8, 2048, 2048, 4096, 1024),
    "32k": Workload("32k", 2, 32, 2, 256, 28672, 8, 2048, 2048, 4096, 4096),
    "128k": Workload("128k", 3, 32, 2, 256, 126973, 8, 2048, 2048, 3548, 16316),
    "1m": Workload("1m", 4, 32, 2, 256, 1044480, 8, 2048, 2048, 4096, 131072,
                   k_mult=4.0),
}


def custom(name="custom", **kw):
    """A Workload with explicit fields (used for edge cases in the tests)."""
    base = dict(seed=0, nq=4, nkv=1, hd=64, cache_len=0, P=1, head_rows=0,
                tail_rows=0, real_rows=0, shard_cap=1, k_mult=1.0,
                interleave=1)
    base.update(kw)
    return Workload(name=name, **base)


def with_fields(w, **kw):
    return replace(w, **kw)


def generate(w):
    """Seeded token-order tensors (CPU, bf16) for workload ``w``."""
    g = torch.Generator().manual_seed(w.seed)
    C, L = w.q_rows, w.cache_len

    def draw(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)

    q = draw(C, w.nq, w.hd)
    k_cache_tok = draw(L, w.nkv, w.hd)
    v_cache_tok = draw(L, w.nkv, w.hd)
    k_cur = draw(C, w.nkv, w.hd)
    v_cur = draw(C, w.nkv, w.hd)
    if w.k_mult != 1.0:
        k_cache_tok = k_cache_tok * w.k_mult
        k_cur = k_cur * w.k_mult
    if w.real_rows < C:
        q[w.real_rows:] = float("nan")
        k_cur[w.real_rows:] = float("nan")
        v_cur[w.real_rows:] = float("nan")
    return dict(q=q, k_cache_tok=k_cache_tok, v_cache_tok=v_cache_tok,
                k_cur=k_cur, v_cur=v_cur)
