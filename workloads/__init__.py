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
``v_cache_tok [L, NKV, HD]``, ``k_cur [N, NKV, HD]``, ``v_cur [N, NKV, HD]``
as float32 ``randn`` rounded to bf16 (round-to-nearest-even); N = C in the
contiguous layout.  ``k_mult`` multiplies both key tensors after rounding (a
power of two, so exact).  Rows ``>= real_rows`` of ``q`` are pads, and so are
current tokens ``>= cur_real``; both are set to NaN.

Rank layout (the PCP page's two-sequence (head, tail) current phase): the
query rows are a head piece at chunk position ``head_pos`` and a tail piece
at ``tail_pos``, and the current K/V are the whole chunk (``cur_len`` tokens,
token order).  ``rank_share`` builds the load-balanced share of rank ``r``:
pieces ``r`` and ``2R-1-r`` of a chunk cut into ``2R``.
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
    head_pos: int = 0       # chunk position of the first head row
    tail_pos: int = -1      # chunk position of the first tail row (-1: after the head)
    cur_len: int = -1       # current tokens in token order (-1: q_rows)
    cur_real: int = -1      # real current tokens (-1: real_rows)

    @property
    def q_rows(self):
        return self.head_rows + self.tail_rows

    @property
    def tail_start(self):
        return self.head_pos + self.head_rows if self.tail_pos < 0 else self.tail_pos

    @property
    def n_cur(self):
        return self.q_rows if self.cur_len < 0 else self.cur_len

    @property
    def n_cur_real(self):
        return self.real_rows if self.cur_real < 0 else self.cur_real

    @property
    def positions(self):
        """Chunk position of each query row."""
        return list(range(self.head_pos, self.head_pos + self.head_rows)) + \
            list(range(self.tail_start, self.tail_start + self.tail_rows))

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
    # 512k: the context the PCP page's Performance section names beside 1M
    # (not in its table); the 4k chunk after 508k cached tokens
    "512k": Workload("512k", 5, 32, 2, 256, 520192, 8, 2048, 2048, 4096, 65536),
}


def rank_share(w, ranks, r, name=None):
    """Rank r's load-balanced share of workload ``w``'s chunk (``w`` in the
    contiguous layout): pieces r and 2*ranks-1-r of the q_rows-token chunk;
    the chunk's real tokens are ``w.real_rows`` (pads at its end)."""
    chunk = w.q_rows
    piece = chunk // (2 * ranks)
    assert piece * 2 * ranks == chunk
    hp, tp = r * piece, (2 * ranks - 1 - r) * piece
    real_head = max(0, min(piece, w.real_rows - hp))
    real_tail = max(0, min(piece, w.real_rows - tp))
    assert real_tail == 0 or real_head == piece  # pads only at the end of the rank's rows
    return replace(w, name=name or f"{w.name}_rank{r}of{ranks}", head_rows=piece,
                   tail_rows=piece, real_rows=real_head + real_tail, head_pos=hp, tail_pos=tp,
                   cur_len=chunk, cur_real=w.real_rows)


# Load-balanced rank shares (the PCP page's pcp=8 over a 4k chunk): 2 x 256
# query rows per rank, the whole chunk's current K/V.  128k rank 0's tail
# piece [3840, 4096) lies past the chunk's 3548 real tokens (an all-pad tail);
# rank 2's tail [3328, 3584) is partly real.
CONFIGS["tiny_rank1of2"] = rank_share(CONFIGS["tiny"], 2, 1)
CONFIGS["32k_rank3of8"] = rank_share(CONFIGS["32k"], 8, 3)
CONFIGS["128k_rank0of8"] = rank_share(CONFIGS["128k"], 8, 0)
CONFIGS["128k_rank2of8"] = rank_share(CONFIGS["128k"], 8, 2)
# long-context rank shares (a few hundred rows over a long cache: the split
# walk's case)
CONFIGS["512k_rank3of8"] = rank_share(CONFIGS["512k"], 8, 3)
CONFIGS["1m_rank3of8"] = rank_share(CONFIGS["1m"], 8, 3)


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
    k_cur = draw(w.n_cur, w.nkv, w.hd)
    v_cur = draw(w.n_cur, w.nkv, w.hd)
    if w.k_mult != 1.0:
        k_cache_tok = k_cache_tok * w.k_mult
        k_cur = k_cur * w.k_mult
    if w.real_rows < C:
        q[w.real_rows:] = float("nan")
    if w.n_cur_real < w.n_cur:
        k_cur[w.n_cur_real:] = float("nan")
        v_cur[w.n_cur_real:] = float("nan")
    return dict(q=q, k_cache_tok=k_cache_tok, v_cache_tok=v_cache_tok,
                k_cur=k_cur, v_cur=v_cur)
