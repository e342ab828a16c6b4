"""Striped KV-cache geometry, written from its definition (test infrastructure).

Source: vLLM tpu-inference pull request "PCP: in-kernel ring cache phase,
fused with the current phase", Design section (each rank holds a striped
shard of the KV cache that travels the ring) and Testing section (the strided
KV-cache write is bit-exact against the gather path).  The pages do not fix
the stripe unit; the reading used here is round-robin over ranks in units of
``interleave`` consecutive tokens (interleave = 1: token round-robin, shard s
receives every P-th token).  Attention over the cache does not depend on the
stripe unit or on the visit order, because every cached token is visible to
every chunk row.

Layout of a striped cache: ``[P, shard_cap, NKV, HD]``; slot ``j`` of shard
``s`` holds the token whose position maps to ``(s, j)``.
"""
import numpy as np


def stripe_position(p, P, interleave):
    """Shard and slot of the cached token at global position ``p``.

    Positions are grouped into units of ``interleave`` tokens; unit ``u``
    goes to shard ``u mod P`` as that shard's ``u div P``-th unit.
    """
    u = p // interleave
    return u % P, (u // P) * interleave + p % interleave


def shard_lengths(cache_len, P, interleave):
    """Number of valid slots in each shard when positions [0, cache_len) are
    cached.  Closed form of counting ``stripe_position`` over the positions:
    every full round of ``P * interleave`` tokens gives each shard
    ``interleave`` tokens; the remainder fills shards in order."""
    round_len = P * interleave
    full, rem = divmod(cache_len, round_len)
    return [full * interleave + min(max(rem - s * interleave, 0), interleave)
            for s in range(P)]


def stripe(tokens, P, interleave, shard_cap, fill=np.nan):
    """Token-order ``[L, ...]`` -> striped ``[P, shard_cap, ...]``; slots that
    hold no token are set to ``fill``.  (``stripe_position`` is applied to
    all positions at once as integer array arithmetic.)"""
    L = tokens.shape[0]
    out = np.full((P, shard_cap) + tokens.shape[1:], fill, dtype=tokens.dtype)
    s, j = stripe_position(np.arange(L, dtype=np.int64), P, interleave)
    out[s, j] = tokens
    return out


def destripe(cache, cache_len, P, interleave):
    """Striped ``[P, shard_cap, ...]`` -> token order ``[cache_len, ...]``.
    Only slots below each shard's length are read."""
    s, j = stripe_position(np.arange(cache_len, dtype=np.int64), P, interleave)
    return cache[s, j]


def kv_cache_write_ref(k_cache, v_cache, k_cur, v_cur, n_tokens, cache_len,
                       P, interleave):
    """Strided KV-cache write: current token ``t`` (global position
    ``cache_len + t``) is copied bit for bit into its shard slot.  Operates on
    copies of the caches (any dtype, e.g. uint16 bf16 bit patterns) and
    returns them; all other slots are left untouched."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    for t in range(n_tokens):
        s, j = stripe_position(cache_len + t, P, interleave)
        kc[s, j] = k_cur[t]
        vc[s, j] = v_cur[t]
    return kc, vc
