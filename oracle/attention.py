"""Fused ring + current attention in fp64 (test infrastructure).

Source: vLLM tpu-inference pull request "PCP: in-kernel ring cache phase,
fused with the current phase".
  * Summary: ring cache rounds and the causal current phase run in one launch
    sharing one online softmax; no separate current launch, no LSE merge.
  * Design: per query block the key walk first visits the ring region (cache
    shards, no causal mask, bounded by each shard's valid length), then the
    current-KV blocks with the causal mask; current KV is handed over in
    token order.
  * Testing: ring must agree with the gather-the-cache strategy.

Agreement with the gather strategy means the fused launch computes exactly
(up to rounding) plain softmax attention of chunk row ``i`` -- global
position ``cache_len + i`` -- over the whole cache followed by current tokens
``0..i``.  ``attention_rows`` is that definition.  ``ring_online`` takes the
method's steps (ring rounds, then current blocks, one running (m, l, acc)).
``two_pass_merge`` is the log-sum-exp merge of the removed two-launch variant
(Summary section), kept only as an identity to check the others against.

Conventions (readings where the pages are silent): GQA heads are contiguous
groups, query head ``h`` uses KV head ``h // (NQ // NKV)``; ``lse`` is the
natural-log log-sum-exp of the scaled scores, laid out ``[NQ, rows]``.

Rank layout (Design section: the current phase keeps a two-sequence (head,
tail) structure).  In the default layout chunk row ``i`` sits at chunk
position ``i``.  With ``positions`` given, row ``i`` of the query tensor sits
at chunk position ``positions[i]`` while the current K/V stay in token order
(Design subtlety 1), so row ``i`` sees current tokens ``0..positions[i]``.
``rank_positions`` gives the positions of one rank's (head, tail) pieces.
"""
import math
import numpy as np


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 / int16 array) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rank_positions(head_rows, tail_rows, head_pos, tail_pos):
    """Chunk positions of a rank's query rows: the head piece (rows
    ``0..head_rows-1``) starts at chunk position ``head_pos``, the tail piece
    (the remaining ``tail_rows`` rows) at ``tail_pos``."""
    return np.concatenate([head_pos + np.arange(head_rows),
                           tail_pos + np.arange(tail_rows)]).astype(np.int64)


def zigzag_pieces(chunk, ranks, r):
    """(head_pos, tail_pos, piece) of rank ``r`` when a chunk of ``chunk``
    tokens is cut into ``2 * ranks`` equal pieces and rank ``r`` owns pieces
    ``r`` and ``2 * ranks - 1 - r`` (the load-balanced context-parallel
    layout: every rank gets one early and one late piece)."""
    piece = chunk // (2 * ranks)
    assert piece * 2 * ranks == chunk
    return r * piece, (2 * ranks - 1 - r) * piece, piece


def attention_rows(q, k_tok, v_tok, k_cur, v_cur, rows, scale,
                   cache=True, current=True, row_block=64, positions=None):
    """Softmax attention of the chosen chunk rows, plain definition.

    q      [C, NQ, HD]   chunk queries (any float dtype; bf16 values are exact)
    k_tok  [L, NKV, HD]  cached keys in token order (L = cache_len)
    v_tok  [L, NKV, HD]
    k_cur  [N, NKV, HD]  current keys in token order, row j at position L + j
    v_cur  [N, NKV, HD]
    rows   iterable of chunk row indices to evaluate (real rows only)
    positions  chunk position of each row of ``q`` (default: row i at i)

    Row ``i`` at chunk position ``p = positions[i]`` sees cache tokens
    ``0..L-1`` (if ``cache``) and current tokens ``0..p`` (if
    ``current``); its scores are ``scale * q . k`` in fp64, and
    ``out = sum_j e^(s_j - m) v_j / l``, ``l = sum_j e^(s_j - m)``,
    ``lse = m + ln l`` with ``m`` the row's max score.  The sum over j is
    taken in two parts: the cache part, identical for every row, as one
    matrix product over a block of rows, and the current part row by row.
    Current keys after row ``i`` are excluded by slicing, never multiplied
    by zero, so NaN or Inf stored there cannot reach the result.  Returns
    ``out [len(rows), NQ, HD]`` and ``lse [NQ, len(rows)]`` in float64; a
    row with no visible key gets out = 0 and lse = -inf.
    """
    rows = list(rows)
    C, NQ, HD = q.shape
    L = k_tok.shape[0] if cache else 0
    NKV = k_cur.shape[1]
    G = NQ // NKV
    pos = np.arange(C) if positions is None else np.asarray(positions)
    out = np.zeros((len(rows), NQ, HD))
    lse = np.full((NQ, len(rows)), -np.inf)
    for g in range(NKV):
        hs = slice(g * G, (g + 1) * G)
        Kc = np.ascontiguousarray(np.asarray(k_tok[:L, g], np.float64))       # [L, HD]
        Vc = np.ascontiguousarray(np.asarray(v_tok[:L, g], np.float64))
        Kn = np.asarray(k_cur[:, g], np.float64)                               # [C, HD]
        Vn = np.asarray(v_cur[:, g], np.float64)
        for r0 in range(0, len(rows), row_block):
            blk = rows[r0:r0 + row_block]
            nb = len(blk)
            Qb = np.stack([np.asarray(q[i, hs], np.float64) for i in blk])      # [nb, G, HD]
            Sc = scale * (Qb.reshape(nb * G, HD) @ Kc.T).reshape(nb, G, L)     # cache scores
            Sn = [scale * (Qb[b] @ Kn[:(pos[i] + 1 if current else 0)].T)     # current scores
                  for b, i in enumerate(blk)]                                  # [G, p+1] each
            # row max over both parts (-inf when a row sees nothing)
            m = np.full((nb, G), -np.inf)
            for b in range(nb):
                if L > 0:
                    m[b] = np.maximum(m[b], Sc[b].max(axis=1))
                if Sn[b].shape[1] > 0:
                    m[b] = np.maximum(m[b], Sn[b].max(axis=1))
            m_safe = np.where(np.isneginf(m), 0.0, m)
            Ec = np.exp(Sc - m_safe[:, :, None])                                # [nb, G, L]
            Oc = (Ec.reshape(nb * G, L) @ Vc).reshape(nb, G, HD)
            for b, i in enumerate(blk):
                En = np.exp(Sn[b] - m_safe[b][:, None])                          # [G, p+1]
                l = Ec[b].sum(axis=1) + En.sum(axis=1)
                if not (l > 0).all():
                    continue
                out[r0 + b, hs] = (Oc[b] + En @ Vn[:En.shape[1]]) / l[:, None]
                lse[hs, r0 + b] = m[b] + np.log(l)
    return out, lse


def ring_attention(q, k_cache, v_cache, k_cur, v_cur, cache_len, P,
                   interleave, rows, scale, positions=None):
    """The fused launch's result from a striped cache: de-stripe the shards
    with the cache map, then ``attention_rows``."""
    from .stripe import destripe
    k_tok = destripe(np.asarray(k_cache), cache_len, P, interleave)
    v_tok = destripe(np.asarray(v_cache), cache_len, P, interleave)
    return attention_rows(q, k_tok, v_tok, k_cur, v_cur, rows, scale,
                          positions=positions)


def ring_online(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, interleave,
                rows, scale, ring_start=0, block=64, positions=None):
    """The method's own walk, in fp64, one chunk row at a time.

    Per row: running max ``m`` = -inf, normaliser ``l`` = 0, accumulator
    ``acc`` = 0.  Ring region: for round k = 0..P-1 visit shard
    ``(ring_start - k) mod P`` and its valid slots in blocks of ``block``
    (no causal mask: every cached token precedes the chunk).  Current
    region: current tokens in blocks of ``block``, keeping only tokens at or
    before the row's chunk position (causal).  Each block updates the shared state with
    ``m' = max(m, max s)``, ``acc = e^(m-m') acc + sum e^(s-m') v``,
    ``l = e^(m-m') l + sum e^(s-m')``.  Finally ``out = acc / l`` and
    ``lse = m + ln l``.  Same return layout as ``attention_rows``.
    """
    from .stripe import shard_lengths
    rows = list(rows)
    C, NQ, HD = q.shape
    NKV = k_cur.shape[1]
    G = NQ // NKV
    lens = shard_lengths(cache_len, P, interleave)
    kc = np.asarray(k_cache, np.float64)
    vc = np.asarray(v_cache, np.float64)
    kcur = np.asarray(k_cur, np.float64)
    vcur = np.asarray(v_cur, np.float64)
    pos = np.arange(C) if positions is None else np.asarray(positions)
    out = np.zeros((len(rows), NQ, HD))
    lse = np.full((NQ, len(rows)), -np.inf)
    for r, i in enumerate(rows):
        qi = np.asarray(q[i], np.float64)
        for g in range(NKV):
            hs = slice(g * G, (g + 1) * G)
            m = np.full(G, -np.inf)
            l = np.zeros(G)
            acc = np.zeros((G, HD))

            def visit(kb, vb):
                nonlocal m, l, acc
                if kb.shape[0] == 0:
                    return
                s = scale * (qi[hs] @ kb.T)
                m_new = np.maximum(m, s.max(axis=1))
                alpha = np.exp(m - m_new)
                p = np.exp(s - m_new[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ vb
                m = m_new

            for k in range(P):                      # ring rounds
                s_id = (ring_start - k) % P
                for b0 in range(0, lens[s_id], block):
                    b1 = min(b0 + block, lens[s_id])
                    visit(kc[s_id, b0:b1, g], vc[s_id, b0:b1, g])
            for c0 in range(0, pos[i] + 1, block):   # current region, causal
                c1 = min(c0 + block, pos[i] + 1)
                visit(kcur[c0:c1, g], vcur[c0:c1, g])
            out[r, hs] = acc / l[:, None]
            lse[hs, r] = m + np.log(l)
    return out, lse


def two_pass_merge(o1, lse1, o2, lse2):
    """Log-sum-exp merge of two partial attentions over disjoint key sets
    (the step of the removed two-launch variant).  ``o*`` are
    ``[rows, NQ, HD]``, ``lse*`` are ``[NQ, rows]``."""
    lse = np.logaddexp(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - lse)).T[:, :, None]
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - lse)).T[:, :, None]
    return w1 * o1 + w2 * o2, lse


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
