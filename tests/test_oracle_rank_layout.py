"""Pins for the oracle's rank layout (chunk rows at explicit positions).

The pages keep a two-sequence (head, tail) structure in the current phase
(vLLM tpu-inference pull request "PCP: in-kernel ring cache phase, fused
with the current phase", Design section) and hand the current K/V over in
token order (Design, subtlety 1).  A rank's query rows are then two pieces of
the chunk at arbitrary chunk positions.  What fixes the expected values here,
other than the oracle itself:
  * brute force: an independent scalar loop (math.fsum) whose row at chunk
    position p lists cache tokens and current tokens 0..p explicitly;
  * reduction to the contiguous layout, which the other oracle pins fix: a
    rank's rows must equal the same chunk positions computed on the whole
    chunk with rows at their own positions;
  * the load-balanced piece assignment: the ranks' pieces tile the chunk
    exactly once and give every rank the same number of causal
    (row, current key) pairs;
  * mutation checks: ignoring the positions, or an off-by-one in them, is
    caught.
"""
import math
import types

import numpy as np
import pytest

import oracle
from oracle import attention as att


def rand_case(seed, C, L, NQ, NKV, HD):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)
    return dict(q=r(C, NQ, HD), k_tok=r(L, NKV, HD), v_tok=r(L, NKV, HD),
                k_cur=r(C, NKV, HD), v_cur=r(C, NKV, HD))


def brute_force_pos(q, k_tok, v_tok, k_cur, v_cur, scale, positions):
    """Row i (chunk position positions[i]) over every cached token, then the
    current tokens 0..positions[i], summed with fsum."""
    C, NQ, HD = q.shape
    L, NKV = k_tok.shape[0], k_cur.shape[1]
    G = NQ // NKV
    out = {}
    for i, p in enumerate(positions):
        for h in range(NQ):
            g = h // G
            keys = [(k_tok[t, g], v_tok[t, g]) for t in range(L)]
            keys += [(k_cur[j, g], v_cur[j, g]) for j in range(p + 1)]
            s = [scale * math.fsum(float(q[i, h, d]) * float(k[d]) for d in range(HD))
                 for k, _ in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            o = [math.fsum(wj * float(v[d]) for wj, (_, v) in zip(w, keys)) / l
                 for d in range(HD)]
            out[(i, h)] = (np.array(o), m + math.log(l))
    return out


@pytest.mark.parametrize("L,head,tail,hp,tp,N", [(5, 2, 3, 3, 9, 12), (0, 3, 2, 0, 6, 8),
                                                  (4, 1, 4, 7, 1, 8), (3, 4, 0, 2, 0, 6)])
def test_positions_match_brute_force(L, head, tail, hp, tp, N):
    c = rand_case(L * 7 + head, head + tail, L, 4, 2, 3)
    c["k_cur"] = np.random.default_rng(99).standard_normal((N, 2, 3))
    c["v_cur"] = np.random.default_rng(98).standard_normal((N, 2, 3))
    pos = oracle.rank_positions(head, tail, hp, tp)
    ref = brute_force_pos(c["q"], c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"], 0.6, pos)
    out, lse = oracle.attention_rows(c["q"], c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"],
                                     range(head + tail), 0.6, positions=pos)
    P = 3
    cap = max(oracle.shard_lengths(L, P, 1) + [1])
    kc = oracle.stripe(c["k_tok"], P, 1, cap, np.nan)
    vc = oracle.stripe(c["v_tok"], P, 1, cap, np.nan)
    out2, lse2 = oracle.ring_online(c["q"], kc, vc, c["k_cur"], c["v_cur"], L, P, 1,
                                    range(head + tail), 0.6, ring_start=1, block=2,
                                    positions=pos)
    for (i, h), (o, l) in ref.items():
        assert np.abs(out[i, h] - o).max() < 1e-12 and abs(lse[h, i] - l) < 1e-12
        assert np.abs(out2[i, h] - o).max() < 1e-12 and abs(lse2[h, i] - l) < 1e-12


@pytest.mark.parametrize("ranks,r", [(2, 0), (2, 1), (4, 1), (4, 3)])
def test_rank_rows_equal_contiguous_chunk(ranks, r):
    """Rank r's rows, with the whole chunk's token-order K/V, equal the same
    positions of the contiguous layout (rows at their own positions)."""
    chunk, L = 16 * ranks, 11
    c = rand_case(ranks * 10 + r, chunk, L, 4, 2, 8)
    hp, tp, piece = oracle.zigzag_pieces(chunk, ranks, r)
    pos = oracle.rank_positions(piece, piece, hp, tp)
    q_rank = c["q"][pos]
    out, lse = oracle.attention_rows(q_rank, c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"],
                                     range(2 * piece), 0.35, positions=pos)
    ref, ref_lse = oracle.attention_rows(c["q"], c["k_tok"], c["v_tok"], c["k_cur"],
                                         c["v_cur"], pos.tolist(), 0.35)
    assert np.abs(out - ref).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


@pytest.mark.parametrize("ranks", [1, 2, 4, 8])
def test_zigzag_pieces_tile_the_chunk_and_balance_work(ranks):
    chunk = 2 * ranks * 32
    seen, work = [], []
    for r in range(ranks):
        hp, tp, piece = oracle.zigzag_pieces(chunk, ranks, r)
        pos = oracle.rank_positions(piece, piece, hp, tp)
        seen += pos.tolist()
        work.append(int((pos + 1).sum()))
    assert sorted(seen) == list(range(chunk))
    assert len(set(work)) == 1


def _mutant(old, new):
    src = open(att.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("pos = np.arange(C) if positions is None else np.asarray(positions)", "pos = np.arange(C)"),
    ("tail_pos + np.arange(tail_rows)", "tail_pos + 1 + np.arange(tail_rows)"),
    ("return r * piece, (2 * ranks - 1 - r) * piece, piece", "return r * piece, (ranks + r) * piece, piece"),
])
def test_position_mutations_are_caught(old, new):
    mod = _mutant(old, new)
    caught = False
    try:
        c = rand_case(5, 5, 4, 4, 2, 3)
        c["k_cur"] = np.random.default_rng(7).standard_normal((12, 2, 3))
        c["v_cur"] = np.random.default_rng(8).standard_normal((12, 2, 3))
        pos = mod.rank_positions(2, 3, 3, 8)
        ref = brute_force_pos(c["q"], c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"], 0.6,
                              oracle.rank_positions(2, 3, 3, 8))
        out, lse = mod.attention_rows(c["q"], c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"],
                                      range(5), 0.6, positions=pos)
        for (i, h), (o, l) in ref.items():
            if np.abs(out[i, h] - o).max() > 1e-9 or abs(lse[h, i] - l) > 1e-9:
                caught = True
        seen, work = [], []
        for r in range(4):
            hp, tp, piece = mod.zigzag_pieces(64, 4, r)
            p = oracle.rank_positions(piece, piece, hp, tp)
            seen += p.tolist()
            work.append(int((p + 1).sum()))
        if sorted(seen) != list(range(64)) or len(set(work)) != 1:
            caught = True
    except (ValueError, IndexError, AssertionError):
        caught = True
    assert caught
