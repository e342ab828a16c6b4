"""Pins for the oracle's attention (plain definition and method walk).

What fixes the expected values here, other than the oracle itself:
  * a hand-worked example (tests/golden/attention_worked.json);
  * brute force: an independent scalar loop with exactly rounded sums
    (math.fsum) over explicitly listed visible keys, on tiny inputs;
  * closed forms: q = 0 gives the mean of the visible values and
    lse = ln(number of visible keys); constant V gives that constant; with
    an empty cache, row 0 returns v_cur[0] with lse = scale * q . k_cur[0];
  * the two-pass identity: cache-only and causal-current-only partials
    merged by log-sum-exp equal the one-pass result;
  * invariance to shard count, stripe unit, ring start and block size;
  * causality: changing current tokens after row i (even to NaN / Inf)
    leaves row i bitwise unchanged, changing earlier ones does not;
  * NaN in unused shard slots never reaches the result;
  * mutation checks: plausible mistakes planted in a copy of the oracle
    (off-by-one causal bound, wrong GQA head map, dropped cache, wrong sign)
    are caught by these pins.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import attention as att

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, C, L, NQ, NKV, HD, dtype=np.float64):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s).astype(dtype)
    return dict(q=r(C, NQ, HD), k_tok=r(L, NKV, HD), v_tok=r(L, NKV, HD),
                k_cur=r(C, NKV, HD), v_cur=r(C, NKV, HD))


def brute_force(q, k_tok, v_tok, k_cur, v_cur, scale, rows=None):
    """Independent scalar evaluation: list row i's visible keys explicitly
    (every cached token, then current tokens 0..i) and sum with fsum."""
    C, NQ, HD = q.shape
    L = k_tok.shape[0]
    NKV = k_cur.shape[1]
    G = NQ // NKV
    rows = range(C) if rows is None else rows
    out = {}
    for i in rows:
        for h in range(NQ):
            g = h // G
            keys = [(k_tok[t, g], v_tok[t, g]) for t in range(L)]
            keys += [(k_cur[j, g], v_cur[j, g]) for j in range(i + 1)]
            s = [scale * math.fsum(float(q[i, h, d]) * float(k[d]) for d in range(HD))
                 for k, _ in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            o = [math.fsum(wj * float(v[d]) for wj, (_, v) in zip(w, keys)) / l
                 for d in range(HD)]
            out[(i, h)] = (o, m + math.log(l))
    return out


def striped(case, P, I, fill=np.nan):
    L = case["k_tok"].shape[0]
    cap = max(oracle.shard_lengths(L, P, I) + [1])
    return (oracle.stripe(case["k_tok"], P, I, cap, fill),
            oracle.stripe(case["v_tok"], P, I, cap, fill))


def load_worked():
    d = json.load(open(os.path.join(GOLDEN, "attention_worked.json")))
    a = lambda k: np.array(d[k], dtype=np.float64)
    case = dict(q=a("q"), k_tok=a("k_cache_tok"), v_tok=a("v_cache_tok"),
                k_cur=a("k_cur"), v_cur=a("v_cur"))
    out = np.array([[[float(Fraction(x)) for x in hd] for hd in row] for row in d["out"]])
    lse = np.log(np.array(d["lse_exp"], dtype=np.float64))
    return case, d, out, lse


def check_worked(mod):
    case, d, out_e, lse_e = load_worked()
    scale = math.log(2.0)
    out, lse = mod.attention_rows(case["q"], case["k_tok"], case["v_tok"],
                                  case["k_cur"], case["v_cur"], range(2), scale)
    return np.abs(out - out_e).max() < 1e-14 and np.abs(lse - lse_e).max() < 1e-14


def test_worked_example_plain():
    assert check_worked(att)


def test_worked_example_striped_and_online():
    case, d, out_e, lse_e = load_worked()
    scale = math.log(2.0)
    kc, vc = striped(case, d["P"], d["interleave"])
    for fn in (oracle.ring_attention, oracle.ring_online):
        out, lse = fn(case["q"], kc, vc, case["k_cur"], case["v_cur"], 2, d["P"],
                      d["interleave"], range(2), scale)
        assert np.abs(out - out_e).max() < 1e-14
        assert np.abs(lse - lse_e).max() < 1e-14


@pytest.mark.parametrize("seed,C,L,NQ,NKV,HD,P,I", [
    (0, 5, 7, 2, 1, 3, 2, 1), (1, 8, 11, 4, 2, 4, 3, 1), (2, 6, 0, 2, 2, 2, 1, 1),
    (3, 4, 9, 6, 3, 4, 3, 2), (4, 3, 2, 1, 1, 4, 3, 1)])
def test_bruteforce_tiny(seed, C, L, NQ, NKV, HD, P, I):
    case = rand_case(seed, C, L, NQ, NKV, HD)
    scale = 0.37
    ref = brute_force(case["q"], case["k_tok"], case["v_tok"], case["k_cur"], case["v_cur"], scale)
    kc, vc = striped(case, P, I)
    results = [
        oracle.attention_rows(case["q"], case["k_tok"], case["v_tok"], case["k_cur"],
                              case["v_cur"], range(C), scale),
        oracle.ring_attention(case["q"], kc, vc, case["k_cur"], case["v_cur"], L, P, I,
                              range(C), scale),
        oracle.ring_online(case["q"], kc, vc, case["k_cur"], case["v_cur"], L, P, I,
                           range(C), scale, ring_start=P - 1, block=2),
    ]
    for out, lse in results:
        for (i, h), (o, l) in ref.items():
            assert np.abs(out[i, h] - np.array(o)).max() < 1e-12
            assert abs(lse[h, i] - l) < 1e-12


def test_closed_form_q_zero():
    case = rand_case(5, 6, 13, 4, 2, 8)
    case["q"][:] = 0.0
    out, lse = oracle.attention_rows(case["q"], case["k_tok"], case["v_tok"], case["k_cur"],
                                     case["v_cur"], range(6), 0.5)
    G = 2
    for i in range(6):
        n = 13 + i + 1
        assert np.allclose(lse[:, i], math.log(n), atol=1e-13, rtol=0)
        for h in range(4):
            vis = np.concatenate([case["v_tok"][:, h // G], case["v_cur"][:i + 1, h // G]])
            assert np.abs(out[i, h] - vis.mean(axis=0)).max() < 1e-13


def test_closed_form_constant_v_per_kv_head():
    case = rand_case(6, 5, 9, 6, 3, 4)
    consts = np.array([[1.5, -2.0, 0.25, 3.0], [-7.0, 0.5, 2.0, 1.0], [4.0, 4.0, -1.0, 0.0]])
    for g in range(3):
        case["v_tok"][:, g] = consts[g]
        case["v_cur"][:, g] = consts[g]
    kc, vc = striped(case, 3, 1)
    for fn in (oracle.ring_attention, oracle.ring_online):
        out, _ = fn(case["q"], kc, vc, case["k_cur"], case["v_cur"], 9, 3, 1, range(5), 0.8)
        for h in range(6):  # head h reads kv head h // 2
            assert np.abs(out[:, h] - consts[h // 2]).max() < 1e-12


def test_closed_form_empty_cache_first_row():
    case = rand_case(7, 4, 0, 3, 1, 5)
    scale = 0.3
    out, lse = oracle.attention_rows(case["q"], case["k_tok"], case["v_tok"], case["k_cur"],
                                     case["v_cur"], [0], scale)
    for h in range(3):
        assert np.array_equal(out[0, h], case["v_cur"][0, 0])
        assert abs(lse[h, 0] - scale * float(case["q"][0, h] @ case["k_cur"][0, 0])) < 1e-13


@pytest.mark.parametrize("L", [0, 1, 17])
def test_two_pass_merge_identity(L):
    case = rand_case(8 + L, 7, L, 4, 2, 6)
    args = (case["q"], case["k_tok"], case["v_tok"], case["k_cur"], case["v_cur"], range(7), 0.6)
    o, l = oracle.attention_rows(*args)
    o1, l1 = oracle.attention_rows(*args, current=False)
    o2, l2 = oracle.attention_rows(*args, cache=False)
    om, lm = oracle.two_pass_merge(o1, l1, o2, l2)
    assert np.abs(om - o).max() < 1e-12 and np.abs(lm - l).max() < 1e-12


def test_invariance_shards_order_blocks():
    case = rand_case(9, 6, 37, 4, 2, 8)
    base, lbase = oracle.attention_rows(case["q"], case["k_tok"], case["v_tok"], case["k_cur"],
                                        case["v_cur"], range(6), 0.45)
    for P in (1, 2, 3, 8):
        for I in (1, 16):
            kc, vc = striped(case, P, I)
            for start in sorted({0, P - 1}):
                for block in (1, 5, 64):
                    o, l = oracle.ring_online(case["q"], kc, vc, case["k_cur"], case["v_cur"],
                                              37, P, I, range(6), 0.45, start, block)
                    assert np.abs(o - base).max() < 1e-12 and np.abs(l - lbase).max() < 1e-12


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, "random"])
def test_causal_future_perturbation(bad):
    case = rand_case(10, 8, 5, 4, 2, 4)
    args = lambda c: (c["q"], c["k_tok"], c["v_tok"], c["k_cur"], c["v_cur"], range(8), 0.5)
    out, lse = oracle.attention_rows(*args(case))
    for i in range(7):
        pert = {k: v.copy() for k, v in case.items()}
        fill = np.random.default_rng(i).standard_normal(pert["k_cur"][i + 1:].shape) * 9 \
            if bad == "random" else bad
        pert["k_cur"][i + 1:] = fill
        pert["v_cur"][i + 1:] = fill
        o2, l2 = oracle.attention_rows(*args(pert))
        assert np.array_equal(o2[:i + 1], out[:i + 1]) and np.array_equal(l2[:, :i + 1], lse[:, :i + 1])
    # teeth: changing token j <= i changes row i
    pert = {k: v.copy() for k, v in case.items()}
    pert["v_cur"][3] += 1.0
    o2, _ = oracle.attention_rows(*args(pert))
    assert np.array_equal(o2[:3], out[:3]) and (np.abs(o2[3:] - out[3:]).max(axis=(1, 2)) > 1e-6).all()


def test_unused_shard_slots_never_read():
    case = rand_case(11, 5, 21, 2, 1, 4)
    for P, I in ((3, 1), (4, 2), (8, 1)):
        L = 21
        cap = max(oracle.shard_lengths(L, P, I)) + 6
        kc_nan = oracle.stripe(case["k_tok"], P, I, cap, np.nan)
        vc_nan = oracle.stripe(case["v_tok"], P, I, cap, np.nan)
        kc_zero = oracle.stripe(case["k_tok"], P, I, cap, 0.0)
        vc_zero = oracle.stripe(case["v_tok"], P, I, cap, 0.0)
        for fn in (oracle.ring_attention, oracle.ring_online):
            a = fn(case["q"], kc_nan, vc_nan, case["k_cur"], case["v_cur"], L, P, I, range(5), 0.5)
            b = fn(case["q"], kc_zero, vc_zero, case["k_cur"], case["v_cur"], L, P, I, range(5), 0.5)
            assert np.isfinite(a[0]).all()
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bf16_bits_decode():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x7F80 = +inf, 0x0001 = 2^-133
    got = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x3E80, 0x7F80, 0x0001], np.uint16))
    assert got[:4].tolist() == [1.0, -2.0, 0.25, math.inf] and got[4] == 2.0 ** -133


def test_default_scale_values():
    """default_scale is the softmax temperature 1/sqrt(HD) of the pages'
    attention; the head dims this library takes have exact values (HD 64,
    256: powers of two) that a wrong formula (1/HD, sqrt(HD), 1/sqrt(HD/2))
    would miss.  The needle closed forms take their score scale from it, so
    this pins it outside them."""
    assert att.default_scale(64) == 0.125
    assert att.default_scale(256) == 0.0625
    assert att.default_scale(4) == 0.5
    assert abs(att.default_scale(128) - 2.0 ** -3.5) < 1e-16


# --- mutation checks: a plausible mistake in the oracle must fail a pin ---

MUTATIONS = [
    ("Kn[:(pos[i] + 1 if current else 0)]", "Kn[:(pos[i] + 2 if current else 0)]"),  # causal off by one
    ("hs = slice(g * G, (g + 1) * G)", "hs = slice(g, NQ, NKV)"),               # interleaved GQA map
    ("Oc = (Ec.reshape", "Oc = 0 * (Ec.reshape"),                               # cache values dropped
    ("Sc = scale * (Qb", "Sc = -scale * (Qb"),                                  # sign of cache scores
    ("lse[hs, r0 + b] = m[b] + np.log(l)", "lse[hs, r0 + b] = np.log(l)"),      # max dropped from lse
    ("En @ Vn[:En.shape[1]]", "En @ Vn[1:En.shape[1] + 1]"),                    # value rows shifted
    ("Kc = np.ascontiguousarray(np.asarray(k_tok[:L, g]", "Kc = np.ascontiguousarray(np.asarray(k_tok[:L, 0]"),  # kv head ignored
]


def _mutant(old, new):
    import types
    src = open(att.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    # the first occurrence is in attention_rows, the function the pins call
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_mutations_are_caught(old, new):
    mod = _mutant(old, new)
    try:  # a mutant that crashes is caught too
        caught = not check_worked(mod)
        case = rand_case(12, 5, 6, 4, 2, 3)
        ref = brute_force(case["q"], case["k_tok"], case["v_tok"], case["k_cur"], case["v_cur"],
                          0.5)
        out, lse = mod.attention_rows(case["q"], case["k_tok"], case["v_tok"], case["k_cur"],
                                      case["v_cur"], range(4), 0.5)
        for (i, h), (o, l) in ref.items():
            if i < 4 and (np.abs(out[i, h] - np.array(o)).max() > 1e-9 or abs(lse[h, i] - l) > 1e-9):
                caught = True
    except (ValueError, IndexError):
        caught = True
    assert caught


@pytest.mark.parametrize("L", [256, 1000])
def test_closed_form_needles(L):
    """The needle inputs (one matching cache key per row, all other keys and
    values zero) have a closed-form softmax; the oracle reproduces it.  The
    GPU tests use the same closed form where the cache is too large for the
    oracle."""
    from helpers import (NEEDLE_G, NEEDLE_HD, NEEDLE_T, needle_expected, needle_positions,
                         needle_q, needle_values)
    pos = needle_positions(L, seed=1)
    w = needle_values(seed=1)
    k_tok = np.zeros((L, 1, NEEDLE_HD))
    v_tok = np.zeros((L, 1, NEEDLE_HD))
    r = np.arange(NEEDLE_T * NEEDLE_G)
    k_tok[pos, 0, r] = 16.0
    v_tok[pos, 0] = w.double().numpy()
    q = needle_q().double().numpy()
    zeros = np.zeros((NEEDLE_T, 1, NEEDLE_HD))
    scale = att.default_scale(NEEDLE_HD)
    o, l = oracle.attention_rows(q, k_tok, v_tok, zeros, zeros, range(NEEDLE_T), scale)
    o_ref, l_ref = needle_expected(L, w, scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(l - l_ref).max() < 1e-12
    # the needle carries a weight well inside (0, 1): both terms matter
    wt = math.exp(16.0) / (math.exp(16.0) + L)
    assert 0.5 < wt < 1.0 - 1e-5


def test_closed_form_needles_in_current_chunk():
    """The same closed form with no cache, the needles in the current chunk
    and the 16 query tokens at chunk positions pos0..pos0+15."""
    from helpers import (NEEDLE_G, NEEDLE_HD, NEEDLE_T, needle_expected, needle_positions,
                         needle_q, needle_values)
    N = 700
    pos0 = N - NEEDLE_T
    pos = needle_positions(pos0, seed=4)
    w = needle_values(seed=4)
    k_cur = np.zeros((N, 1, NEEDLE_HD))
    v_cur = np.zeros((N, 1, NEEDLE_HD))
    k_cur[pos, 0, np.arange(NEEDLE_T * NEEDLE_G)] = 16.0
    v_cur[pos, 0] = w.double().numpy()
    empty = np.zeros((0, 1, NEEDLE_HD))
    scale = att.default_scale(NEEDLE_HD)
    o, l = oracle.attention_rows(needle_q().double().numpy(), empty, empty, k_cur, v_cur,
                                 range(NEEDLE_T), scale, positions=pos0 + np.arange(NEEDLE_T))
    o_ref, l_ref = needle_expected(0, w, scale, pos0=pos0)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(l - l_ref).max() < 1e-12
