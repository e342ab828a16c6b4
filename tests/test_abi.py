"""The C ABI library loads, exports every entry point its header declares,
and rejects bad arguments on the host before any HIP call.

Every validation case below is invalid in at least one argument, so nothing
is ever launched and the fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import context_causal_attention_ring_amd as ra
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000  # aligned fake device address; never dereferenced


def header_functions():
    src = open(os.path.join(ROOT, "include", "ringattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_header_declares_the_binding_names():
    assert header_functions() == set(ra.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ra.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert ra.ra_version().startswith("libringattn")


@pytest.mark.parametrize("P,I", [(1, 1), (2, 1), (3, 2), (8, 1), (8, 16), (5, 3)])
def test_shard_len_matches_oracle(P, I):
    for L in (0, 1, 2, 7, 511, 512, 126973, 1044480):
        exp = oracle.shard_lengths(L, P, I)
        got = [ra.ra_shard_len(L, P, ra.StripeLayout(I, 0), s) for s in range(P)]
        assert got == exp


def dims(**kw):
    base = dict(num_q_heads=4, num_kv_heads=1, head_dim=64, q_rows=128, head_rows=64,
                real_rows=128, head_pos=0, tail_pos=64, cur_len=128, shard_cap=320, scale=0.0,
                out_dtype=0)
    base.update(kw)
    return ra.Dims(**base)


def call_prefill(d, cache_len=512, P=2, layout=(1, 0), ptrs=None, out=FAKE + 0x8000000,
                 lse=None):
    q, kc, vc, kcur, vcur = ptrs or (FAKE, FAKE + 0x1000000, FAKE + 0x2000000,
                                     FAKE + 0x3000000, FAKE + 0x4000000)
    return ra.lib().ring_attn_prefill(q, kc, vc, kcur, vcur, cache_len, P,
                                      ra.StripeLayout(*layout), out, lse, ctypes.byref(d), None)


BAD_PREFILL = [
    (dict(d=dims(num_q_heads=6, num_kv_heads=4)), 1, "multiple"),
    (dict(d=dims(head_dim=96)), 2, "head_dim"),
    (dict(d=dims(num_kv_heads=0)), 1, ">= 1"),
    (dict(d=dims(), P=0), 1, "P must"),
    (dict(d=dims(), layout=(0, 0)), 1, "interleave"),
    (dict(d=dims(), layout=(1, 2)), 1, "ring_start"),
    (dict(d=dims(), cache_len=-1), 1, "cache_len"),
    (dict(d=dims(shard_cap=255)), 1, "shard_cap"),
    (dict(d=dims(real_rows=129)), 1, "real_rows"),
    (dict(d=dims(head_rows=-1)), 1, "head_rows"),
    (dict(d=dims(q_rows=-5, real_rows=0, head_rows=0)), 1, "q_rows"),
    (dict(d=dims(out_dtype=7)), 1, "out_dtype"),
    (dict(d=dims(scale=float("inf"))), 1, "scale"),
    (dict(d=dims(scale=-0.125)), 1, "scale"),
    (dict(d=dims(scale=float("nan"))), 1, "scale"),
    (dict(d=dims(), out=None), 1, "NULL"),
    (dict(d=dims(), ptrs=(FAKE + 8, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                          FAKE + 0x4000000)), 1, "aligned"),
    (dict(d=dims(), ptrs=(FAKE, 0, 0, FAKE + 0x3000000, FAKE + 0x4000000)), 1, "k_cache"),
    (dict(d=dims(), out=FAKE + 0x10), 1, "overlaps"),
    (dict(d=dims(), lse=FAKE + 0x3000000), 1, "overlaps"),
    (dict(d=dims(num_kv_heads=1, head_dim=256, shard_cap=1 << 23), cache_len=1 << 24), 2, "2 GiB"),
    (dict(d=dims(num_q_heads=5462 * 256, num_kv_heads=5462, head_dim=256)), 2, "num_q_heads=1398272"),
    (dict(d=dims(head_pos=-1)), 1, "head_pos"),
    (dict(d=dims(tail_pos=-3)), 1, "tail_pos"),
    (dict(d=dims(cur_len=-1)), 1, "cur_len"),
    (dict(d=dims(cur_len=127)), 1, "cur_len=127"),                   # tail reaches position 127
    (dict(d=dims(head_pos=40, tail_pos=0, cur_len=103)), 1, "position 103"),  # head reaches 103
    (dict(d=dims(num_kv_heads=1, head_dim=256, cur_len=1 << 22, q_rows=4, head_rows=4,
                 real_rows=4, tail_pos=4)), 2, "2 GiB"),
]


@pytest.mark.parametrize("kw,code,msg", BAD_PREFILL)
def test_prefill_rejects_bad_arguments(kw, code, msg):
    rc = call_prefill(**kw)
    assert rc == code
    assert msg in ra.lib().ra_last_error().decode()


def test_pad_rows_do_not_need_current_tokens():
    # the tail piece is all pads (real_rows == head_rows): its positions may
    # lie past cur_len; validation passes and fails only later on the
    # overlap check planted here, i.e. after the position checks
    rc = call_prefill(dims(real_rows=64, tail_pos=4000, cur_len=64), out=FAKE + 0x10)
    assert rc == 1 and "overlaps" in ra.lib().ra_last_error().decode()


def test_prefill_no_real_rows_is_a_no_op():
    # nothing real to compute: returns OK without touching the (fake) buffers
    assert call_prefill(dims(real_rows=0)) == 0


@pytest.mark.parametrize("regions", [0, 4, -1])
def test_partial_rejects_bad_regions(regions):
    q, kc, vc, kcur, vcur = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000
    rc = ra.lib().ring_attn_partial(q, kc, vc, kcur, vcur, 512, 2, ra.StripeLayout(1, 0), regions,
                                    FAKE + 0x8000000, None, ctypes.byref(dims()), None)
    assert rc == 1 and "regions" in ra.lib().ra_last_error().decode()


def test_partial_validates_like_prefill():
    q, kc, vc, kcur, vcur = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000
    rc = ra.lib().ring_attn_partial(q, kc, vc, kcur, vcur, 512, 0, ra.StripeLayout(1, 0),
                                    ra.RA_REGION_CACHE, FAKE + 0x8000000, None,
                                    ctypes.byref(dims()), None)
    assert rc == 1 and "P must" in ra.lib().ra_last_error().decode()


def call_split(d, splits=4, ws=FAKE + 0x20000000, ws_bytes=1 << 30):
    q, kc, vc, kcur, vcur = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000
    return ra.lib().ring_attn_prefill_split(q, kc, vc, kcur, vcur, 512, 2, ra.StripeLayout(1, 0),
                                            splits, ws, ws_bytes, FAKE + 0x8000000, None,
                                            ctypes.byref(d), None)


def test_split_workspace_bytes():
    d = dims()
    assert ra.ra_split_workspace_bytes(d, 1) == 0
    # partial outputs [S, C, NQ, HD] fp32 (whatever the output dtype) then LSEs
    # [S, NQ, C] fp32, 256-byte aligned
    assert ra.ra_split_workspace_bytes(d, 3) == 3 * 128 * 4 * 64 * 4 + 3 * 4 * 128 * 4
    d32 = dims(out_dtype=1, q_rows=5, head_rows=5, real_rows=5, tail_pos=5)
    assert ra.ra_split_workspace_bytes(d32, 2) == 2 * 5 * 4 * 64 * 4 + 256  # 160 B of LSE rounds up


@pytest.mark.parametrize("rows,group,nkv,cus,expect", [
    (4096, 16, 2, 256, 1),    # 512 workgroups: two full waves
    (3548, 16, 2, 256, 4),    # 444 workgroups: 1.73 waves; x4 gives 6.94 waves
    (512, 16, 2, 256, 4),     # a rank's 2 x 256 rows: 64 workgroups
    (0, 16, 2, 256, 1),
])
def test_split_suggest(rows, group, nkv, cus, expect):
    d = dims(num_q_heads=group * nkv, num_kv_heads=nkv, head_dim=256, q_rows=max(rows, 1),
             head_rows=max(rows, 1), real_rows=rows, tail_pos=max(rows, 1), cur_len=max(rows, 1))
    assert ra.ra_split_suggest(d, cus) == expect


@pytest.mark.parametrize("kw,msg", [
    (dict(splits=0), "splits"), (dict(splits=65), "splits"),
    (dict(ws=None), "workspace must not be NULL"), (dict(ws=FAKE + 0x20000008), "aligned"),
    (dict(ws_bytes=1000), "workspace_bytes"), (dict(ws=FAKE + 0x3000000), "overlaps"),
])
def test_split_rejects_bad_arguments(kw, msg):
    assert call_split(dims(), **kw) == 1
    assert msg in ra.lib().ra_last_error().decode()


def call_merge(d, ptrs=None, out=FAKE + 0x8000000, lse=None, parts=1):
    o1, l1, o2, l2 = ptrs or (FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000)
    return ra.lib().merge_attn_states(o1, l1, o2, l2, parts, out, lse, ctypes.byref(d), None)


BAD_MERGE = [
    (dict(d=dims(head_dim=80)), 2, "head_dim"),
    (dict(d=dims(num_q_heads=0)), 1, "num_q_heads"),
    (dict(d=dims(real_rows=200)), 1, "real_rows"),
    (dict(d=dims(out_dtype=3)), 1, "out_dtype"),
    (dict(d=dims(), out=None), 1, "NULL"),
    (dict(d=dims(), ptrs=(FAKE, 0, FAKE + 0x2000000, FAKE + 0x3000000)), 1, "NULL"),
    (dict(d=dims(), ptrs=(FAKE + 4, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000)), 1,
     "aligned"),
    (dict(d=dims(), out=FAKE + 0x2000100), 1, "overlaps"),
    (dict(d=dims(), lse=FAKE + 0x3000000), 1, "overlaps"),
    (dict(d=dims(), lse=FAKE + 0x8000100), 1, "out and lse overlap"),
    (dict(d=dims(), parts=2), 1, "parts_dtype"),
    (dict(d=dims(), parts=0, out=FAKE + 0x2000100), 1, "overlaps"),   # bf16 o2 is 64 KiB
]


@pytest.mark.parametrize("kw,code,msg", BAD_MERGE)
def test_merge_rejects_bad_arguments(kw, code, msg):
    assert call_merge(**kw) == code
    assert msg in ra.lib().ra_last_error().decode()


def test_merge_no_real_rows_is_a_no_op():
    assert call_merge(dims(real_rows=0)) == 0


def call_write(d, n=128, cache_len=512, P=2, layout=(1, 0), ptrs=None):
    kcur, vcur, kc, vc = ptrs or (FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000)
    return ra.lib().kv_cache_write(kcur, vcur, n, kc, vc, cache_len, P, ra.StripeLayout(*layout),
                                   ctypes.byref(d), None)


BAD_WRITE = [
    (dict(d=dims(shard_cap=319)), 1, "shard_cap"),
    (dict(d=dims(), n=-1), 1, "n_tokens"),
    (dict(d=dims(), P=0), 1, "P must"),
    (dict(d=dims(head_dim=48)), 2, "head_dim"),
    (dict(d=dims(), ptrs=(FAKE, FAKE + 0x1000000, FAKE + 0x2000008, FAKE + 0x3000000)), 1, "aligned"),
    (dict(d=dims(), ptrs=(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x2000000)), 1, "overlap"),
    (dict(d=dims(), ptrs=(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 0)), 1, "NULL"),
]


@pytest.mark.parametrize("kw,code,msg", BAD_WRITE)
def test_write_rejects_bad_arguments(kw, code, msg):
    assert call_write(**kw) == code
    assert msg in ra.lib().ra_last_error().decode()


def test_write_zero_tokens_is_a_no_op():
    assert call_write(dims(), n=0) == 0


def call_prefill_write(d, n=128, cache_len=512, P=2, layout=(1, 0), ptrs=None,
                       out=FAKE + 0x8000000, lse=None):
    q, kc, vc, kcur, vcur = ptrs or (FAKE, FAKE + 0x1000000, FAKE + 0x2000000,
                                     FAKE + 0x3000000, FAKE + 0x4000000)
    return ra.lib().ring_attn_prefill_write(q, kc, vc, kcur, vcur, cache_len, P,
                                            ra.StripeLayout(*layout), n, out, lse,
                                            ctypes.byref(d), None)


BAD_PREFILL_WRITE = [
    (dict(d=dims(), n=-1), 1, "n_tokens"),
    (dict(d=dims(), n=129), 1, "n_tokens"),                       # k_cur holds cur_len=128
    (dict(d=dims(shard_cap=319)), 1, "shard_cap"),               # the write needs 320 slots
    (dict(d=dims(), ptrs=(FAKE, 0, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000)),
     1, "NULL"),
    (dict(d=dims(), out=FAKE + 0x1000010), 1, "overlaps"),        # out inside k_cache
    (dict(d=dims(), lse=FAKE + 0x2000000), 1, "overlaps"),        # lse inside v_cache
    (dict(d=dims(), ptrs=(FAKE + 0x1000000, FAKE + 0x1000000, FAKE + 0x2000000,
                          FAKE + 0x3000000, FAKE + 0x4000000)), 1, "overlaps"),  # q = k_cache
    (dict(d=dims(num_q_heads=6, num_kv_heads=4)), 1, "multiple"),
    (dict(d=dims(), layout=(1, 2)), 1, "ring_start"),
    (dict(d=dims(scale=-1.0)), 1, "scale"),                       # the attention's own checks
]


@pytest.mark.parametrize("kw,code,msg", BAD_PREFILL_WRITE)
def test_prefill_write_rejects_bad_arguments(kw, code, msg):
    assert call_prefill_write(**kw) == code
    assert msg in ra.lib().ra_last_error().decode()


def test_split_write_checks_the_write_and_the_workspace():
    d = dims()
    q, kc, vc, kcur, vcur = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000
    need = ra.ra_split_workspace_bytes(d, 4)
    L = ra.lib()

    def call(n=128, ws=FAKE + 0x9000000, nbytes=need):
        return L.ring_attn_prefill_split_write(q, kc, vc, kcur, vcur, 512, 2, ra.StripeLayout(1, 0),
                                               4, ws, nbytes, n, FAKE + 0x8000000, None,
                                               ctypes.byref(d), None)
    assert call(n=129) == 1 and "n_tokens" in L.ra_last_error().decode()
    assert call(ws=kc) == 1 and "workspace overlaps" in L.ra_last_error().decode()
    assert call(nbytes=need - 16) == 1 and "workspace_bytes" in L.ra_last_error().decode()
    assert call(ws=0) == 1 and "workspace must not be NULL" in L.ra_last_error().decode()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ra, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ra, "_lib", None)
    with pytest.raises(ImportError):
        ra.lib()


@pytest.mark.parametrize("gen", ["gen_tile_hd256.py", "gen_tile_pipe.py"])
def test_generated_tile_block_is_current(gen):
    """The tile blocks (HD = 256; the three-tile blocks at HD = 128 and 64)
    are generated; each committed include must be what its generator writes
    (else the kernel runs a stale schedule)."""
    import subprocess
    import sys
    gen = os.path.join(ROOT, "context_causal_attention_ring_amd", "csrc", gen)
    res = subprocess.run([sys.executable, gen, "--check"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_checking_build_exports_the_same_symbols():
    """The checking build (every tile fenced) is the same ABI under another name."""
    if not os.path.exists(ra.SYNC_LIB_PATH):
        pytest.skip("checking build not built")
    L = ra.load(ra.SYNC_LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name
    assert b"checking build" in L.ra_version()
    assert b"checking build" not in ra.lib().ra_version()


def test_noalloc_split_refuses_workspace_beyond_its_own():
    """The no-allocation split keeps its partials in the library's own
    RA_NOALLOC_SCRATCH_BYTES per GPU; a request that needs more is refused
    before any HIP call (splits = 4 over 4096 rows x 32 heads x 256 needs
    512 MiB), and bad split counts are refused as for the split entry."""
    d = dims(num_q_heads=32, num_kv_heads=2, head_dim=256, q_rows=4096, head_rows=2048,
             real_rows=4096, tail_pos=2048, cur_len=4096, shard_cap=4096)
    need = ra.ra_split_workspace_bytes(d, 4)
    assert need > ra.RA_NOALLOC_SCRATCH_BYTES
    args = (FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000,
            28672, 8, ra.StripeLayout(1, 0))
    rc = ra.lib().ring_attn_prefill_split_noalloc(*args, 4, FAKE + 0x8000000, None,
                                                  ctypes.byref(d), None)
    assert rc == 2 and b"workspace" in ra.lib().ra_last_error()
    for bad in (0, ra.RA_MAX_SPLITS + 1):
        rc = ra.lib().ring_attn_prefill_split_noalloc(*args, bad, FAKE + 0x8000000, None,
                                                      ctypes.byref(d), None)
        assert rc == 1 and b"splits" in ra.lib().ra_last_error()
    # the largest rank share the workspace was sized for fits: 512 rows, 4 splits
    d.q_rows, d.real_rows, d.head_rows = 512, 512, 256
    assert ra.ra_split_workspace_bytes(d, 4) <= ra.RA_NOALLOC_SCRATCH_BYTES
