"""Python binding of libringattn (fused ring + current attention, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libringattn.so``.  PyTorch supplies device memory and the
stream.  The C entry points and their contracts are declared in
``include/ringattn.h``; the functions here carry the same names.

The library must have been built (``python -m
context_causal_attention_ring_amd.build``); importing a missing library
raises instead of falling back to anything else.
"""
import ctypes
import os

__all__ = ["StripeLayout", "Dims", "RingAttnError", "lib", "ring_attn_prefill",
           "ring_attn_partial", "merge_attn_states", "kv_cache_write", "ra_shard_len",
           "ra_version", "prefill", "two_launch_prefill", "LIB_PATH", "EXPORTED_SYMBOLS",
           "RA_REGION_CACHE", "RA_REGION_CURRENT", "ring_attn_prefill_split",
           "ra_split_workspace_bytes", "ra_split_suggest", "RA_MAX_SPLITS", "load",
           "SYNC_LIB_PATH", "ring_attn_prefill_split_noalloc", "RA_NOALLOC_SCRATCH_BYTES",
           "ring_attn_prefill_write", "ring_attn_prefill_split_write"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn.so")
# The checking build (every tile of the fused kernel fenced by a wait and a
# barrier); tests compare it bit for bit with the product library.
SYNC_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn_sync.so")
EXPORTED_SYMBOLS = ("ring_attn_prefill", "ring_attn_prefill_write", "ring_attn_prefill_split",
                    "ring_attn_prefill_split_write",
                    "ra_split_workspace_bytes",
                    "ring_attn_prefill_split_noalloc",
                    "ra_split_suggest",
                    "ring_attn_partial", "merge_attn_states", "kv_cache_write", "ra_shard_len",
                    "ra_last_error", "ra_version")
RA_MAX_SPLITS = 64
RA_NOALLOC_SCRATCH_BYTES = 72 << 20

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, 1, 2, 3
RA_DTYPE_BF16, RA_DTYPE_FP32 = 0, 1
RA_REGION_CACHE, RA_REGION_CURRENT = 1, 2


class StripeLayout(ctypes.Structure):
    _fields_ = [("interleave", ctypes.c_int32), ("ring_start", ctypes.c_int32)]


class Dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_rows", ctypes.c_int32),
                ("head_rows", ctypes.c_int32), ("real_rows", ctypes.c_int32),
                ("head_pos", ctypes.c_int32), ("tail_pos", ctypes.c_int32),
                ("cur_len", ctypes.c_int32),
                ("shard_cap", ctypes.c_int64), ("scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32)]


class RingAttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libringattn error {code}: {msg}")
        self.code = code


_lib = None


def load(path):
    """Open one build of the library with the C signatures declared."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -m context_causal_attention_ring_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.ring_attn_prefill.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout, vp, vp,
                                    ctypes.POINTER(Dims), vp]
    L.ring_attn_prefill.restype = ctypes.c_int
    L.ring_attn_prefill_write.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout, i32, vp,
                                          vp, ctypes.POINTER(Dims), vp]
    L.ring_attn_prefill_write.restype = ctypes.c_int
    L.ring_attn_prefill_split_write.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout, i32,
                                                vp, i64, i32, vp, vp, ctypes.POINTER(Dims), vp]
    L.ring_attn_prefill_split_write.restype = ctypes.c_int
    L.ring_attn_prefill_split.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout, i32,
                                          vp, i64, vp, vp, ctypes.POINTER(Dims), vp]
    L.ring_attn_prefill_split.restype = ctypes.c_int
    L.ring_attn_prefill_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout,
                                                  i32, vp, vp, ctypes.POINTER(Dims), vp]
    L.ring_attn_prefill_split_noalloc.restype = ctypes.c_int
    L.ra_split_workspace_bytes.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(i64)]
    L.ra_split_workspace_bytes.restype = ctypes.c_int
    L.ra_split_suggest.argtypes = [ctypes.POINTER(Dims), i32, ctypes.POINTER(i32)]
    L.ra_split_suggest.restype = ctypes.c_int
    L.ring_attn_partial.argtypes = [vp, vp, vp, vp, vp, i64, i32, StripeLayout, i32, vp, vp,
                                    ctypes.POINTER(Dims), vp]
    L.ring_attn_partial.restype = ctypes.c_int
    L.merge_attn_states.argtypes = [vp, vp, vp, vp, i32, vp, vp, ctypes.POINTER(Dims), vp]
    L.merge_attn_states.restype = ctypes.c_int
    L.kv_cache_write.argtypes = [vp, vp, i32, vp, vp, i64, i32, StripeLayout,
                                 ctypes.POINTER(Dims), vp]
    L.kv_cache_write.restype = ctypes.c_int
    L.ra_shard_len.argtypes = [i64, i32, StripeLayout, i32, ctypes.POINTER(i64)]
    L.ra_shard_len.restype = ctypes.c_int
    L.ra_last_error.argtypes = []
    L.ra_last_error.restype = ctypes.c_char_p
    L.ra_version.argtypes = []
    L.ra_version.restype = ctypes.c_char_p
    return L


def lib():
    """Load libringattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def _check(rc):
    if rc != RA_OK:
        raise RingAttnError(rc, lib().ra_last_error().decode())


def _ptr(t):
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libringattn takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libringattn takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def ra_version():
    return lib().ra_version().decode()


def ra_shard_len(cache_len, P, stripe_layout, shard):
    n = ctypes.c_int64()
    _check(lib().ra_shard_len(cache_len, P, stripe_layout, shard, ctypes.byref(n)))
    return n.value


def ring_attn_prefill(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, out, lse,
                      dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers."""
    _check(lib().ring_attn_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cur),
                                   _ptr(v_cur), cache_len, P, stripe_layout, _ptr(out),
                                   _ptr(lse), ctypes.byref(dims), _stream(stream)))


def ring_attn_prefill_write(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                            n_tokens, out, lse, dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers."""
    _check(lib().ring_attn_prefill_write(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cur),
                                         _ptr(v_cur), cache_len, P, stripe_layout, n_tokens,
                                         _ptr(out), _ptr(lse), ctypes.byref(dims),
                                         _stream(stream)))


def ring_attn_prefill_split_write(q, k_cache, v_cache, k_cur, v_cur, cache_len, P,
                                  stripe_layout, splits, workspace, n_tokens, out, lse, dims,
                                  stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers
    (``workspace`` as in ring_attn_prefill_split)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ring_attn_prefill_split_write(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(k_cur), _ptr(v_cur), cache_len, P,
                                               stripe_layout, splits, _ptr(workspace), nbytes,
                                               n_tokens, _ptr(out), _ptr(lse),
                                               ctypes.byref(dims), _stream(stream)))


def ra_split_suggest(dims, num_cus):
    s = ctypes.c_int32()
    _check(lib().ra_split_suggest(ctypes.byref(dims), num_cus, ctypes.byref(s)))
    return s.value


def ra_split_workspace_bytes(dims, splits):
    n = ctypes.c_int64()
    _check(lib().ra_split_workspace_bytes(ctypes.byref(dims), splits, ctypes.byref(n)))
    return n.value


def ring_attn_prefill_split(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                            splits, workspace, out, lse, dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers
    (``workspace`` a device tensor of at least ra_split_workspace_bytes
    bytes, or None when splits == 1)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ring_attn_prefill_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cur),
                                         _ptr(v_cur), cache_len, P, stripe_layout, splits,
                                         _ptr(workspace), nbytes, _ptr(out), _ptr(lse),
                                         ctypes.byref(dims), _stream(stream)))


def ring_attn_prefill_split_noalloc(q, k_cache, v_cache, k_cur, v_cur, cache_len, P,
                                    stripe_layout, splits, out, lse, dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers."""
    _check(lib().ring_attn_prefill_split_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(k_cur), _ptr(v_cur), cache_len, P,
                                                 stripe_layout, splits, _ptr(out), _ptr(lse),
                                                 ctypes.byref(dims), _stream(stream)))


def ring_attn_partial(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, regions,
                      out, lse, dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers."""
    _check(lib().ring_attn_partial(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cur),
                                   _ptr(v_cur), cache_len, P, stripe_layout, regions, _ptr(out),
                                   _ptr(lse), ctypes.byref(dims), _stream(stream)))


def merge_attn_states(o1, lse1, o2, lse2, out, lse, dims, stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers
    (the partials' dtype is taken from o1)."""
    import torch
    if o1.dtype != o2.dtype:
        raise ValueError("o1 and o2 must have the same dtype")
    parts = RA_DTYPE_FP32 if o1.dtype == torch.float32 else RA_DTYPE_BF16
    _check(lib().merge_attn_states(_ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), parts, _ptr(out),
                                   _ptr(lse), ctypes.byref(dims), _stream(stream)))


def kv_cache_write(k_cur, v_cur, n_tokens, k_cache, v_cache, cache_len, P, stripe_layout, dims,
                   stream=None):
    """Same arguments as the C entry point, with torch tensors for buffers."""
    _check(lib().kv_cache_write(_ptr(k_cur), _ptr(v_cur), n_tokens, _ptr(k_cache),
                                _ptr(v_cache), cache_len, P, stripe_layout,
                                ctypes.byref(dims), _stream(stream)))


def make_dims(q, k_cur, shard_cap, real_rows=None, head_rows=None, scale=0.0, out_fp32=False,
              head_pos=0, tail_pos=None):
    """Dims for q [C, NQ, HD] and token-order k_cur [cur_len, NKV, HD].  The
    default layout is contiguous: head piece at chunk position 0, tail piece
    right after it."""
    C, NQ, HD = q.shape
    NKV = k_cur.shape[1]
    head_rows = C if head_rows is None else head_rows
    return Dims(num_q_heads=NQ, num_kv_heads=NKV, head_dim=HD, q_rows=C, head_rows=head_rows,
                real_rows=C if real_rows is None else real_rows, head_pos=head_pos,
                tail_pos=head_pos + head_rows if tail_pos is None else tail_pos,
                cur_len=k_cur.shape[0], shard_cap=shard_cap, scale=scale,
                out_dtype=RA_DTYPE_FP32 if out_fp32 else RA_DTYPE_BF16)


def prefill(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, interleave=1, ring_start=0,
            real_rows=None, head_rows=None, scale=0.0, out_fp32=False, with_lse=True,
            stream=None, head_pos=0, tail_pos=None):
    """Allocate out/lse with torch and run ring_attn_prefill.

    q [C, NQ, HD] bf16, k_cache/v_cache [P, shard_cap, NKV, HD] bf16,
    k_cur/v_cur [cur_len, NKV, HD] bf16 (token order).  Returns (out, lse)."""
    import torch
    C, NQ, HD = q.shape
    out = torch.empty(C, NQ, HD, device=q.device,
                      dtype=torch.float32 if out_fp32 else torch.bfloat16)
    lse = torch.empty(NQ, C, device=q.device, dtype=torch.float32) if with_lse else None
    dims = make_dims(q, k_cur, k_cache.shape[1], real_rows, head_rows, scale, out_fp32,
                     head_pos, tail_pos)
    ring_attn_prefill(q, k_cache, v_cache, k_cur, v_cur, cache_len, P,
                      StripeLayout(interleave, ring_start), out, lse, dims, stream)
    return out, lse


def two_launch_prefill(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, out, lse,
                       dims, parts, stream=None):
    """The removed two-launch variant: cache-only launch, current-only launch,
    LSE merge.  ``parts`` = (o1, lse1, o2, lse2): caller-allocated buffers of
    the partial outputs [C, NQ, HD] (bf16, the model dtype, or fp32) and
    their fp32 LSEs [NQ, C]."""
    import torch
    o1, l1, o2, l2 = parts
    d = Dims.from_buffer_copy(dims)
    d.out_dtype = RA_DTYPE_FP32 if o1.dtype == torch.float32 else RA_DTYPE_BF16
    ring_attn_partial(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                      RA_REGION_CACHE, o1, l1, d, stream)
    ring_attn_partial(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                      RA_REGION_CURRENT, o2, l2, d, stream)
    merge_attn_states(o1, l1, o2, l2, out, lse, dims, stream)
