"""ctypes binding of libattn36.so (include/attn.h).

Argument marshalling only: shapes and dtypes are read off the tensors, outputs
and the workspace are allocated with torch on the inputs' device, and the
call is enqueued on torch's current stream.  Every computation happens in the
library's HIP kernels; if the library is missing this module raises instead
of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn36.so")

ATTN_OK, ATTN_EINVAL, ATTN_ENOTSUP, ATTN_EHIP = 0, 1, 2, 3
ATTN_BF16, ATTN_FP16, ATTN_FP32 = 0, 1, 2

EXPORTED = (
    "attn_fwd", "attn_fwd_workspace_size", "attn_bwd", "attn_bwd_workspace_size", "attn_bwd_noalloc",
    "attn_fwd_kvcache", "attn_fwd_kvcache_workspace_size", "attn_kvcache_append", "attn_rotary",
    "attn_fwd_varlen", "attn_fwd_varlen_workspace_size", "attn_bwd_varlen",
    "attn_bwd_varlen_workspace_size", "attn_last_error", "attn_version", "attn_timing_enable", "attn_timing_select",
    "attn_timing_read",
)
KERNELS = ("fwd", "fwd_combine", "bwd_dsink", "bwd_dq", "bwd_dkdv", "order")


class AttnError(RuntimeError):
    """A non-OK status from the library; .status holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__("attn status %d: %s" % (status, msg))
        self.status = status


class attn_params(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("sinks", ctypes.c_void_p), ("num_sinks", ctypes.c_int32), ("sinks_shared", ctypes.c_int32),
        ("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p), ("alibi_per_batch", ctypes.c_int32),
        ("seqused_q", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p),
    ]


_lib = None


def load_library():
    """Load libattn36.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libattn36.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(attn_params)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.attn_fwd.argtypes = [P, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_fwd_workspace_size.argtypes = [P, i64, i64, i64]
    lib.attn_bwd.argtypes = [P, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.attn_bwd_workspace_size.argtypes = [P, i64, i64, i64, i32]
    lib.attn_bwd_noalloc.argtypes = [P, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.attn_fwd_kvcache.argtypes = [P, i64, i64, vp, vp, vp, vp, vp, i32, i32, i64, vp, vp, vp, sz, vp]
    lib.attn_fwd_kvcache_workspace_size.argtypes = [P, i64, i64, vp, i32, i32, i64]
    lib.attn_kvcache_append.argtypes = [P, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, vp, vp, i32, i32,
                                        i64, vp]
    lib.attn_rotary.argtypes = [P, i64, i64, i32, vp, vp, vp, i32, vp, vp, i32, i32, i64, vp]
    lib.attn_fwd_varlen.argtypes = [P, i32, i64, i64, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_fwd_varlen_workspace_size.argtypes = [P, i32, i64, i64, i32, i32]
    lib.attn_bwd_varlen.argtypes = [P, i32, i64, i64, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, i32, vp, sz, vp]
    lib.attn_bwd_varlen_workspace_size.argtypes = [P, i32, i64, i64, i32, i32, i32]
    lib.attn_timing_enable.argtypes = [i32]
    lib.attn_timing_select.argtypes = [ctypes.c_uint32]
    lib.attn_timing_read.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
    for name in EXPORTED:
        if name.endswith("workspace_size"):
            getattr(lib, name).restype = ctypes.c_size_t
        elif name == "attn_last_error":
            lib.attn_last_error.restype = ctypes.c_char_p
        else:
            getattr(lib, name).restype = ctypes.c_int32
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().attn_last_error().decode()


def version() -> int:
    return int(load_library().attn_version())


def attn_timing_enable(on: bool = True, kernels=None) -> None:
    """Start (or stop) bracketing library kernel launches with HIP events:
    every kernel, or only those named in ``kernels`` (names from KERNELS)."""
    lib = load_library()
    mask = (1 << len(KERNELS)) - 1 if kernels is None else sum(1 << KERNELS.index(k) for k in kernels)
    _check(lib.attn_timing_select(mask))
    _check(lib.attn_timing_enable(1 if on else 0))


def attn_timing_read(kernel: str):
    """(launches, total milliseconds) of one kernel since attn_timing_enable."""
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(load_library().attn_timing_read(KERNELS.index(kernel), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return ATTN_BF16
    if t == torch.float16:
        return ATTN_FP16
    if t == torch.float32:
        return ATTN_FP32
    raise ValueError("unsupported dtype %s" % t)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(cond, msg):
    """Raise ValueError(msg) unless cond; msg may be a callable that builds the
    message, so that the checks of a launch-bound call format nothing when
    they pass."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _check_tensors(named, dtype=None, shapes=None):
    """Reject what the C ABI cannot see: every tensor in `named` (name ->
    tensor or None) must be contiguous and on one CUDA device; `dtype` names
    the tensors that must share the 16-bit input dtype; `shapes` maps a name
    to its required shape (None entries of a shape are free).  Shape and
    dtype are checked before the device, so host tensors of a wrong shape
    are reported by shape."""
    present = {n: t for n, t in named.items() if t is not None}
    for n, want in (shapes or {}).items():
        t = present.get(n)
        if t is None or want is None:
            continue
        got = t.shape
        ok = len(got) == len(want)
        if ok:
            for w, g in zip(want, got):
                if w is not None and w != g:
                    ok = False
                    break
        _need(ok, lambda: "%s must have shape %s, got %s" % (n, tuple("*" if w is None else int(w) for w in want),
                                                              tuple(got)))
    if dtype:
        ref = present[dtype[0]].dtype
        _need(ref in (torch.bfloat16, torch.float16), lambda: "%s must be bf16 or fp16, got %s" % (dtype[0], ref))
        for n in dtype[1:]:
            if n in present:
                _need(present[n].dtype == ref,
                      lambda: "%s must have %s's dtype %s, got %s" % (n, dtype[0], ref, present[n].dtype))
    for n, t in present.items():
        _need(t.is_contiguous(), lambda: "%s must be contiguous (got strides %s)" % (n, tuple(t.stride())))
    devs = {t.get_device() for t in present.values()}  # -1 off the GPU
    _need(len(devs) == 1, lambda: "all tensors must be on one device, got %s"
          % sorted({str(t.device) for t in present.values()}))
    _need(devs.pop() >= 0 and next(iter(present.values())).is_cuda,
          lambda: "tensors must be on a GPU (got %s)" % next(iter(present.values())).device)


def _check_f32(name, t, shape):
    if t is not None:
        _need(t.dtype == torch.float32, lambda: "%s must be fp32, got %s" % (name, t.dtype))
        _need(tuple(t.shape) == tuple(shape),
              lambda: "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_i32(name, t, shape):
    if t is not None:
        _need(t.dtype == torch.int32, lambda: "%s must be int32, got %s" % (name, t.dtype))
        _need(tuple(t.shape) == tuple(shape),
              lambda: "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def make_params(q, k, causal=False, window=(-1, -1), sinks=None, softmax_scale=None, softcap=0.0,
                alibi_slopes=None, sinks_shared=False, nseq=None, seqused_q=None,
                seqused_k=None) -> attn_params:
    """sinks: fp32 [Hq] (one per head), [Hq, n], or [n] with sinks_shared (one row
    for every head); alibi_slopes: fp32 [Hq] or [B, Hq]; softcap: 0 = off;
    seqused_q, seqused_k: int32 [B] (or [num_seqs]) used lengths per slot."""
    hq = q.shape[-2]
    if sinks is not None:
        ok = sinks.dim() == 1 if sinks_shared else (tuple(sinks.shape) == (hq,) or
                                                    (sinks.dim() == 2 and sinks.shape[0] == hq))
        if not ok or sinks.dtype != torch.float32 or not sinks.is_contiguous():
            raise ValueError("sinks must be contiguous fp32 [Hq], [Hq, n] or (shared) [n]; got %s %s"
                             % (tuple(sinks.shape), sinks.dtype))
    if alibi_slopes is not None:
        if (alibi_slopes.shape[-1] != hq or alibi_slopes.dim() not in (1, 2) or
                (alibi_slopes.dim() == 2 and alibi_slopes.shape[0] != nseq) or
                alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_contiguous()):
            raise ValueError("alibi_slopes must be contiguous fp32 [Hq] or [%s, Hq]; got %s %s"
                             % (nseq, tuple(alibi_slopes.shape), alibi_slopes.dtype))
    p = attn_params()
    p.dtype = _dtype_code(q.dtype)
    p.head_dim = q.shape[-1]
    p.heads_q = q.shape[-2]
    p.heads_kv = k.shape[-2]
    p.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.sinks = _ptr(sinks)
    if sinks is not None:
        p.sinks_shared = 1 if sinks_shared else 0
        p.num_sinks = sinks.numel() if sinks_shared else (1 if sinks.dim() == 1 else int(sinks.shape[-1]))
    p.softcap = float(softcap)
    p.alibi_slopes = _ptr(alibi_slopes)
    p.alibi_per_batch = 1 if alibi_slopes is not None and alibi_slopes.dim() == 2 else 0
    for name, t in (("seqused_q", seqused_q), ("seqused_k", seqused_k)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (nseq,) or not t.is_contiguous()):
            raise ValueError("%s must be contiguous int32 [%s]; got %s %s" % (name, nseq, tuple(t.shape), t.dtype))
        setattr(p, name, _ptr(t))
    if sinks is not None or alibi_slopes is not None or seqused_q is not None or seqused_k is not None:
        _check_tensors(dict(q=q, sinks=sinks, alibi_slopes=alibi_slopes, seqused_q=seqused_q, seqused_k=seqused_k))
    return p


def _check(st):
    if st != ATTN_OK:
        raise AttnError(st, last_error())


# torch's current-stream handle as a plain integer, without building a Stream
# object (a few microseconds a call); the public call where torch lacks it
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev):
    if _RAW_STREAM is not None:
        return ctypes.c_void_p(_RAW_STREAM(torch.cuda.current_device() if dev.index is None else dev.index))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(nbytes, dev):
    """Device workspace of nbytes, or None when the call needs none (the
    library accepts a NULL workspace of size 0)."""
    return torch.empty(int(nbytes), dtype=torch.uint8, device=dev) if nbytes else None


def attn_fwd(q, k, v, causal=False, window=(-1, -1), sinks=None, softmax_scale=None, softcap=0.0,
             alibi_slopes=None, sinks_shared=False, seqused_q=None, seqused_k=None, out=None, lse=None):
    """Batched forward: q [B,Sq,Hq,D], k, v [B,Sk,Hkv,D] -> (o, lse [B,Hq,Sq] fp32)."""
    lib = load_library()
    _need(q.dim() == 4 and k.dim() == 4, "q, k, v must be [B, S, H, D]")
    B, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    _check_f32("lse", lse, (B, hq, sq))
    _check_tensors(dict(q=q, k=k, v=v, out=out, lse=lse), dtype=("q", "k", "v", "out"),
                   shapes=dict(k=(B, None, None, d), v=(B, sk, hkv, d), out=(B, sq, hq, d)))
    p = make_params(q, k, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=B, seqused_q=seqused_q, seqused_k=seqused_k)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, hq, sq), dtype=torch.float32, device=q.device) if lse is None else lse
    n = lib.attn_fwd_workspace_size(ctypes.byref(p), B, sq, sk)
    ws = _workspace(n, q.device)
    _check(lib.attn_fwd(ctypes.byref(p), B, sq, sk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                        _ptr(ws), n, _stream(q.device)))
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, causal=False, window=(-1, -1), sinks=None, softmax_scale=None, softcap=0.0,
             alibi_slopes=None, sinks_shared=False, seqused_q=None, seqused_k=None,
             grad_dtype=None):
    """Batched backward -> (dq, dk, dv, dsinks or None)."""
    lib = load_library()
    _need(q.dim() == 4 and k.dim() == 4, "q, k, v must be [B, S, H, D]")
    B, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    _need(grad_dtype in (None, q.dtype, torch.float32),
          "grad_dtype must be the input dtype or torch.float32, got %s" % grad_dtype)
    _check_f32("lse", lse, (B, hq, sq))
    _check_tensors(dict(q=q, k=k, v=v, o=o, lse=lse, dout=dout), dtype=("q", "k", "v", "o", "dout"),
                   shapes=dict(k=(B, None, None, d), v=(B, sk, hkv, d), o=(B, sq, hq, d), dout=(B, sq, hq, d)))
    p = make_params(q, k, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=B, seqused_q=seqused_q, seqused_k=seqused_k)
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device)
    dk = torch.empty(k.shape, dtype=gd, device=q.device)
    dv = torch.empty(v.shape, dtype=gd, device=q.device)
    dsinks = torch.empty(sinks.shape, dtype=torch.float32, device=q.device) if sinks is not None else None
    n = lib.attn_bwd_workspace_size(ctypes.byref(p), B, sq, sk, _dtype_code(gd))
    ws = _workspace(n, q.device)
    _check(lib.attn_bwd(ctypes.byref(p), B, sq, sk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                        _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), _dtype_code(gd),
                        _ptr(ws), n, _stream(q.device)))
    return dq, dk, dv, dsinks


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


def attn_bwd_noalloc(q, k, v, o, lse, dout, causal=False, window=(-1, -1), sinks=None, softmax_scale=None,
                     softcap=0.0, alibi_slopes=None, sinks_shared=False, seqused_q=None, seqused_k=None,
                     grad_dtype=None, dq=None, dk=None, dv=None, dsinks=None):
    """Batched backward through attn_bwd_noalloc (the library's fixed scratch
    instead of a workspace) -> (dq, dk, dv, dsinks or None).  Pass dq, dk, dv
    (and dsinks) to have nothing allocated on this side either."""
    lib = load_library()
    _need(q.dim() == 4 and k.dim() == 4, "q, k, v must be [B, S, H, D]")
    B, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    _need(grad_dtype in (None, q.dtype, torch.float32),
          "grad_dtype must be the input dtype or torch.float32, got %s" % grad_dtype)
    gd = q.dtype if grad_dtype is None else grad_dtype
    _check_f32("lse", lse, (B, hq, sq))
    for n, t, shp in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, v.shape)):
        if t is not None:
            _need(t.dtype == gd and tuple(t.shape) == tuple(shp), lambda: "%s must be %s %s" % (n, gd, tuple(shp)))
    if dsinks is not None and sinks is not None:
        _check_f32("dsinks", dsinks, tuple(sinks.shape))
    _check_tensors(dict(q=q, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, dsinks=dsinks),
                   dtype=("q", "k", "v", "o", "dout"),
                   shapes=dict(k=(B, None, None, d), v=(B, sk, hkv, d), o=(B, sq, hq, d), dout=(B, sq, hq, d)))
    p = make_params(q, k, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=B, seqused_q=seqused_q, seqused_k=seqused_k)
    dq = torch.empty(q.shape, dtype=gd, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=gd, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=gd, device=q.device) if dv is None else dv
    if sinks is not None and dsinks is None:
        dsinks = torch.empty(sinks.shape, dtype=torch.float32, device=q.device)
    _check(lib.attn_bwd_noalloc(ctypes.byref(p), B, sq, sk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks if sinks is not None else None),
                                _dtype_code(gd), _stream(q.device)))
    return dq, dk, dv, (dsinks if sinks is not None else None)


def _check_rotary(rotary_cos, rotary_sin):
    for t in (rotary_cos, rotary_sin):
        if t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("rotary_cos / rotary_sin must be contiguous fp32 [seqlen_ro, rotary_dim / 2]")
    if rotary_cos.shape != rotary_sin.shape:
        raise ValueError("rotary_cos and rotary_sin must have the same shape")
    return 2 * int(rotary_cos.shape[1]), int(rotary_cos.shape[0])


def attn_rotary(x, positions, rotary_cos, rotary_sin, interleaved=True, per_token=True, out=None):
    """Rotary embedding of x [B,S,H,D] at positions[b] + i (per_token) or positions[b]
    (int32 [B]); rotary_cos, rotary_sin fp32 [seqlen_ro, rotary_dim / 2] -> out."""
    lib = load_library()
    _need(x.dim() == 4, "x must be [B, S, H, D]")
    B, S, H, d = x.shape
    rdim, nro = _check_rotary(rotary_cos, rotary_sin)
    _check_i32("positions", positions, (B,))
    _check_tensors(dict(x=x, out=out, positions=positions, rotary_cos=rotary_cos, rotary_sin=rotary_sin),
                   dtype=("x", "out"), shapes=dict(out=tuple(x.shape)))
    p = make_params(x, x)
    out = torch.empty_like(x) if out is None else out
    _check(lib.attn_rotary(ctypes.byref(p), B, S, H, _ptr(x), _ptr(out), _ptr(positions), 1 if per_token else 0,
                           _ptr(rotary_cos), _ptr(rotary_sin), rdim, 1 if interleaved else 0, nro,
                           _stream(x.device)))
    return out


def attn_kvcache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, block_table=None, rotary_cos=None,
                        rotary_sin=None, rotary_interleaved=True, seqlens_out=None):
    """Write k_new, v_new [B,Sn,Hkv,D] into the cache in place at positions
    cache_seqlens[b] + i (keys rotated there when rotary tables are given);
    returns seqlens_out (int32 [B]) = cache_seqlens + Sn."""
    lib = load_library()
    _need(k_new.dim() == 4 and k_cache.dim() == 4, "k_new, v_new and the caches must be 4-d")
    B, sn, hkv, d = k_new.shape
    _check_i32("cache_seqlens", cache_seqlens, (B,))
    _check_i32("seqlens_out", seqlens_out, (B,))
    if block_table is not None:
        _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be int32 [B, max_blocks]")
        _check_i32("block_table", block_table, tuple(block_table.shape))
    _check_tensors(dict(k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens,
                        seqlens_out=seqlens_out, block_table=block_table, rotary_cos=rotary_cos,
                        rotary_sin=rotary_sin),
                   dtype=("k_new", "v_new", "k_cache", "v_cache"),
                   shapes=dict(v_new=tuple(k_new.shape), k_cache=(None if block_table is not None else B, None, hkv, d),
                               v_cache=tuple(k_cache.shape)))
    p = make_params(k_new, k_new)
    if block_table is not None:
        nblk, page, cap = int(block_table.shape[1]), int(k_cache.shape[1]), 0
    else:
        nblk, page, cap = 0, 0, int(k_cache.shape[1])
    rdim, nro = _check_rotary(rotary_cos, rotary_sin) if rotary_cos is not None else (0, 0)
    seqlens_out = torch.empty_like(cache_seqlens) if seqlens_out is None else seqlens_out
    _check(lib.attn_kvcache_append(ctypes.byref(p), B, sn, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(cache_seqlens), _ptr(seqlens_out), _ptr(block_table), nblk, page, cap,
                                   _ptr(rotary_cos), _ptr(rotary_sin), rdim, 1 if rotary_interleaved else 0, nro,
                                   _stream(k_new.device)))
    return seqlens_out


def attn_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, causal=False, window=(-1, -1),
                     sinks=None, softmax_scale=None, softcap=0.0, alibi_slopes=None, sinks_shared=False, seqused_q=None,
                     seqused_k=None, out=None, lse=None, k_new=None, v_new=None, rotary_cos=None, rotary_sin=None,
                     rotary_interleaved=True):
    """Forward over a KV cache: q [B,Sq,Hq,D]; cache_seqlens int32 [B] (used keys per slot);
    k_cache, v_cache [B,capacity,Hkv,D], or pages [num_blocks,page,Hkv,D] with
    block_table int32 [B,max_blocks] -> (o, lse [B,Hq,Sq]).  With k_new, v_new
    [B,Sn,Hkv,D] the cache is first updated in place at cache_seqlens (the
    caller then advances its lengths by Sn) and attention covers the grown
    cache; with rotary tables the new keys, and q, are rotated at their
    positions (q at cache_seqlens + i when causal or windowed, else all at
    cache_seqlens), as flash_attn_with_kvcache does."""
    lib = load_library()
    _need(seqused_k is None, "attn_fwd_kvcache takes the used keys per slot from cache_seqlens; "
                             "seqused_k is not accepted here")
    _need(q.dim() == 4 and k_cache.dim() == 4, "q and the caches must be 4-d")
    B, sq, hq, d = q.shape
    hkv = k_cache.shape[2]
    _check_i32("cache_seqlens", cache_seqlens, (B,))
    if block_table is not None:
        _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be int32 [B, max_blocks]")
        _check_i32("block_table", block_table, tuple(block_table.shape))
    _check_f32("lse", lse, (B, hq, sq))
    _check_tensors(dict(q=q, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens, block_table=block_table,
                        out=out, lse=lse, k_new=k_new, v_new=v_new),
                   dtype=("q", "k_cache", "v_cache", "out", "k_new", "v_new"),
                   shapes=dict(k_cache=(None if block_table is not None else B, None, hkv, d),
                               v_cache=tuple(k_cache.shape), out=(B, sq, hq, d),
                               k_new=(B, None, hkv, d),
                               v_new=tuple(k_new.shape) if k_new is not None else None))
    if k_new is not None:
        old = cache_seqlens  # the first new token's position in each slot
        cache_seqlens = attn_kvcache_append(k_new, v_new, k_cache, v_cache, old, block_table, rotary_cos,
                                            rotary_sin, rotary_interleaved)
        if rotary_cos is not None:
            local = causal or tuple(window) != (-1, -1)
            q = attn_rotary(q, old, rotary_cos, rotary_sin, rotary_interleaved, per_token=local)
    p = make_params(q, k_cache, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=B, seqused_q=seqused_q, seqused_k=seqused_k)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, hq, sq), dtype=torch.float32, device=q.device) if lse is None else lse
    if block_table is not None:
        nblk, page, cap = int(block_table.shape[1]), int(k_cache.shape[1]), 0
    else:
        nblk, page, cap = 0, 0, int(k_cache.shape[1])
    n = lib.attn_fwd_kvcache_workspace_size(ctypes.byref(p), B, sq, _ptr(block_table), nblk, page, cap)
    ws = _workspace(n, q.device)
    _check(lib.attn_fwd_kvcache(ctypes.byref(p), B, sq, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                _ptr(block_table), nblk, page, cap, _ptr(o), _ptr(lse), _ptr(ws), n,
                                _stream(q.device)))
    return o, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=False,
                    window=(-1, -1), sinks=None, softmax_scale=None, softcap=0.0, alibi_slopes=None,
                    sinks_shared=False, seqused_q=None, seqused_k=None, out=None, lse=None):
    """Packed forward: q [Tq,Hq,D], k, v [Tk,Hkv,D], int32 cu_seqlens [N+1] -> (o, lse [Hq,Tq])."""
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 3, "packed q, k, v must be [T, H, D]")
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape[0] >= 2, "cu_seqlens_q must be int32 [N+1], N >= 1")
    n = cu_seqlens_q.shape[0] - 1
    _check_i32("cu_seqlens_q", cu_seqlens_q, (n + 1,))
    _check_i32("cu_seqlens_k", cu_seqlens_k, (n + 1,))
    _check_f32("lse", lse, (hq, tq))
    _check_tensors(dict(q=q, k=k, v=v, out=out, lse=lse, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k),
                   dtype=("q", "k", "v", "out"), shapes=dict(k=(None, None, d), v=(tk, hkv, d), out=(tq, hq, d)))
    p = make_params(q, k, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=n, seqused_q=seqused_q, seqused_k=seqused_k)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device) if lse is None else lse
    nb = lib.attn_fwd_varlen_workspace_size(ctypes.byref(p), n, tq, tk, max_seqlen_q, max_seqlen_k)
    ws = _workspace(nb, q.device)
    _check(lib.attn_fwd_varlen(ctypes.byref(p), n, tq, tk, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                               int(max_seqlen_q), int(max_seqlen_k), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(o), _ptr(lse), _ptr(ws), nb, _stream(q.device)))
    return o, lse


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    causal=False, window=(-1, -1), sinks=None, softmax_scale=None, softcap=0.0, alibi_slopes=None,
                    sinks_shared=False, seqused_q=None, seqused_k=None, grad_dtype=None):
    """Packed backward -> (dq, dk, dv, dsinks or None)."""
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 3, "packed q, k, v must be [T, H, D]")
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape[0] >= 2, "cu_seqlens_q must be int32 [N+1], N >= 1")
    n = cu_seqlens_q.shape[0] - 1
    _check_i32("cu_seqlens_q", cu_seqlens_q, (n + 1,))
    _check_i32("cu_seqlens_k", cu_seqlens_k, (n + 1,))
    _need(grad_dtype in (None, q.dtype, torch.float32),
          "grad_dtype must be the input dtype or torch.float32, got %s" % grad_dtype)
    _check_f32("lse", lse, (hq, tq))
    _check_tensors(dict(q=q, k=k, v=v, o=o, lse=lse, dout=dout, cu_seqlens_q=cu_seqlens_q,
                        cu_seqlens_k=cu_seqlens_k),
                   dtype=("q", "k", "v", "o", "dout"),
                   shapes=dict(k=(None, None, d), v=(tk, hkv, d), o=(tq, hq, d), dout=(tq, hq, d)))
    p = make_params(q, k, causal, window, sinks, softmax_scale, softcap, alibi_slopes, sinks_shared,
                    nseq=n, seqused_q=seqused_q, seqused_k=seqused_k)
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device)
    dk = torch.empty(k.shape, dtype=gd, device=q.device)
    dv = torch.empty(v.shape, dtype=gd, device=q.device)
    dsinks = torch.empty(sinks.shape, dtype=torch.float32, device=q.device) if sinks is not None else None
    nb = lib.attn_bwd_varlen_workspace_size(ctypes.byref(p), n, tq, tk, max_seqlen_q, max_seqlen_k,
                                            _dtype_code(gd))
    ws = _workspace(nb, q.device)
    _check(lib.attn_bwd_varlen(ctypes.byref(p), n, tq, tk, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                               int(max_seqlen_q), int(max_seqlen_k), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(dsinks), _dtype_code(gd), _ptr(ws), nb, _stream(q.device)))
    return dq, dk, dv, dsinks
