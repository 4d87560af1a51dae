"""Plain fp64 CPU oracle for exact attention (ctypes wrapper around attn_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code that may import this module.
It shares no code with the GPU library and imports nothing from it.

The arithmetic lives in ``attn_oracle.c`` (one query row at a time, the full
score row materialised, masked, soft-maxed in double).  This wrapper only
marshals arrays and sums the per-row sink terms:

* ``dsink_h = -sum over rows of (1 - gate_i) * D_i`` -- the sink is a logit
  with no value, so its gradient is minus its softmax share times D_i
  (dew-flash-attn page, sinks paragraph, differentiated by the chain rule).
  With several sinks per head (ejkernel flash_attention API page,
  softmax_aux [num_heads, num_sinks] or [num_sinks]) sink k of head h takes
  the share exp(s_hk) / sum_k' exp(s_hk') of that sum, and sinks shared by
  all heads sum their per-head gradients.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
# ATTN36_ORACLE_LIB selects another build of the same source (the tests run
# an AddressSanitizer build through it)
_LIB_PATH = os.environ.get("ATTN36_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int64), ("window_right", ctypes.c_int64),
        ("nseq", ctypes.c_int64), ("hq", ctypes.c_int64), ("hkv", ctypes.c_int64),
        ("d", ctypes.c_int64), ("scale", ctypes.c_double),
        ("q_start", ctypes.c_void_p), ("q_len", ctypes.c_void_p),
        ("k_start", ctypes.c_void_p), ("k_len", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dout", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("softcap", ctypes.c_double), ("alibi", ctypes.c_void_p), ("num_sinks", ctypes.c_int64),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        lib.oracle_rows.argtypes = [P, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_rows.restype = ctypes.c_int
        lib.oracle_cols.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    vp, vp, vp, vp, vp, vp]
        lib.oracle_cols.restype = ctypes.c_int
        lib.oracle_visible.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64]
        lib.oracle_visible.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int32, ctypes.c_uint16]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


@dataclass
class Problem:
    """An attention problem in token-major packed form.

    q: [Tq, Hq, D] raw bf16/fp16 bits (uint16) or float64 values (dtype
    "f64"); k, v: [Tk, Hkv, D]; dout: [Tq, Hq, D] or None; sinks: [Hq],
    [Hq, n] or, with sinks_shared, [n] (one row for every head), or None
    (widened to float64); softcap: > 0 caps the logits; alibi: ALiBi slopes
    [Hq] or [nseq, Hq], or None.
    Sequence s occupies q tokens [q_start[s], q_start[s]+q_len[s]) and
    k/v tokens [k_start[s], k_start[s]+k_len[s]).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_start: np.ndarray
    q_len: np.ndarray
    k_start: np.ndarray
    k_len: np.ndarray
    scale: float
    causal: bool = False
    window: tuple = (-1, -1)
    dout: np.ndarray | None = None
    sinks: np.ndarray | None = None
    dtype: str = "bf16"
    softcap: float = 0.0
    alibi: np.ndarray | None = None
    sinks_shared: bool = False
    _keep: list = field(default_factory=list, repr=False)

    @property
    def hq(self):
        return self.q.shape[1]

    @property
    def hkv(self):
        return self.k.shape[1]

    @property
    def d(self):
        return self.q.shape[2]

    @property
    def nseq(self):
        return len(self.q_len)

    def sink_table(self):
        """The sinks as [Hq, n] float64 (n sinks per q head), or None."""
        if self.sinks is None:
            return None
        s = np.asarray(self.sinks, np.float64)
        if self.sinks_shared:
            return np.broadcast_to(s.reshape(1, -1), (self.hq, s.size))
        return s.reshape(self.hq, -1)

    def _struct(self):
        et = np.float64 if self.dtype == "f64" else np.uint16
        arrs = dict(
            q=np.ascontiguousarray(self.q, dtype=et),
            k=np.ascontiguousarray(self.k, dtype=et),
            v=np.ascontiguousarray(self.v, dtype=et),
            q_start=np.ascontiguousarray(self.q_start, dtype=np.int64),
            q_len=np.ascontiguousarray(self.q_len, dtype=np.int64),
            k_start=np.ascontiguousarray(self.k_start, dtype=np.int64),
            k_len=np.ascontiguousarray(self.k_len, dtype=np.int64),
            dout=None if self.dout is None else np.ascontiguousarray(self.dout, dtype=et),
            sinks=None if self.sinks is None else np.ascontiguousarray(self.sink_table()),
            alibi=None if self.alibi is None else np.ascontiguousarray(
                np.broadcast_to(np.asarray(self.alibi, np.float64).reshape(-1, self.hq), (self.nseq, self.hq))),
        )
        self._keep = list(arrs.values())
        s = _Problem()
        s.dtype = {"bf16": 0, "fp16": 1, "f64": 2}[self.dtype]
        s.causal = 1 if self.causal else 0
        s.window_left, s.window_right = int(self.window[0]), int(self.window[1])
        s.nseq, s.hq, s.hkv, s.d = self.nseq, self.hq, self.hkv, self.d
        s.scale = float(self.scale)
        for name in ("q_start", "q_len", "k_start", "k_len", "q", "k", "v", "dout", "sinks", "alibi"):
            setattr(s, name, _ptr(arrs[name]))
        s.softcap = float(self.softcap)
        s.num_sinks = 0 if self.sinks is None else arrs["sinks"].shape[1]
        return s


def _used(slot_len, seqused):
    """Lengths a slot uses: its first seqused[b] tokens (fa4-jax page, varlen
    semantics paragraph: seqused_q / seqused_k), or all of them."""
    slot_len = np.asarray(slot_len, np.int64)
    if seqused is None:
        return slot_len
    return np.minimum(np.maximum(np.asarray(seqused, np.int64), 0), slot_len)


def batched(q, k, v, scale, causal=False, window=(-1, -1), dout=None, sinks=None, dtype="bf16", seqused_q=None,
            seqused_k=None, **variants):
    """Wrap [B,S,H,D] uint16 arrays as a Problem (sequence b starts at token b*S
    and uses its first seqused_q[b] / seqused_k[b] tokens when given).
    ``variants``: softcap, alibi, sinks_shared (see Problem)."""
    B, sq, hq, d = q.shape
    sk = k.shape[1]
    return Problem(
        q=q.reshape(B * sq, hq, d), k=k.reshape(B * sk, k.shape[2], d),
        v=v.reshape(B * sk, v.shape[2], d),
        q_start=np.arange(B, dtype=np.int64) * sq, q_len=_used(np.full(B, sq), seqused_q),
        k_start=np.arange(B, dtype=np.int64) * sk, k_len=_used(np.full(B, sk), seqused_k),
        scale=scale, causal=causal, window=window,
        dout=None if dout is None else dout.reshape(B * sq, hq, d), sinks=sinks, dtype=dtype, **variants)


def varlen(q, k, v, cu_q, cu_k, scale, causal=False, window=(-1, -1), dout=None, sinks=None,
           dtype="bf16", seqused_q=None, seqused_k=None, **variants):
    """Wrap packed [T,H,D] arrays plus int cu_seqlens [N+1] as a Problem
    (sequence i uses the first seqused_q[i] / seqused_k[i] tokens of its slot
    when given)."""
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    return Problem(q=q, k=k, v=v, q_start=cu_q[:-1], q_len=_used(np.diff(cu_q), seqused_q),
                   k_start=cu_k[:-1], k_len=_used(np.diff(cu_k), seqused_k), scale=scale, causal=causal,
                   window=window, dout=dout, sinks=sinks, dtype=dtype, **variants)


def kvcache(q, k_cache, v_cache, cache_seqlens, scale, block_table=None, causal=False, window=(-1, -1),
            sinks=None, dtype="bf16", **variants):
    """A forward over a KV cache as a Problem.  Slot b's queries q[b] attend to
    the first cache_seqlens[b] keys of its slot, the band aligned to that used
    length (fa4-jax page, varlen semantics paragraph: seqused_k).  Without a
    block table the slot is k_cache[b] ([B, capacity, Hkv, D]); with one, key j
    of slot b is row j % page of page block_table[b][j // page] of the paged
    cache [num_blocks, page, Hkv, D] (vllm-project/flash-attention README on
    the GitHub search page, flash_attn_with_kvcache: paged KV cache).  The used
    keys are gathered into packed form; the attention itself is the packed
    Problem's."""
    B, sq, hq, d = q.shape
    lens = np.asarray(cache_seqlens, np.int64)
    rows_per = k_cache.shape[1]  # slot capacity, or page size with a block table
    kf = k_cache.reshape(-1, k_cache.shape[2], d)
    vf = v_cache.reshape(-1, v_cache.shape[2], d)
    idx = []
    for b in range(B):
        j = np.arange(lens[b], dtype=np.int64)
        if block_table is None:
            idx.append(b * rows_per + j)
        else:
            idx.append(np.asarray(block_table[b], np.int64)[j // rows_per] * rows_per + j % rows_per)
    idx = np.concatenate(idx)
    return Problem(q=q.reshape(B * sq, hq, d), k=kf[idx], v=vf[idx],
                   q_start=np.arange(B, dtype=np.int64) * sq, q_len=np.full(B, sq, np.int64),
                   k_start=np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64), k_len=lens,
                   scale=scale, causal=causal, window=window, sinks=sinks, dtype=dtype, **variants)


def rotary(x, cos, sin, positions, rotary_dim, interleaved):
    """Rotary embedding of x [B, S, H, D] (float64) at integer positions [B, S]:
    the first rotary_dim dims form rotary_dim/2 pairs, pair j of a token at
    position p turns by the angle whose cosine and sine are cos[p, j],
    sin[p, j]: (a, b) -> (a cos - b sin, a sin + b cos); the other dims are
    unchanged.  Pairs are dims (2j, 2j+1) when interleaved, else (j, j +
    rotary_dim/2) (vllm-project/flash-attention README on the GitHub search
    page, flash_attn_with_kvcache: rotary_cos, rotary_sin, rotary_interleaved)."""
    x = np.array(x, np.float64, copy=True)
    half = rotary_dim // 2
    positions = np.minimum(positions, len(cos) - 1)  # positions past the table: its last row
    c = np.asarray(cos, np.float64)[positions][:, :, None, :]  # [B, S, 1, half]
    s = np.asarray(sin, np.float64)[positions][:, :, None, :]
    if interleaved:
        a, b = x[..., 0:rotary_dim:2].copy(), x[..., 1:rotary_dim:2].copy()
        x[..., 0:rotary_dim:2] = a * c - b * s
        x[..., 1:rotary_dim:2] = a * s + b * c
    else:
        a, b = x[..., :half].copy(), x[..., half:rotary_dim].copy()
        x[..., :half] = a * c - b * s
        x[..., half:rotary_dim] = a * s + b * c
    return x


def decode_array(dtype: str, bits) -> np.ndarray:
    """bf16 / fp16 bit patterns -> float64, exactly (a bf16 value is the top
    half of a binary32; fp16 is numpy's binary16)."""
    bits = np.asarray(bits, np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode(dtype: str, x) -> np.ndarray:
    """float64 -> bf16 / fp16 bit patterns, rounded to nearest, ties to even,
    in one rounding from the float64 value."""
    x = np.asarray(x, np.float64)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    # bf16: the nearest of the two bf16 values around x (float32 keeps x
    # between them: it has more precision than bf16)
    lo = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint32)
    hi = lo + 1
    vlo = (lo << 16).view(np.float32).astype(np.float64)
    vhi = (hi << 16).view(np.float32).astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(np.isfinite(x), pick, lo)
    return pick.astype(np.uint16)


def kvcache_append(k_cache, v_cache, cache_seqlens, k_new, v_new, block_table=None, rotary_cos=None,
                   rotary_sin=None, rotary_dim=0, rotary_interleaved=True, dtype="bf16"):
    """The cache after writing new keys and values in place: token i of slot b
    goes to key position cache_seqlens[b] + i of the slot (a row of k_cache[b],
    or of the page the block table names), the keys rotated at that position
    when rotary tables are given and rounded to the cache's dtype
    (flash_attn_with_kvcache docstring: k, v, cache_seqlens, rotary_cos).
    Positions past the slot (its capacity, or its pages) are not written: the
    pages leave them to the caller, and the library drops them.  Arrays are
    bit patterns; returns new (k_cache, v_cache, seqlens)."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    B, sn = k_new.shape[0], k_new.shape[1]
    lens = np.asarray(cache_seqlens, np.int64)
    pos = lens[:, None] + np.arange(sn)[None, :]
    kn = k_new
    if rotary_cos is not None:
        kn = encode(dtype, rotary(decode_array(dtype, k_new), rotary_cos, rotary_sin, pos, rotary_dim,
                                  rotary_interleaved))
    rows = kc.shape[1]
    for b in range(B):
        for i in range(sn):
            p = int(pos[b, i])
            if block_table is None:
                if p >= rows:
                    continue
                slot, r = b, p
            else:
                if p // rows >= len(block_table[b]):
                    continue
                slot, r = int(block_table[b][p // rows]), p % rows
            kc[slot, r] = kn[b, i]
            vc[slot, r] = v_new[b, i]
    return kc, vc, (lens + sn).astype(np.int32)


def visible(causal, left, right, lq, lk, i, j) -> bool:
    """The bottom-right aligned causal/window predicate, as the oracle applies it."""
    return bool(_load().oracle_visible(int(causal), int(left), int(right), int(lq), int(lk),
                                       int(i), int(j)))


def decode(dtype: str, bits: int) -> float:
    """Exact value of one bf16/fp16 encoding, as the oracle decodes it."""
    return float(_load().oracle_decode(0 if dtype == "bf16" else 1, int(bits)))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def rows(p: Problem, seq, head, row, grads: bool = False):
    """Per-row results for requests (seq[r], head[r], row[r]).

    Returns dict with o [n,D], lse [n], gate [n] and, when ``grads`` (needs
    p.dout), delta [n] and dq [n,D]; all float64.
    """
    lib = _load()
    seq = np.ascontiguousarray(seq, np.int64)
    head = np.ascontiguousarray(head, np.int64)
    row = np.ascontiguousarray(row, np.int64)
    n = len(seq)
    out = dict(o=np.zeros((n, p.d)), lse=np.zeros(n), gate=np.zeros(n))
    if grads:
        if p.dout is None:
            raise ValueError("grads need dout")
        out["delta"] = np.zeros(n)
        out["dq"] = np.zeros((n, p.d))
    st = p._struct()
    rc = lib.oracle_rows(ctypes.byref(st), n, _ptr(seq), _ptr(head), _ptr(row),
                         _ptr(out["o"]), _ptr(out["lse"]), _ptr(out["gate"]),
                         _ptr(out.get("delta")), _ptr(out.get("dq")))
    if rc != 0:
        raise RuntimeError("oracle_rows failed: %d" % rc)
    return out


def group_row_stats(p: Problem, s: int, g: int):
    """lse, gate, delta for every row of the q heads of kv group g in sequence s ([G, Lq])."""
    G = p.hq // p.hkv
    lq = int(p.q_len[s])
    heads = np.repeat(np.arange(g * G, (g + 1) * G), lq)
    rr = np.tile(np.arange(lq), G)
    r = rows(p, np.full(len(rr), s), heads, rr, grads=True)
    return (r["lse"].reshape(G, lq), r["gate"].reshape(G, lq), r["delta"].reshape(G, lq))


def cols(p: Problem, s: int, g: int, col, stats=None):
    """dK, dV [n, D] for keys col of sequence s, kv head g (fp64)."""
    lib = _load()
    col = np.ascontiguousarray(col, np.int64)
    if stats is None:
        stats = group_row_stats(p, s, g)
    lse, gate, delta = (np.ascontiguousarray(a, np.float64) for a in stats)
    dk = np.zeros((len(col), p.d))
    dv = np.zeros((len(col), p.d))
    st = p._struct()
    rc = lib.oracle_cols(ctypes.byref(st), int(s), int(g), len(col), _ptr(col), _ptr(lse),
                         _ptr(gate), _ptr(delta), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise RuntimeError("oracle_cols failed: %d" % rc)
    return dk, dv


def full(p: Problem, grads: bool = True):
    """Every output of a (small) problem.

    Returns dict: o [Tq,Hq,D], lse [Hq,Tq] (the packed layout; a batched
    caller reshapes), and with grads dq [Tq,Hq,D], dk, dv [Tk,Hkv,D],
    dsinks in the layout of p.sinks ([Hq], [Hq, n] or shared [n]; zeros [Hq]
    when p.sinks is None).
    """
    Tq, Tk = p.q.shape[0], p.k.shape[0]
    seqs, heads, rws, toks = [], [], [], []
    for s in range(p.nseq):
        for h in range(p.hq):
            for i in range(int(p.q_len[s])):
                seqs.append(s)
                heads.append(h)
                rws.append(i)
                toks.append(int(p.q_start[s]) + i)
    out = dict(o=np.zeros((Tq, p.hq, p.d)), lse=np.full((p.hq, Tq), np.nan))
    if grads:
        out.update(dq=np.zeros((Tq, p.hq, p.d)), dk=np.zeros((Tk, p.hkv, p.d)),
                   dv=np.zeros((Tk, p.hkv, p.d)),
                   dsinks=np.zeros(p.hq) if p.sinks is None else np.zeros(np.shape(p.sinks)))
    if not seqs:
        return out
    r = rows(p, seqs, heads, rws, grads=grads)
    toks = np.asarray(toks)
    heads = np.asarray(heads)
    out["o"][toks, heads] = r["o"]
    out["lse"][heads, toks] = r["lse"]
    if not grads:
        return out
    out["dq"][toks, heads] = r["dq"]
    if p.sinks is not None:
        per_head = np.zeros(p.hq)
        np.add.at(per_head, heads, -(1.0 - r["gate"]) * r["delta"])
        tab = p.sink_table()
        share = np.exp(tab - tab.max(axis=1, keepdims=True))
        share /= share.sum(axis=1, keepdims=True)
        per_sink = per_head[:, None] * share  # [Hq, n]
        out["dsinks"] = (per_sink.sum(axis=0) if p.sinks_shared else per_sink).reshape(np.shape(p.sinks))
    G = p.hq // p.hkv
    for s in range(p.nseq):
        lq, lk = int(p.q_len[s]), int(p.k_len[s])
        if lk == 0:
            continue
        for g in range(p.hkv):
            if lq == 0:
                continue
            sel = (np.asarray(seqs) == s) & (heads // G == g)
            # rows were emitted head-major then row-major, matching [G, Lq]
            stats = (r["lse"][sel].reshape(G, lq), r["gate"][sel].reshape(G, lq),
                     r["delta"][sel].reshape(G, lq))
            dk, dv = cols(p, s, g, np.arange(lk), stats=stats)
            k0 = int(p.k_start[s])
            out["dk"][k0:k0 + lk, g] = dk
            out["dv"][k0:k0 + lk, g] = dv
    return out
