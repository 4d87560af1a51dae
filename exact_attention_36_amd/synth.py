"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and encodes them; it holds none of the
attention arithmetic.  Every tensor is drawn from numpy's PCG64 generator
(``numpy.random.default_rng(seed)``) as float32 N(0,1) and rounded to bf16
with round-to-nearest-even (or converted to fp16 by numpy, also RNE), and is
returned as raw uint16 bits so that any consumer can decode it exactly.

Draw order for one problem: (packed lengths), q, k, v, dout, (sinks).
"""
from __future__ import annotations

import math

import numpy as np

_CHUNK = 1 << 24  # elements per draw, bounds peak host memory


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Exact float32 value of bf16/fp16 bit patterns."""
    bits = np.ascontiguousarray(bits, np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def normal_bits(rng: np.random.Generator, shape, dtype: str = "bf16") -> np.ndarray:
    """i.i.d. N(0,1) float32 draws encoded as bf16/fp16 bits, drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if dtype == "bf16":
            out[s:e] = f32_to_bf16_bits(x)
        else:
            out[s:e] = x.astype(np.float16).view(np.uint16)
    return out.reshape(shape)


def packed_lengths(rng: np.random.Generator, n: int = 64, total: int = 65536,
                   max_len: int = 4096, n_zero: int = 8) -> np.ndarray:
    """Sequence lengths for a packed batch.

    Draw n lengths log-uniform on [1, max_len], set n_zero of them (chosen
    without replacement) to zero, rescale the rest to sum to ``total``, floor
    them (nonzero entries kept >= 1) and hand the remainder out one token at a
    time to the entries with the largest fractional parts (or take it back
    from the largest entries when negative).
    """
    L = np.exp(rng.uniform(0.0, math.log(max_len), n))
    z = rng.choice(n, n_zero, replace=False)
    L[z] = 0.0
    L *= total / L.sum()
    Li = np.floor(L).astype(np.int64)
    nz = L > 0
    Li[nz] = np.maximum(Li[nz], 1)
    rem = total - int(Li.sum())
    if rem > 0:
        frac = np.where(nz, L - np.floor(L), -1.0)
        order = np.argsort(-frac, kind="stable")
        for i in order[:rem]:
            Li[i] += 1
    while rem < 0:
        i = int(np.argmax(Li))
        Li[i] -= 1
        rem += 1
    assert int(Li.sum()) == total
    return Li


def cu_seqlens(lengths) -> np.ndarray:
    """int32 offsets [N+1] from 0 to the token count."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def default_scale(d: int) -> float:
    """1/sqrt(D) rounded to float32, the value both sides use."""
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def batched_inputs(seed: int, B: int, sq: int, sk: int, hq: int, hkv: int, d: int,
                   grads: bool = True, sinks: bool = False, dtype: str = "bf16"):
    """q, k, v, dout ([B,S,H,D] uint16 bits) and sinks (float32 [hq]) for one seed."""
    rng = np.random.default_rng(seed)
    q = normal_bits(rng, (B, sq, hq, d), dtype)
    k = normal_bits(rng, (B, sk, hkv, d), dtype)
    v = normal_bits(rng, (B, sk, hkv, d), dtype)
    dout = normal_bits(rng, (B, sq, hq, d), dtype) if grads else None
    s = rng.standard_normal(hq, dtype=np.float32) if sinks else None
    return dict(q=q, k=k, v=v, dout=dout, sinks=s)


def kvcache_inputs(seed: int, B: int, sq: int, hq: int, hkv: int, d: int, lens, capacity: int,
                   page: int = 0, sinks: bool = False, dtype: str = "bf16"):
    """q [B,sq,hq,d] and a KV cache holding lens[b] used keys per slot (uint16 bits).

    page == 0: k_cache, v_cache [B, capacity, hkv, d]; else pages of `page` rows,
    ceil(capacity / page) per slot, dealt to the slots in a seeded random order:
    k_cache, v_cache [B * pages, page, hkv, d] and block_table int32 [B, pages].
    Rows past a slot's used length hold random values too (they must stay
    invisible)."""
    rng = np.random.default_rng(seed)
    q = normal_bits(rng, (B, sq, hq, d), dtype)
    if page:
        npg = -(-capacity // page)
        k = normal_bits(rng, (B * npg, page, hkv, d), dtype)
        v = normal_bits(rng, (B * npg, page, hkv, d), dtype)
        table = rng.permutation(B * npg).astype(np.int32).reshape(B, npg)
    else:
        k = normal_bits(rng, (B, capacity, hkv, d), dtype)
        v = normal_bits(rng, (B, capacity, hkv, d), dtype)
        table = None
    s = rng.standard_normal(hq, dtype=np.float32) if sinks else None
    return dict(q=q, k=k, v=v, lens=np.asarray(lens, np.int32), block_table=table, sinks=s)


def varlen_inputs(seed: int, lengths_q, lengths_k, hq: int, hkv: int, d: int,
                  grads: bool = True, sinks: bool = False, dtype: str = "bf16"):
    """Packed q, k, v, dout ([T,H,D] uint16 bits), cu_seqlens and sinks for given lengths."""
    rng = np.random.default_rng(seed)
    cq, ck = cu_seqlens(lengths_q), cu_seqlens(lengths_k)
    q = normal_bits(rng, (int(cq[-1]), hq, d), dtype)
    k = normal_bits(rng, (int(ck[-1]), hkv, d), dtype)
    v = normal_bits(rng, (int(ck[-1]), hkv, d), dtype)
    dout = normal_bits(rng, (int(cq[-1]), hq, d), dtype) if grads else None
    s = rng.standard_normal(hq, dtype=np.float32) if sinks else None
    return dict(q=q, k=k, v=v, dout=dout, sinks=s, cu_q=cq, cu_k=ck)


def packed_workload(seed: int = 4, n: int = 64, total: int = 65536, hq: int = 16,
                    hkv: int = 4, d: int = 128, grads: bool = True, dtype: str = "bf16"):
    """The packed-batch workload: lengths drawn first, then the tensors, one generator."""
    rng = np.random.default_rng(seed)
    L = packed_lengths(rng, n=n, total=total)
    cu = cu_seqlens(L)
    T = int(cu[-1])
    q = normal_bits(rng, (T, hq, d), dtype)
    k = normal_bits(rng, (T, hkv, d), dtype)
    v = normal_bits(rng, (T, hkv, d), dtype)
    dout = normal_bits(rng, (T, hq, d), dtype) if grads else None
    return dict(q=q, k=k, v=v, dout=dout, sinks=None, cu_q=cu, cu_k=cu, lengths=L)


def sink_table(seed: int, rows: int, n: int) -> np.ndarray:
    """Sink logits, float32 [rows, n] (rows = q heads, or 1 for a shared row):
    N(0, 1.5^2), seeded on their own."""
    rng = np.random.default_rng(int(seed) + 7919)
    return (1.5 * rng.standard_normal((rows, n))).astype(np.float32)


def alibi_slopes(hq: int, batch: int = 0, seed: int = 0) -> np.ndarray:
    """ALiBi slopes, float32: the geometric sequence 2^(-8 (h+1) / hq) of the
    ALiBi paper (Press et al., 2021) for [hq]; with batch > 0, [batch, hq]
    rows of it scaled by seeded factors in [0.5, 2)."""
    base = np.exp2(-8.0 * (np.arange(hq) + 1) / hq)
    if batch <= 0:
        return base.astype(np.float32)
    rng = np.random.default_rng(int(seed) + 104729)
    return (base[None, :] * rng.uniform(0.5, 2.0, (batch, 1))).astype(np.float32)


def device_normal(seed: int, shapes, device="cuda", dtype: str = "bf16"):
    """Large inputs drawn on the GPU: i.i.d. N(0,1) float32 from torch's seeded
    device generator (Philox), rounded to bf16/fp16 (RNE), in the order of
    `shapes`.  Returns device tensors; `host_bits` gives their uint16 encodings.
    Used where drawing on the host would take minutes (multi-GB K/V caches).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    out = []
    for shp in shapes:
        t = torch.empty(shp, dtype=td, device=device)
        flat = t.view(-1)
        for s in range(0, flat.numel(), _CHUNK):
            e = min(flat.numel(), s + _CHUNK)
            flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(td)
        out.append(t)
    return out


def host_bits(t) -> np.ndarray:
    """uint16 encodings of a 16-bit tensor, copied to the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
