"""GPU parity of the score variants and of several sinks per head against the
fp64 oracle: the soft cap cap*tanh(x/cap) of each scaled logit, the ALiBi
bias -slope*|i + Lk - Lq - j| with per-head or per-sequence slopes, both
together, and n sinks per q head or one row shared by all heads -- forward
and backward (all gradients, dsinks in the sinks' layout), batched, packed,
split-KV, KV cache, head dims 64/96/128/256, bf16 and fp16."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_attention_36_amd import synth
import exact_attention_36_amd as ea
from _helpers import assert_close, assert_lse, check_dsinks, dev_tensor, host, scale_of

pytestmark = pytest.mark.gpu


def _sinks(seed, inp, hq, spec):
    """(numpy sinks or None, shared flag) for a sinks spec: 0, 1, n, or "sharedN"."""
    if spec == 0:
        return None, False
    if spec == 1:
        return inp["sinks"], False
    if isinstance(spec, str):
        return synth.sink_table(seed, 1, int(spec[6:]))[0], True
    return synth.sink_table(seed, hq, spec), False


def _slopes(kind, hq, nseq, seed):
    if kind is None:
        return None
    return synth.alibi_slopes(hq) if kind == "head" else synth.alibi_slopes(hq, nseq, seed)


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


BATCHED = [
    # id, B, sq, sk, hq, hkv, d, causal, window, sinks, softcap, alibi, dtype
    ("cap_causal_gqa", 2, 200, 200, 4, 2, 128, True, (-1, -1), 0, 1.2, None, "bf16"),
    ("cap_window_sinks_fp16", 1, 257, 190, 2, 2, 64, True, (37, 0), 1, 0.7, None, "fp16"),
    ("alibi_causal_sq_lt_sk", 2, 150, 333, 4, 4, 128, True, (-1, -1), 0, 0.0, "head", "bf16"),
    ("alibi_batch_two_sided", 2, 190, 150, 4, 1, 64, False, (40, 25), 1, 0.0, "batch", "bf16"),
    ("alibi_noncausal_full_fp16", 1, 129, 300, 2, 2, 128, False, (-1, -1), 0, 0.0, "head", "fp16"),
    ("cap_alibi_multisink_g8", 1, 96, 200, 8, 1, 128, True, (-1, -1), 3, 2.0, "head", "bf16"),
    ("multisink_shared_fp16", 1, 150, 150, 4, 2, 128, True, (-1, -1), "shared4", 0.0, None, "fp16"),
    ("multisink_per_head", 2, 100, 100, 4, 4, 64, False, (-1, -1), 2, 0.0, None, "bf16"),
    ("cap_alibi_d256", 1, 130, 130, 2, 1, 256, True, (-1, -1), 1, 1.5, "batch", "bf16"),
    ("cap_alibi_d96_pad", 2, 100, 140, 4, 2, 96, True, (30, 0), 2, 1.0, "head", "bf16"),
    ("cap_alibi_decode_split", 2, 3, 5000, 8, 2, 128, True, (-1, -1), 1, 3.0, "head", "bf16"),
    ("alibi_sq_gt_sk_empty_rows", 1, 333, 150, 4, 1, 128, True, (-1, -1), 1, 0.0, "head", "bf16"),
]


@pytest.mark.parametrize("case", BATCHED, ids=[c[0] for c in BATCHED])
def test_variant_batched_matches_oracle(case):
    name, B, sq, sk, hq, hkv, d, causal, window, sspec, cap, akind, dt = case
    print("case", name, flush=True)
    seed = zlib.crc32(name.encode()) % 1000
    inp = synth.batched_inputs(seed, B, sq, sk, hq, hkv, d, grads=True, sinks=sspec == 1, dtype=dt)
    sinks, shared = _sinks(seed, inp, hq, sspec)
    slopes = _slopes(akind, hq, B, seed)
    cap = float(np.float32(cap))
    scale = scale_of(d)
    prob = oracle.batched(inp["q"], inp["k"], inp["v"], scale, causal=causal, window=window, dout=inp["dout"],
                          sinks=sinks, dtype=dt, softcap=cap, alibi=slopes, sinks_shared=shared)
    ref = oracle.full(prob)
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    kw = dict(causal=causal, window=window, sinks=_dev(sinks), sinks_shared=shared, softcap=cap,
              alibi_slopes=_dev(slopes))
    o, lse = ea.attn_fwd(q, k, v, **kw)
    o2, lse2 = ea.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "forward is not bitwise repeatable"
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], dt)
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])
    for gd in (torch.float32, torch.bfloat16 if dt == "bf16" else torch.float16):
        dq, dk, dv, ds = ea.attn_bwd(q, k, v, o, lse, do, grad_dtype=gd, **kw)
        torch.cuda.synchronize()
        od = "f32" if gd == torch.float32 else dt
        assert_close(name + ".dq", host(dq).reshape(B * sq, hq, d), ref["dq"], od)
        assert_close(name + ".dk", host(dk).reshape(B * sk, hkv, d), ref["dk"], od)
        assert_close(name + ".dv", host(dv).reshape(B * sk, hkv, d), ref["dv"], od)
        if sinks is not None:
            check_dsinks(name, host(ds), ref["dsinks"], prob)


VARLEN = [
    # id, lens_q, lens_k, hq, hkv, d, causal, window, sinks, softcap, alibi, dtype
    ("varlen_cap_alibi_multisink", [0, 17, 283, 128, 1, 77], None, 4, 2, 128, True, (-1, -1), 2, 1.5, "batch",
     "bf16"),
    ("varlen_alibi_mixed_fp16", [5, 0, 130, 64, 9], [200, 3, 130, 0, 9], 2, 2, 64, True, (50, 0), 1, 0.0, "head",
     "fp16"),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_variant_varlen_matches_oracle(case):
    name, lq, lk, hq, hkv, d, causal, window, sspec, cap, akind, dt = case
    print("case", name, flush=True)
    lk = lq if lk is None else lk
    seed = zlib.crc32(name.encode()) % 1000
    inp = synth.varlen_inputs(seed, lq, lk, hq, hkv, d, grads=True, sinks=sspec == 1, dtype=dt)
    sinks, shared = _sinks(seed, inp, hq, sspec)
    slopes = _slopes(akind, hq, len(lq), seed)
    cap = float(np.float32(cap))
    scale = scale_of(d)
    prob = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], scale, causal=causal,
                         window=window, dout=inp["dout"], sinks=sinks, dtype=dt, softcap=cap, alibi=slopes,
                         sinks_shared=shared)
    ref = oracle.full(prob)
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    cq, ck = torch.from_numpy(inp["cu_q"]).cuda(), torch.from_numpy(inp["cu_k"]).cuda()
    kw = dict(causal=causal, window=window, sinks=_dev(sinks), sinks_shared=shared, softcap=cap,
              alibi_slopes=_dev(slopes))
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), **kw)
    torch.cuda.synchronize()
    assert_close(name + ".o", host(o), ref["o"], dt)
    assert_lse(name + ".lse", host(lse), ref["lse"])
    dq, dk, dv, ds = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, max(lq), max(lk), grad_dtype=torch.float32,
                                        **kw)
    torch.cuda.synchronize()
    assert_close(name + ".dq", host(dq), ref["dq"], "f32")
    assert_close(name + ".dk", host(dk), ref["dk"], "f32")
    assert_close(name + ".dv", host(dv), ref["dv"], "f32")
    if sinks is not None:
        check_dsinks(name, host(ds), ref["dsinks"], prob)


def test_variant_kvcache_matches_oracle():
    """Paged KV cache, split-KV, cap + per-slot ALiBi + 3 sinks per head; the
    ALiBi diagonal uses each slot's used length."""
    name = "kv_cap_alibi_paged"
    print("case", name, flush=True)
    B, sq, hq, hkv, d, lens, capacity, page = 2, 8, 8, 1, 128, [5000, 700], 5056, 64
    inp = synth.kvcache_inputs(11, B, sq, hq, hkv, d, lens, capacity, page=page)
    sinks = synth.sink_table(11, hq, 3)
    slopes = synth.alibi_slopes(hq, B, 11)
    cap = float(np.float32(2.5))
    q, kc, vc = (dev_tensor(inp[n]) for n in ("q", "k", "v"))
    o, lse = ea.attn_fwd_kvcache(q, kc, vc, _dev(inp["lens"]), block_table=_dev(inp["block_table"]), causal=True,
                                 sinks=_dev(sinks), softcap=cap, alibi_slopes=_dev(slopes))
    torch.cuda.synchronize()
    ref = oracle.full(oracle.kvcache(inp["q"], inp["k"], inp["v"], inp["lens"], scale_of(d),
                                     block_table=inp["block_table"], causal=True, sinks=sinks, softcap=cap,
                                     alibi=slopes), grads=False)
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], "bf16")
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])


def test_one_sink_row_equals_single_sinks():
    """n = 1 given as [Hq, 1] is the one-sink call bit for bit; a shared row
    of one sink equals the same value repeated per head (forward bitwise,
    dsinks summed over heads)."""
    inp = synth.batched_inputs(4, 1, 160, 160, 4, 2, 128, grads=True, sinks=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    s1 = _dev(inp["sinks"])
    o, lse = ea.attn_fwd(q, k, v, causal=True, sinks=s1)
    o2, lse2 = ea.attn_fwd(q, k, v, causal=True, sinks=s1.reshape(4, 1).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    g = ea.attn_bwd(q, k, v, o, lse, do, causal=True, sinks=s1)
    g2 = ea.attn_bwd(q, k, v, o, lse, do, causal=True, sinks=s1.reshape(4, 1).contiguous())
    torch.cuda.synchronize()
    for a, b in zip(g[:3], g2[:3]):
        assert torch.equal(a, b)
    assert torch.equal(g[3], g2[3].reshape(4))
    shared = s1[:1].contiguous()
    o3, _ = ea.attn_fwd(q, k, v, causal=True, sinks=shared, sinks_shared=True)
    o4, _ = ea.attn_fwd(q, k, v, causal=True, sinks=shared.repeat(4))
    torch.cuda.synchronize()
    assert torch.equal(o3, o4)
    d3 = ea.attn_bwd(q, k, v, o3, lse, do, causal=True, sinks=shared, sinks_shared=True)[3]
    d4 = ea.attn_bwd(q, k, v, o4, lse, do, causal=True, sinks=shared.repeat(4))[3]
    torch.cuda.synchronize()
    assert torch.allclose(d3, d4.sum().reshape(1), rtol=1e-4, atol=1e-5)


def test_backward_is_deterministic_with_sinks():
    """Every output of the backward, d(sink) included, is the same bit for bit
    on repeated calls: a packed batch with GQA, a soft cap, ALiBi and 3 sinks
    per head, whose sink gradients sum partials from many workgroups."""
    lens = [700, 1, 0, 1500, 333]
    inp = synth.varlen_inputs(21, lens, lens, 8, 2, 128, grads=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    kw = dict(causal=True, sinks=_dev(synth.sink_table(21, 8, 3)), softcap=float(np.float32(4.0)),
              alibi_slopes=_dev(synth.alibi_slopes(8, len(lens), 21)))
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, cq, max(lens), max(lens), **kw)
    first = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, cq, max(lens), max(lens), **kw)
    for _ in range(2):
        again = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, cq, max(lens), max(lens), **kw)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_zero_alibi_slopes_equal_plain_kernels(d):
    """ALiBi slopes of 0 add -0 * |dist| to every score: the ALiBi instances
    then give the plain instances' results bit for bit (forward, every
    gradient, split-KV decode included)."""
    for B, sq, sk in ((2, 150, 230), (1, 3, 4000)):
        inp = synth.batched_inputs(d + sk, B, sq, sk, 4, 2, d, grads=True, sinks=True)
        q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
        kw = dict(causal=True, sinks=_dev(inp["sinks"]))
        zero = torch.zeros(4, dtype=torch.float32, device="cuda")
        o, lse = ea.attn_fwd(q, k, v, **kw)
        oz, lsez = ea.attn_fwd(q, k, v, alibi_slopes=zero, **kw)
        g = ea.attn_bwd(q, k, v, o, lse, do, **kw)
        gz = ea.attn_bwd(q, k, v, o, lse, do, alibi_slopes=zero, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, oz) and torch.equal(lse, lsez), (d, sq, sk)
        for a, b in zip(g, gz):
            assert torch.equal(a, b), (d, sq, sk)
