"""GPU parity across head dims: kernels are built 64, 128 and 256 wide, and
any multiple of 8 up to 256 runs on the next width up, whose tile columns past
the head dim are zero on load and never stored (fa4-jax page, restrictions paragraph: head
dims that are multiples of 8).  Each case is checked against the fp64 oracle,
forward and backward, batched, packed and from a KV cache; and the padded
kernels must equal, bit for bit, the unpadded kernels run on inputs that carry
the zero columns explicitly."""
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from exact_attention_36_amd import synth
import exact_attention_36_amd as ea
from _helpers import check_dsinks, assert_close, assert_lse, dev_tensor, host, oracle_batched, scale_of

pytestmark = pytest.mark.gpu

BATCHED = [
    # id, B, sq, sk, hq, hkv, d, causal, window, sinks, dtype
    ("d8_causal_gqa", 2, 130, 130, 4, 2, 8, True, (-1, -1), False, "bf16"),
    ("d16_window_sinks", 1, 200, 260, 4, 4, 16, True, (40, 0), True, "bf16"),
    ("d40_two_sided_fp16", 1, 257, 190, 2, 1, 40, False, (20, 13), False, "fp16"),
    ("d56_sq_gt_sk", 1, 150, 70, 4, 2, 56, True, (-1, -1), True, "bf16"),
    ("d72_noncausal_g8", 2, 96, 200, 8, 1, 72, False, (-1, -1), False, "bf16"),
    ("d96_causal_ragged", 2, 200, 333, 4, 2, 96, True, (-1, -1), True, "bf16"),
    ("d120_fp16_sinks", 1, 129, 129, 2, 2, 120, True, (-1, -1), True, "fp16"),
    # split-KV forward (decode shape): partials and combine with a padded head
    ("d80_decode_split", 2, 3, 5000, 8, 2, 80, True, (-1, -1), True, "bf16"),
    # the 256-wide kernels (one wave per SIMD), exact and padded
    ("d256_causal_gqa_sinks", 2, 200, 200, 4, 2, 256, True, (-1, -1), True, "bf16"),
    ("d256_two_sided_fp16", 1, 257, 190, 2, 2, 256, False, (20, 13), False, "fp16"),
    ("d192_sq_lt_sk_window", 2, 150, 333, 4, 1, 192, True, (64, 0), False, "bf16"),
    ("d136_sq_gt_sk", 1, 333, 150, 4, 4, 136, True, (-1, -1), True, "bf16"),
    ("d160_decode_split", 2, 3, 5000, 8, 2, 160, True, (-1, -1), True, "bf16"),
    ("d256_decode_split_fp16", 1, 4, 3000, 32, 1, 256, True, (-1, -1), False, "fp16"),
]


def _torch_dtype(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float16


@pytest.mark.parametrize("case", BATCHED, ids=[c[0] for c in BATCHED])
def test_headdim_batched_matches_oracle(case):
    name, B, sq, sk, hq, hkv, d, causal, window, sinks, dt = case
    print("case", name, flush=True)
    inp = synth.batched_inputs(zlib.crc32(name.encode()) % 1000, B, sq, sk, hq, hkv, d, grads=True,
                               sinks=sinks, dtype=dt)
    scale = scale_of(d)
    p = oracle_batched(inp, causal, window, scale, dt)
    ref = oracle.full(p)
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd(q, k, v, causal=causal, window=window, sinks=s_dev)
    torch.cuda.synchronize()
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], dt)
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])
    for gd in (torch.float32, _torch_dtype(dt)):
        dq, dk, dv, ds = ea.attn_bwd(q, k, v, o, lse, do, causal=causal, window=window, sinks=s_dev,
                                     grad_dtype=gd)
        torch.cuda.synchronize()
        od = "f32" if gd == torch.float32 else dt
        assert_close(name + ".dq", host(dq).reshape(B * sq, hq, d), ref["dq"], od)
        assert_close(name + ".dk", host(dk).reshape(B * sk, hkv, d), ref["dk"], od)
        assert_close(name + ".dv", host(dv).reshape(B * sk, hkv, d), ref["dv"], od)
        if sinks:
            check_dsinks(name + ".dsinks", host(ds), ref["dsinks"], p)


VARLEN = [
    # id, lens_q, lens_k, hq, hkv, d, causal, window, sinks, dtype
    ("varlen_d24_gqa_sinks", [0, 17, 283, 1, 77], None, 4, 2, 24, True, (-1, -1), True, "bf16"),
    ("varlen_d104_mixed", [5, 0, 130, 64, 9], [200, 3, 130, 0, 9], 2, 2, 104, True, (50, 0), False, "fp16"),
    ("varlen_d256_gqa", [33, 190, 1, 0], [64, 190, 300, 5], 6, 2, 256, True, (-1, -1), True, "bf16"),
    ("varlen_d200_noncausal", [5, 130, 64], None, 2, 1, 200, False, (-1, -1), False, "bf16"),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_headdim_varlen_matches_oracle(case):
    name, lq, lk, hq, hkv, d, causal, window, sinks, dt = case
    print("case", name, flush=True)
    lk = lq if lk is None else lk
    inp = synth.varlen_inputs(zlib.crc32(name.encode()) % 1000, lq, lk, hq, hkv, d, grads=True, sinks=sinks,
                              dtype=dt)
    scale = scale_of(d)
    ref = oracle.full(oracle.varlen(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], scale,
                                    causal=causal, window=window, dout=inp["dout"], sinks=inp["sinks"],
                                    dtype=dt))
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    cq, ck = torch.from_numpy(inp["cu_q"]).cuda(), torch.from_numpy(inp["cu_k"]).cuda()
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=causal, window=window, sinks=s_dev)
    torch.cuda.synchronize()
    assert_close(name + ".o", host(o), ref["o"], dt)
    assert_lse(name + ".lse", host(lse), ref["lse"])
    dq, dk, dv, ds = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, max(lq), max(lk), causal=causal,
                                        window=window, sinks=s_dev, grad_dtype=_torch_dtype(dt))
    torch.cuda.synchronize()
    assert_close(name + ".dq", host(dq), ref["dq"], dt)
    assert_close(name + ".dk", host(dk), ref["dk"], dt)
    assert_close(name + ".dv", host(dv), ref["dv"], dt)


KVCACHE = [
    # id, B, sq, hq, hkv, d, lens, capacity, page, causal, window, sinks, dtype
    ("kv_d80_paged64_split", 2, 4, 8, 2, 80, [5000, 700], 5056, 64, True, (-1, -1), True, "bf16"),
    ("kv_d96_contig_q1", 4, 1, 8, 1, 96, [4096, 1, 0, 2000], 4096, 0, True, (-1, -1), False, "fp16"),
    ("kv_d256_paged256_split", 2, 8, 8, 1, 256, [6000, 257], 6144, 256, True, (-1, -1), True, "bf16"),
    ("kv_d192_contig", 3, 5, 4, 2, 192, [700, 313, 1], 700, 0, True, (-1, -1), False, "bf16"),
]


@pytest.mark.parametrize("case", KVCACHE, ids=[c[0] for c in KVCACHE])
def test_headdim_kvcache_matches_oracle(case):
    name, B, sq, hq, hkv, d, lens, cap, page, causal, window, sinks, dt = case
    print("case", name, flush=True)
    inp = synth.kvcache_inputs(zlib.crc32(name.encode()) % 1000, B, sq, hq, hkv, d, lens, cap, page=page,
                               sinks=sinks, dtype=dt)
    scale = scale_of(d)
    q, kc, vc = (dev_tensor(inp[n], dt) for n in ("q", "k", "v"))
    used = torch.from_numpy(inp["lens"]).cuda()
    bt = torch.from_numpy(inp["block_table"]).cuda() if page else None
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd_kvcache(q, kc, vc, used, block_table=bt, causal=causal, window=window, sinks=s_dev)
    torch.cuda.synchronize()
    ref = oracle.full(oracle.kvcache(inp["q"], inp["k"], inp["v"], inp["lens"], scale,
                                     block_table=inp["block_table"], causal=causal,
                                     window=window, sinks=inp["sinks"], dtype=dt), grads=False)
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], dt)
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])


@pytest.mark.parametrize("d,dt", [(8, "bf16"), (48, "fp16"), (72, "bf16"), (120, "bf16"), (136, "bf16"),
                                  (192, "fp16"), (248, "bf16")])
def test_padded_equals_explicit_zero_columns(d, dt):
    """A head dim d < D on the D-wide kernels equals, bitwise, the D-wide
    kernels on the same tensors with the zero columns written out (same
    scale): outputs, lse, dQ, dK and dV, with zero gradients in the extra
    columns of the explicit call.  Causal GQA with sinks, batched and split-KV."""
    print("case pad", d, dt, flush=True)
    D = 64 if d <= 64 else 128 if d <= 128 else 256
    for B, sq, sk in ((2, 190, 190), (1, 3, 4000)):
        inp = synth.batched_inputs(d + sq, B, sq, sk, 8, 2, d, grads=True, sinks=True, dtype=dt)
        q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
        s_dev = torch.from_numpy(inp["sinks"]).cuda()
        scale = float(synth.default_scale(d))
        pad = lambda t: F.pad(t, (0, D - d)).contiguous()  # noqa: E731
        qp, kp, vp, dop = pad(q), pad(k), pad(v), pad(do)
        o, lse = ea.attn_fwd(q, k, v, causal=True, sinks=s_dev, softmax_scale=scale)
        op, lsep = ea.attn_fwd(qp, kp, vp, causal=True, sinks=s_dev, softmax_scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(op[..., :d], o) and torch.equal(lsep, lse), (d, sq, sk)
        assert not op[..., d:].any()
        g = ea.attn_bwd(q, k, v, o, lse, do, causal=True, sinks=s_dev, softmax_scale=scale)
        gp = ea.attn_bwd(qp, kp, vp, op, lsep, dop, causal=True, sinks=s_dev, softmax_scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), g[:3], gp[:3]):
            assert torch.equal(b[..., :d], a), (name, d)
            assert not b[..., d:].any(), (name, d)
        assert torch.equal(g[3], gp[3])
