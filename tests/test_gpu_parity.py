"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs, element by element, on shapes that span several tiles and end
in ragged tails, with the edge cases of the method: grouped-query heads,
causal and two-sided windows aligned bottom-right with s_q < s_k and
s_q > s_k (empty rows), attention sinks, fp16, split-KV decode, and packed
batches with zero-length sequences."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_attention_36_amd import synth
import exact_attention_36_amd as ea
from _helpers import (assert_close, assert_lse, check_dsinks, dev_tensor, host, oracle_batched, scale_of)

pytestmark = pytest.mark.gpu

BATCHED = [
    # id, B, sq, sk, hq, hkv, d, causal, window, sinks, dtype, bwd
    ("cfg1_fwd", 1, 128, 128, 2, 2, 64, False, (-1, -1), False, "bf16", False),
    ("causal_ragged", 2, 200, 200, 4, 2, 128, True, (-1, -1), False, "bf16", True),
    ("window_sinks_gqa4", 1, 300, 300, 8, 2, 128, True, (37, 0), True, "bf16", True),
    ("sq_lt_sk", 2, 150, 333, 4, 4, 64, True, (-1, -1), True, "bf16", True),
    ("sq_gt_sk_empty_rows", 1, 333, 150, 4, 1, 128, True, (-1, -1), False, "bf16", True),
    ("two_sided_fp16", 1, 257, 190, 2, 2, 64, False, (20, 13), False, "fp16", True),
    ("sinks_fp16_full", 1, 100, 100, 2, 1, 128, False, (-1, -1), True, "fp16", True),
    ("split_kv_decode", 2, 3, 5000, 8, 2, 128, True, (-1, -1), True, "bf16", True),
    # batched decode that does not split (15 key tiles): one work tile per
    # (sequence, kv head), so the K/V tiles take the read-once path
    ("decode_unsplit_read_once", 16, 2, 900, 32, 4, 128, True, (-1, -1), True, "bf16", True),
    # 16 q heads per kv head (8 queries fill a 128-row tile), left window only, no causal
    ("mqa_g16_left_window", 1, 96, 200, 16, 1, 64, False, (50, -1), True, "bf16", True),
    # right window only, no causal: keys up to 7 past the diagonal
    ("right_window_only", 2, 65, 65, 2, 2, 128, False, (-1, 7), False, "bf16", True),
    # one query, one key per sequence
    ("single_token", 3, 1, 1, 2, 1, 128, True, (-1, -1), True, "bf16", True),
    # 32 q heads on one kv head, 4 queries over 3000 keys (split-KV with a full 128-row tile)
    ("g32_decode_split", 1, 4, 3000, 32, 1, 128, True, (-1, -1), False, "bf16", True),
    # groups above 32 q heads per kv head with sinks: the dQ kernel's per-head
    # d(sink) sums take fewer row chunks (48 does not divide the 128-row tile).
    # fp16: each key's dV sums P over thousands of (row, head) pairs here, and
    # with bf16 inputs P enters that product rounded to bf16 (2^-9), which
    # summed over ~2900 pairs gives a mean error of 2.7e-3 (measured), above
    # the 2e-3 bar; fp16's P (2^-11) stays inside it
    ("sinks_g48_window_fp16", 1, 70, 70, 48, 1, 64, False, (30, 30), True, "fp16", True),
    ("sinks_g64_window_fp16", 2, 50, 60, 64, 1, 64, True, (10, 5), True, "fp16", True),
    ("sinks_g128_full_fp16", 1, 40, 40, 128, 1, 64, False, (-1, -1), True, "fp16", True),
    # no mask with 16 or more (sequence, kv head) groups: the batched grids run
    # each XCD's groups one after the other, every block of a group side by
    # side (ragged last query and key blocks)
    ("unmasked_16_groups", 4, 300, 300, 8, 4, 64, False, (-1, -1), False, "bf16", True),
    ("unmasked_16_groups_sq_ne_sk_sinks_fp16", 8, 260, 390, 4, 2, 128, False, (-1, -1), True, "fp16", True),
]


# the small forward workload is drawn with its workload number as the seed
SEEDS = {"cfg1_fwd": 1}


def _torch_dtype(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float16


@pytest.mark.parametrize("case", BATCHED, ids=[c[0] for c in BATCHED])
def test_batched_matches_oracle(case):
    name, B, sq, sk, hq, hkv, d, causal, window, sinks, dt, bwd = case
    print("case", name, flush=True)
    seed = SEEDS.get(name, zlib.crc32(name.encode()) % 1000)
    inp = synth.batched_inputs(seed, B, sq, sk, hq, hkv, d, grads=True, sinks=sinks, dtype=dt)
    scale = scale_of(d)
    ref = oracle.full(oracle_batched(inp, causal, window, scale, dt), grads=bwd)
    q, k, v = (dev_tensor(inp[n], dt) for n in ("q", "k", "v"))
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd(q, k, v, causal=causal, window=window, sinks=s_dev)
    o2, lse2 = ea.attn_fwd(q, k, v, causal=causal, window=window, sinks=s_dev)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "forward is not bitwise repeatable"
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], dt)
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])
    if not bwd:
        return
    do = dev_tensor(inp["dout"], dt)
    for gd in (torch.float32, _torch_dtype(dt)):
        dq, dk, dv, ds = ea.attn_bwd(q, k, v, o, lse, do, causal=causal, window=window, sinks=s_dev,
                                     grad_dtype=gd)
        torch.cuda.synchronize()
        od = "f32" if gd == torch.float32 else dt
        if gd != torch.float32:  # no output accumulates with atomics: bitwise repeatable
            dq2, dk2, dv2, ds2 = ea.attn_bwd(q, k, v, o, lse, do, causal=causal, window=window, sinks=s_dev,
                                             grad_dtype=gd)
            torch.cuda.synchronize()
            assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "backward not repeatable"
            assert ds is None or torch.equal(ds, ds2), "dsinks not repeatable"
        assert_close(name + ".dq", host(dq).reshape(B * sq, hq, d), ref["dq"], od)
        assert_close(name + ".dk", host(dk).reshape(B * sk, hkv, d), ref["dk"], od)
        assert_close(name + ".dv", host(dv).reshape(B * sk, hkv, d), ref["dv"], od)
        if sinks:
            r = oracle.rows(oracle_batched(inp, causal, window, scale, dt),
                            *_all_rows(B, sq, hq), grads=True)
            mag = np.zeros(hq)
            np.add.at(mag, _all_rows(B, sq, hq)[1], np.abs((1 - r["gate"]) * r["delta"]))
            err = np.abs(host(ds) - ref["dsinks"])
            assert np.all(err <= 2e-2 + 1e-3 * mag), (err, mag)


def _all_rows(B, sq, hq):
    s, h, i = np.meshgrid(np.arange(B), np.arange(hq), np.arange(sq), indexing="ij")
    return s.ravel(), h.ravel(), i.ravel()


VARLEN = [
    # id, lens_q, lens_k, hq, hkv, d, causal, window, sinks, dtype
    ("varlen_gqa_sinks", [0, 17, 283, 128, 1, 0, 77], None, 4, 2, 128, True, (-1, -1), True, "bf16"),
    ("varlen_mixed_pack", [5, 0, 130, 64, 9], [200, 3, 130, 0, 9], 2, 2, 64, True, (50, 0), False, "bf16"),
    ("varlen_noncausal_fp16", [33, 190, 1], [64, 190, 300], 6, 2, 128, False, (-1, -1), False, "fp16"),
    # every sequence empty but one, which is shorter than one tile, with a window
    ("varlen_one_live", [0, 0, 45, 0], [0, 0, 45, 0], 8, 4, 128, True, (10, 0), True, "bf16"),
    # queries and keys of different lengths per sequence, bottom-right aligned, GQA 8
    ("varlen_q_shorter_g8", [7, 64, 3], [300, 64, 129], 8, 1, 64, True, (-1, -1), False, "bf16"),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen_matches_oracle(case):
    name, lq, lk, hq, hkv, d, causal, window, sinks, dt = case
    print("case", name, flush=True)
    lk = lq if lk is None else lk
    inp = synth.varlen_inputs(zlib.crc32(name.encode()) % 1000, lq, lk, hq, hkv, d, grads=True, sinks=sinks,
                              dtype=dt)
    scale = scale_of(d)
    p = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], scale, causal=causal,
                      window=window, dout=inp["dout"], sinks=inp["sinks"], dtype=dt)
    ref = oracle.full(p)
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    ck = torch.from_numpy(inp["cu_k"]).cuda()
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=causal, window=window,
                                sinks=s_dev)
    torch.cuda.synchronize()
    assert_close(name + ".o", host(o), ref["o"], dt)
    assert_lse(name + ".lse", host(lse), ref["lse"])
    for gd in (torch.float32, _torch_dtype(dt)):
        dq, dk, dv, ds = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, max(lq), max(lk),
                                            causal=causal, window=window, sinks=s_dev, grad_dtype=gd)
        torch.cuda.synchronize()
        od = "f32" if gd == torch.float32 else dt
        assert_close(name + ".dq", host(dq), ref["dq"], od)
        assert_close(name + ".dk", host(dk), ref["dk"], od)
        assert_close(name + ".dv", host(dv), ref["dv"], od)
        if sinks:
            check_dsinks(name + ".dsinks", host(ds), ref["dsinks"], p)


def test_varlen_equals_batched_calls():
    """Each sequence of a packed call equals the batched call on that sequence alone (bitwise)."""
    lens = [0, 96, 200, 1, 64]
    inp = synth.varlen_inputs(3, lens, lens, 4, 1, 128, grads=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, cq, max(lens), max(lens), causal=True)
    for s, L in enumerate(lens):
        if L == 0:
            continue
        a, b = int(inp["cu_q"][s]), int(inp["cu_q"][s + 1])
        ob, lb = ea.attn_fwd(q[a:b][None].contiguous(), k[a:b][None].contiguous(), v[a:b][None].contiguous(),
                             causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], ob[0]), s
        assert torch.equal(lse[:, a:b], lb[0]), s


def test_unmasked_group_order_bitwise():
    """Without a mask a batched grid of 16 or more (sequence, kv head) groups
    runs each XCD's groups one after the other, every block of a group side
    by side, where a smaller grid runs heaviest block first over the chip.  A
    workgroup's result does not depend on when it runs, so each batch entry's
    forward and backward equal a call on that entry alone (2 groups, the other
    order) bit for bit.  Neither side splits the keys (5 key tiles)."""
    B, S, hq, hkv, d = 8, 260, 4, 2, 128
    inp = synth.batched_inputs(21, B, S, S, hq, hkv, d, grads=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    print("case unmasked_group_order", B, S, hq, hkv, d, flush=True)
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv, _ = ea.attn_bwd(q, k, v, o, lse, do, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        sl = lambda t: t[b:b + 1].contiguous()  # noqa: E731
        ob, lb = ea.attn_fwd(sl(q), sl(k), sl(v))
        dqb, dkb, dvb, _ = ea.attn_bwd(sl(q), sl(k), sl(v), ob, lb, sl(do), grad_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o[b], ob[0]), b
        assert torch.equal(lse[b], lb[0]), b
        assert torch.equal(dq[b], dqb[0]), b
        assert torch.equal(dk[b], dkb[0]), b
        assert torch.equal(dv[b], dvb[0]), b


SCHEDULE = [
    # id, causal, window, sinks, seqused
    ("causal", True, (-1, -1), False, False),
    ("causal_window_sinks", True, (700, 0), True, False),
    ("two_sided_window", False, (300, 40), False, False),
    ("causal_seqused", True, (-1, -1), False, True),
]


@pytest.mark.parametrize("case", SCHEDULE, ids=[c[0] for c in SCHEDULE])
def test_packed_schedule_tables_bitwise(case):
    """A packed batch large enough that its backward grids run in the order
    of the device-built schedule tables (longest blocks first: a dK/dV grid of
    2048 workgroups or more, a sequence of 1024 queries or more): every
    sequence's forward and backward equal a packed call on that sequence
    alone, whose grids are under the threshold and keep the layout order, bit
    for bit, and a second call on the batch repeats the first.  A block the
    tables missed would leave its rows unwritten.  (Packed calls never split
    the keys, so the two sides run the same kernels.)  With sinks, the
    batch's d(sink) is the sum of the sequences' (to rounding: the order of
    the sum differs)."""
    name, causal, window, sinks, seqused = case
    lens = [3000, 0, 17, 5000, 128, 1, 2500, 640, 0, 4095, 33, 1200, 2000, 300, 999, 4000, 666]
    lens.append(32768 - sum(lens))  # a long last sequence (8189)
    hq, hkv, d = 16, 8, 64  # dQ grid 32768*2/128+18 = 530 blocks x 8, dK/dV grid 274 x 8
    inp = synth.varlen_inputs(11, lens, lens, hq, hkv, d, grads=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    sk = torch.from_numpy(np.random.default_rng(12).standard_normal(hq).astype(np.float32)).cuda() if sinks else None
    used = None
    if seqused:  # every other sequence uses part of its slot
        used = [L if i % 2 else (L * 3) // 4 for i, L in enumerate(lens)]
    uq = torch.tensor(used, dtype=torch.int32, device="cuda") if seqused else None
    kw = dict(causal=causal, window=window, sinks=sk)
    print("case packed_schedule", name, lens, used, flush=True)
    outs = []
    for _ in range(2):
        o, lse = ea.attn_fwd_varlen(q, k, v, cq, cq, max(lens), max(lens), seqused_q=uq, seqused_k=uq, **kw)
        dq, dk, dv, ds = ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, cq, max(lens), max(lens), seqused_q=uq,
                                            seqused_k=uq, grad_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        outs.append((o, lse, dq, dk, dv, ds))
    rows = torch.ones(q.shape[0], dtype=torch.bool, device="cuda")  # query rows the call writes
    if seqused:
        for s_, L in enumerate(lens):
            a = int(inp["cu_q"][s_])
            rows[a + used[s_]:a + L] = False
    for i, (x, y) in enumerate(zip(outs[0][:5], outs[1][:5])):
        if i in (0, 2):  # o, dq: rows past the used lengths are unspecified
            x, y = x[rows], y[rows]
        elif i == 1:
            x, y = x[:, rows], y[:, rows]
        assert torch.equal(x, y), i
    if sinks:
        assert torch.equal(outs[0][5], outs[1][5])
    o, lse, dq, dk, dv, ds = outs[0]
    ds_sum = torch.zeros(hq, dtype=torch.float64, device="cuda")
    for s_, L in enumerate(lens):
        if L == 0:
            continue
        a, b = int(inp["cu_q"][s_]), int(inp["cu_q"][s_ + 1])
        sl = lambda t: t[a:b].contiguous()  # noqa: E731
        c1 = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        u1 = torch.tensor([used[s_]], dtype=torch.int32, device="cuda") if seqused else None
        ob, lb = ea.attn_fwd_varlen(sl(q), sl(k), sl(v), c1, c1, L, L, seqused_q=u1, seqused_k=u1, **kw)
        dqb, dkb, dvb, dsb = ea.attn_bwd_varlen(sl(q), sl(k), sl(v), ob, lb, sl(do), c1, c1, L, L, seqused_q=u1,
                                                seqused_k=u1, grad_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        n = used[s_] if seqused else L
        assert torch.equal(o[a:a + n], ob[:n]), s_
        assert torch.equal(lse[:, a:a + n], lb[:, :n]), s_
        assert torch.equal(dq[a:a + n], dqb[:n]), s_
        assert torch.equal(dk[a:b], dkb), s_
        assert torch.equal(dv[a:b], dvb), s_
        if sinks:
            ds_sum += dsb.double()
    if sinks:
        assert torch.allclose(ds.double(), ds_sum, rtol=1e-4, atol=1e-4), (ds, ds_sum)


RANGE = [
    # id, multipliers of q, k, v, dout (mq * mk = 1 keeps every score, hence P, unchanged)
    ("q_x1e3_k_x1e-3", 1e3, 1e-3, 1.0, 1.0),
    ("q_x1e-4_k_x1e4", 1e-4, 1e4, 1.0, 1.0),
    ("dout_x1e3", 1.0, 1.0, 1.0, 1e3),
    ("v_x1e-4_dout_x1e-2", 1.0, 1.0, 1e-4, 1e-2),
]


@pytest.mark.parametrize("case", RANGE, ids=[c[0] for c in RANGE])
def test_bf16_backward_numeric_range(case):
    """bf16 inputs far from unit scale.  The dK/dV kernel holds Q, K and dS in
    fp16 (exact for bf16 values within fp16's range, |x| <= 65504; fp16
    subnormals below 6.1e-5 keep fewer bits).  With q, k, v, dout scaled by
    mq, mk, mv, mdo (mq * mk = 1), P is unchanged, dS scales by mdo * mv, and
    dQ, dK, dV by mdo * mv * mk, mdo * mv * mq and mdo: each fp32 gradient,
    divided by its factor, must meet the unit-scale tolerance against the
    oracle's gradient of the same scaled inputs, divided likewise."""
    name, mq, mk, mv, mdo = case
    print("case", name, flush=True)
    B, S, hq, hkv, d = 1, 300, 4, 2, 128
    base = synth.batched_inputs(zlib.crc32(name.encode()) % 1000, B, S, S, hq, hkv, d, grads=True)
    scaled = lambda bits, m: synth.f32_to_bf16_bits(synth.bits_to_f32(bits) * np.float32(m))  # noqa: E731
    inp = dict(q=scaled(base["q"], mq), k=scaled(base["k"], mk), v=scaled(base["v"], mv),
               dout=scaled(base["dout"], mdo), sinks=None)
    ref = oracle.full(oracle_batched(inp, True, (100, 0), scale_of(d)))
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    o, lse = ea.attn_fwd(q, k, v, causal=True, window=(100, 0))
    dq, dk, dv, _ = ea.attn_bwd(q, k, v, o, lse, do, causal=True, window=(100, 0), grad_dtype=torch.float32)
    torch.cuda.synchronize()
    fq, fk, fv = mdo * mv * mk, mdo * mv * mq, mdo
    assert_close(name + ".dq", host(dq).reshape(B * S, hq, d) / fq, ref["dq"] / fq, "f32")
    assert_close(name + ".dk", host(dk).reshape(B * S, hkv, d) / fk, ref["dk"] / fk, "f32")
    assert_close(name + ".dv", host(dv).reshape(B * S, hkv, d) / fv, ref["dv"] / fv, "f32")
