"""GPU parity of the KV-cache forward (attn_fwd_kvcache) against the fp64
oracle on seeded caches: per-slot used lengths (seqused_k) including an empty
slot and lengths that end inside a tile and inside a page, paged caches with
shuffled pages of 64 and 256 rows, GQA, causal and windowed bands aligned to
the used length, sinks, fp16, and the split-KV path for long caches."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_attention_36_amd import synth
import exact_attention_36_amd as ea
from _helpers import check_dsinks, assert_close, assert_lse, dev_tensor, host, scale_of

pytestmark = pytest.mark.gpu

CASES = [
    # id, B, sq, hq, hkv, d, lens, capacity, page, causal, window, sinks, dtype
    ("contig_seqused", 3, 5, 8, 2, 128, [700, 313, 1], 700, 0, True, (-1, -1), False, "bf16"),
    ("paged256_split_sinks", 4, 16, 16, 2, 128, [5000, 4097, 256, 0], 5120, 256, True, (-1, -1), True, "bf16"),
    ("paged64_window_fp16", 2, 33, 4, 4, 64, [650, 97], 704, 64, True, (100, 0), False, "fp16"),
    ("paged128_noncausal_gqa8", 2, 7, 16, 2, 128, [129, 1000], 1024, 128, False, (-1, -1), True, "bf16"),
    ("contig_decode_q1", 8, 1, 8, 1, 128, [4096, 1, 64, 65, 2000, 3333, 0, 4095], 4096, 0, True, (-1, -1), False,
     "bf16"),
    # 4688 pages of one tile over at most 64 splits: every split's range spans more than the 64
    # block-table entries held at a time
    ("paged64_long_split", 1, 4, 2, 1, 64, [300000], 300032, 64, True, (-1, -1), False, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kvcache_matches_oracle(case):
    name, B, sq, hq, hkv, d, lens, cap, page, causal, window, sinks, dt = case
    print("case", name, flush=True)
    seed = zlib.crc32(name.encode()) % 1000
    inp = synth.kvcache_inputs(seed, B, sq, hq, hkv, d, lens, cap, page=page, sinks=sinks, dtype=dt)
    scale = scale_of(d)
    q, kc, vc = (dev_tensor(inp[n], dt) for n in ("q", "k", "v"))
    seqlens = torch.from_numpy(inp["lens"]).cuda()
    table = torch.from_numpy(inp["block_table"]).cuda() if page else None
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd_kvcache(q, kc, vc, seqlens, block_table=table, causal=causal, window=window, sinks=s_dev)
    o2, lse2 = ea.attn_fwd_kvcache(q, kc, vc, seqlens, block_table=table, causal=causal, window=window, sinks=s_dev)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "not bitwise repeatable"
    ref = oracle.full(oracle.kvcache(inp["q"], inp["k"], inp["v"], inp["lens"], scale, block_table=inp["block_table"],
                                     causal=causal, window=window, sinks=inp["sinks"], dtype=dt), grads=False)
    assert_close(name + ".o", host(o).reshape(B * sq, hq, d), ref["o"], dt)
    assert_lse(name + ".lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])


def test_kvcache_equals_plain_forward_on_full_slots():
    """A contiguous cache whose slots are full is the batched forward, bit for bit."""
    inp = synth.kvcache_inputs(3, 2, 9, 4, 2, 128, [300, 300], 300)
    q, kc, vc = (dev_tensor(inp[n]) for n in ("q", "k", "v"))
    seqlens = torch.from_numpy(inp["lens"]).cuda()
    o, lse = ea.attn_fwd_kvcache(q, kc, vc, seqlens, causal=True)
    o2, lse2 = ea.attn_fwd(q, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_kvcache_paged_unsplit_rows_sampled():
    """Enough work tiles that the forward does not split the keys: each
    workgroup walks 100+ pages of 64 rows itself (block-table window moves);
    sampled rows plus the edges against the oracle."""
    B, sq, hq, hkv, d, page = 2, 2048, 16, 16, 128, 64
    lens = [8192, 5000]
    inp = synth.kvcache_inputs(21, B, sq, hq, hkv, d, lens, 8192, page=page)
    q, kc, vc = (dev_tensor(inp[n]) for n in ("q", "k", "v"))
    seqlens = torch.from_numpy(inp["lens"]).cuda()
    table = torch.from_numpy(inp["block_table"]).cuda()
    o, lse = ea.attn_fwd_kvcache(q, kc, vc, seqlens, block_table=table, causal=True)
    torch.cuda.synchronize()
    p = oracle.kvcache(inp["q"], inp["k"], inp["v"], inp["lens"], scale_of(d), block_table=inp["block_table"],
                       causal=True)
    rng = np.random.default_rng(22)
    seqs = np.r_[rng.integers(0, B, 256), 0, 0, 1, 1]
    heads = np.r_[rng.integers(0, hq, 256), 0, hq - 1, 0, hq - 1]
    rows = np.r_[rng.integers(0, sq, 256), 0, sq - 1, 0, sq - 1]
    r = oracle.rows(p, seqs, heads, rows)
    tok = seqs * sq + rows
    assert_close("paged_unsplit.o[rows]", host(o).reshape(B * sq, hq, d)[tok, heads], r["o"], "bf16")
    assert_lse("paged_unsplit.lse[rows]", host(lse).transpose(1, 0, 2).reshape(hq, B * sq)[heads, tok], r["lse"])


SEQUSED = [
    # id, packed, slot_q, slot_k, used_q, used_k, hq, hkv, d, causal, window, sinks, dtype
    ("seqused_packed_gqa_sinks", True, [100, 7, 0, 300, 64], [150, 64, 20, 300, 64], [60, 7, 0, 1, 64],
     [90, 0, 20, 129, 64], 4, 2, 128, True, (-1, -1), True, "bf16"),
    ("seqused_packed_window_fp16", True, [33, 190], [64, 190], [33, 100], [50, 190], 2, 1, 64, True, (20, 0),
     False, "fp16"),
    ("seqused_batched_noncausal", False, [80] * 3, [200] * 3, [80, 33, 1], [200, 64, 5], 8, 2, 128, False,
     (-1, -1), True, "bf16"),
]


@pytest.mark.parametrize("case", SEQUSED, ids=[c[0] for c in SEQUSED])
def test_seqused_forward_backward(case):
    """Slots that use only their first seqused_q / seqused_k tokens: the used
    rows' O, lse, dQ, every key's dK, dV (zero for unused keys) and dsinks
    against the oracle on the same slot layout; unused query rows are not
    compared (unspecified)."""
    name, packed, slot_q, slot_k, used_q, used_k, hq, hkv, d, causal, window, sinks, dt = case
    print("case", name, flush=True)
    seed = zlib.crc32(name.encode()) % 1000
    if packed:
        inp = synth.varlen_inputs(seed, slot_q, slot_k, hq, hkv, d, grads=True, sinks=sinks, dtype=dt)
        p = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], scale_of(d), causal=causal,
                          window=window, dout=inp["dout"], sinks=inp["sinks"], dtype=dt, seqused_q=used_q,
                          seqused_k=used_k)
        cq = np.asarray(inp["cu_q"])
    else:
        B, sq, sk = len(slot_q), slot_q[0], slot_k[0]
        inp = synth.batched_inputs(seed, B, sq, sk, hq, hkv, d, grads=True, sinks=sinks, dtype=dt)
        p = oracle.batched(inp["q"], inp["k"], inp["v"], scale_of(d), causal=causal, window=window,
                           dout=inp["dout"], sinks=inp["sinks"], dtype=dt, seqused_q=used_q, seqused_k=used_k)
        cq = np.arange(B + 1) * sq
    ref = oracle.full(p)
    q, k, v, do = (dev_tensor(inp[n], dt) for n in ("q", "k", "v", "dout"))
    kw = dict(causal=causal, window=window, sinks=torch.from_numpy(inp["sinks"]).cuda() if sinks else None,
              seqused_q=torch.tensor(used_q, dtype=torch.int32, device="cuda"),
              seqused_k=torch.tensor(used_k, dtype=torch.int32, device="cuda"))
    if packed:
        cqd, ckd = torch.from_numpy(inp["cu_q"]).cuda(), torch.from_numpy(inp["cu_k"]).cuda()
        o, lse = ea.attn_fwd_varlen(q, k, v, cqd, ckd, max(slot_q), max(slot_k), **kw)
        dq, dk, dv, ds = ea.attn_bwd_varlen(q, k, v, o, lse, do, cqd, ckd, max(slot_q), max(slot_k),
                                            grad_dtype=torch.float32, **kw)
        oh, lh, dqh = host(o), host(lse), host(dq)
        dkh, dvh = host(dk), host(dv)
    else:
        o, lse = ea.attn_fwd(q, k, v, **kw)
        dq, dk, dv, ds = ea.attn_bwd(q, k, v, o, lse, do, grad_dtype=torch.float32, **kw)
        oh = host(o).reshape(-1, hq, d)
        lh = host(lse).transpose(1, 0, 2).reshape(hq, -1)
        dqh = host(dq).reshape(-1, hq, d)
        dkh, dvh = host(dk).reshape(-1, hkv, d), host(dv).reshape(-1, hkv, d)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(cq[b], cq[b] + used_q[b]) for b in range(len(used_q))]).astype(np.int64)
    assert_close(name + ".o", oh[rows], ref["o"][rows], dt)
    assert_lse(name + ".lse", lh[:, rows], ref["lse"][:, rows])
    assert_close(name + ".dq", dqh[rows], ref["dq"][rows], "f32")
    assert_close(name + ".dk", dkh, ref["dk"], "f32")  # unused keys: exactly 0 on both sides
    assert_close(name + ".dv", dvh, ref["dv"], "f32")
    if sinks:
        check_dsinks(name + ".dsinks", host(ds), ref["dsinks"], p)
