"""GPU parity of the KV-cache update path against the fp64 oracle: rotary
embedding (interleaved and half-split pairs, per-token or shared positions,
bf16 and fp16), the in-place append of new keys and values into contiguous
and paged caches (keys rotated at their cache positions), and the whole
decode step of flash_attn_with_kvcache -- append, rotate q, attend over the
grown cache.  Rotated values are rounded to 16 bits from fp32 in the kernel
and from fp64 in the oracle, so they may differ by one unit in the last
place; copied values and untouched cache rows must be equal."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_36_amd import synth
import exact_attention_36_amd as ea
from _helpers import assert_close, assert_lse, dev_tensor, host, scale_of

pytestmark = pytest.mark.gpu


def _tables(n_pos, rotary_dim):
    theta = 10000.0 ** (-np.arange(0, rotary_dim, 2) / rotary_dim)
    ang = np.arange(n_pos)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _within_one_ulp(name, got, ref):
    """16-bit patterns: equal, or neighbours (same sign, codes one apart)."""
    g, r = got.astype(np.int32), ref.astype(np.int32)
    same_sign = (g & 0x8000) == (r & 0x8000)
    ok = (g == r) | (same_sign & (np.abs(g - r) == 1))
    assert ok.all(), "%s: %d codes differ by more than one ulp" % (name, int((~ok).sum()))
    assert (g == r).mean() > 0.9, "%s: only %.3f equal" % (name, (g == r).mean())


def _rng_bits(rng, shape, dt):
    return oracle.encode(dt, rng.standard_normal(shape))


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("rdim,per_token", [(64, True), (128, False), (32, True)])
def test_rotary_matches_oracle(dt, interleaved, rdim, per_token):
    rng = np.random.default_rng(rdim + 2 * interleaved + per_token)
    B, S, H, d = 2, 7, 3, 128
    xb = _rng_bits(rng, (B, S, H, d), dt)
    pos0 = np.array([5, 100], np.int32)
    cos, sin = _tables(128, rdim)
    x = dev_tensor(xb, dt)
    out = ea.attn_rotary(x, torch.from_numpy(pos0).cuda(), torch.from_numpy(cos).cuda(),
                         torch.from_numpy(sin).cuda(), interleaved=interleaved, per_token=per_token)
    torch.cuda.synchronize()
    pos = pos0[:, None] + (np.arange(S)[None, :] if per_token else 0)
    ref = oracle.encode(dt, oracle.rotary(oracle.decode_array(dt, xb), cos.astype(np.float64),
                                          sin.astype(np.float64), pos, rdim, interleaved))
    _within_one_ulp("rotary", _bits(out), ref)
    np.testing.assert_array_equal(_bits(out)[..., rdim:], xb[..., rdim:])
    # in place
    ea.attn_rotary(x, torch.from_numpy(pos0).cuda(), torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(),
                   interleaved=interleaved, per_token=per_token, out=x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(x), _bits(out))


@pytest.mark.parametrize("paged,rotary", [(False, False), (False, True), (True, True), (True, False)])
def test_append_matches_oracle(paged, rotary):
    rng = np.random.default_rng(10 + 2 * paged + rotary)
    B, sn, hkv, d, cap, page = 3, 5, 2, 128, 256, 64
    lens = np.array([0, 100, cap - 2], np.int32)  # the last slot has room for 2 of the 5 new rows
    kn, vn = _rng_bits(rng, (B, sn, hkv, d), "bf16"), _rng_bits(rng, (B, sn, hkv, d), "bf16")
    if paged:
        npg = cap // page
        table = rng.permutation(B * npg).reshape(B, npg).astype(np.int32)
        kc, vc = _rng_bits(rng, (B * npg, page, hkv, d), "bf16"), _rng_bits(rng, (B * npg, page, hkv, d), "bf16")
    else:
        table = None
        kc, vc = _rng_bits(rng, (B, cap, hkv, d), "bf16"), _rng_bits(rng, (B, cap, hkv, d), "bf16")
    cos, sin = _tables(cap, 64) if rotary else (None, None)
    kcd, vcd = dev_tensor(kc), dev_tensor(vc)
    lens_d = torch.from_numpy(lens).cuda()
    new = ea.attn_kvcache_append(dev_tensor(kn), dev_tensor(vn), kcd, vcd, lens_d,
                                 block_table=None if table is None else torch.from_numpy(table).cuda(),
                                 rotary_cos=None if cos is None else torch.from_numpy(cos).cuda(),
                                 rotary_sin=None if sin is None else torch.from_numpy(sin).cuda(),
                                 rotary_interleaved=False)
    torch.cuda.synchronize()
    rk, rv, rl = oracle.kvcache_append(kc, vc, lens, kn, vn, block_table=table,
                                       rotary_cos=None if cos is None else cos.astype(np.float64),
                                       rotary_sin=None if sin is None else sin.astype(np.float64), rotary_dim=64,
                                       rotary_interleaved=False)
    np.testing.assert_array_equal(new.cpu().numpy(), rl)
    np.testing.assert_array_equal(_bits(vcd), rv)
    if rotary:
        _within_one_ulp("k cache", _bits(kcd), rk)
    else:
        np.testing.assert_array_equal(_bits(kcd), rk)
    # in-place lengths
    ea.attn_kvcache_append(dev_tensor(kn), dev_tensor(vn), kcd, vcd, lens_d,
                           block_table=None if table is None else torch.from_numpy(table).cuda(), seqlens_out=lens_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lens_d.cpu().numpy(), lens + sn)


@pytest.mark.parametrize("paged,causal,interleaved", [(False, True, False), (True, True, True), (True, False, False)])
def test_decode_step_matches_oracle(paged, causal, interleaved):
    """attn_fwd_kvcache with new keys/values and rotary tables: the cache grows
    in place, q and the new keys are rotated at their positions (q all at the
    old length when neither causal nor windowed), and attention covers the
    grown cache."""
    rng = np.random.default_rng(20 + paged + 2 * causal)
    B, sq, hq, hkv, d, cap, page, rdim = 3, 4, 8, 2, 128, 512, 128, 64
    lens = np.array([300, 0, 77], np.int32)
    q = _rng_bits(rng, (B, sq, hq, d), "bf16")
    kn, vn = _rng_bits(rng, (B, sq, hkv, d), "bf16"), _rng_bits(rng, (B, sq, hkv, d), "bf16")
    if paged:
        npg = cap // page
        table = rng.permutation(B * npg).reshape(B, npg).astype(np.int32)
        kc, vc = _rng_bits(rng, (B * npg, page, hkv, d), "bf16"), _rng_bits(rng, (B * npg, page, hkv, d), "bf16")
    else:
        table = None
        kc, vc = _rng_bits(rng, (B, cap, hkv, d), "bf16"), _rng_bits(rng, (B, cap, hkv, d), "bf16")
    cos, sin = _tables(cap, rdim)
    kcd, vcd = dev_tensor(kc), dev_tensor(vc)
    o, lse = ea.attn_fwd_kvcache(dev_tensor(q), kcd, vcd, torch.from_numpy(lens).cuda(),
                                 block_table=None if table is None else torch.from_numpy(table).cuda(),
                                 causal=causal, k_new=dev_tensor(kn), v_new=dev_tensor(vn),
                                 rotary_cos=torch.from_numpy(cos).cuda(), rotary_sin=torch.from_numpy(sin).cuda(),
                                 rotary_interleaved=interleaved)
    torch.cuda.synchronize()
    c64, s64 = cos.astype(np.float64), sin.astype(np.float64)
    rk, rv, rl = oracle.kvcache_append(kc, vc, lens, kn, vn, block_table=table, rotary_cos=c64, rotary_sin=s64,
                                       rotary_dim=rdim, rotary_interleaved=interleaved)
    qpos = lens[:, None] + (np.arange(sq)[None, :] if causal else 0)
    qr = oracle.encode("bf16", oracle.rotary(oracle.decode_array("bf16", q), c64, s64, qpos, rdim, interleaved))
    ref = oracle.full(oracle.kvcache(qr, rk, rv, rl, scale_of(d), block_table=table, causal=causal), grads=False)
    _within_one_ulp("k cache", _bits(kcd), rk)
    np.testing.assert_array_equal(_bits(vcd), rv)
    assert_close("o", host(o).reshape(B * sq, hq, d), ref["o"], "bf16")
    assert_lse("lse", host(lse).transpose(1, 0, 2).reshape(hq, B * sq), ref["lse"])
