"""The Python binding rejects tensors the C ABI cannot describe (wrong shapes,
mixed dtypes, strided views, caller-supplied outputs of the wrong shape, host
tensors) with ValueError before any library call.  Host tensors only: every
case fails validation before a pointer reaches the library."""
import pytest
import torch

import exact_attention_36_amd as ea

B, S, HQ, HKV, D = 2, 16, 4, 2, 64


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _qkv():
    return _t(B, S, HQ, D), _t(B, S, HKV, D), _t(B, S, HKV, D)


def test_well_formed_host_tensors_are_refused_for_the_device():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU"):
        ea.attn_fwd(q, k, v)


@pytest.mark.parametrize("case,needle", [
    ("v_shape", "v must have shape"),
    ("k_batch", "k must have shape"),
    ("k_headdim", "k must have shape"),
    ("kv_dtype", "k must have q's dtype"),
    ("fp32_q", "q must be bf16 or fp16"),
    ("strided_q", "q must be contiguous"),
    ("out_shape", "out must have shape"),
    ("out_dtype", "out must have q's dtype"),
    ("lse_shape", "lse must have shape"),
    ("lse_dtype", "lse must be fp32"),
    ("three_d", "must be \\[B, S, H, D\\]"),
])
def test_forward_rejections(case, needle):
    q, k, v = _qkv()
    kw = {}
    if case == "v_shape":
        v = _t(B, S + 1, HKV, D)
    elif case == "k_batch":
        k = _t(B + 1, S, HKV, D)
    elif case == "k_headdim":
        k = _t(B, S, HKV, D + 8)
    elif case == "kv_dtype":
        k, v = k.half(), v.half()
    elif case == "fp32_q":
        q, k, v = q.float(), k.float(), v.float()
    elif case == "strided_q":
        q = _t(B, HQ, S, D).transpose(1, 2)
    elif case == "out_shape":
        kw["out"] = _t(B, S, HQ, D + 8)
    elif case == "out_dtype":
        kw["out"] = _t(B, S, HQ, D, dtype=torch.float16)
    elif case == "lse_shape":
        kw["lse"] = _t(B, S, HQ, dtype=torch.float32)
    elif case == "lse_dtype":
        kw["lse"] = _t(B, HQ, S, dtype=torch.bfloat16)
    elif case == "three_d":
        q = _t(B * S, HQ, D)
    with pytest.raises(ValueError, match=needle):
        ea.attn_fwd(q, k, v, **kw)


@pytest.mark.parametrize("case,needle", [
    ("dout_expanded", "dout must be contiguous"),
    ("dout_shape", "dout must have shape"),
    ("o_dtype", "o must have q's dtype"),
    ("lse_shape", "lse must have shape"),
    ("grad_dtype", "grad_dtype"),
])
def test_backward_rejections(case, needle):
    q, k, v = _qkv()
    o, do = _t(B, S, HQ, D), _t(B, S, HQ, D)
    lse = _t(B, HQ, S, dtype=torch.float32)
    kw = {}
    if case == "dout_expanded":
        do = _t(1, S, HQ, D).expand(B, S, HQ, D)
    elif case == "dout_shape":
        do = _t(B, S, HQ + 1, D)
    elif case == "o_dtype":
        o = o.half()
    elif case == "lse_shape":
        lse = _t(HQ, B * S, dtype=torch.float32)
    elif case == "grad_dtype":
        kw["grad_dtype"] = torch.float16
    with pytest.raises(ValueError, match=needle):
        ea.attn_bwd(q, k, v, o, lse, do, **kw)


def test_varlen_rejections():
    q, k, v = _t(40, HQ, D), _t(40, HKV, D), _t(40, HKV, D)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens_k must have shape"):
        ea.attn_fwd_varlen(q, k, v, cu, torch.tensor([0, 40], dtype=torch.int32), 30, 30)
    with pytest.raises(ValueError, match="cu_seqlens_q must be int32"):
        ea.attn_fwd_varlen(q, k, v, cu.long(), cu, 30, 30)
    with pytest.raises(ValueError, match="lse must have shape"):
        ea.attn_fwd_varlen(q, k, v, cu, cu, 30, 30, lse=_t(40, HQ, dtype=torch.float32))
    with pytest.raises(ValueError, match="v must have shape"):
        ea.attn_fwd_varlen(q, k, _t(41, HKV, D), cu, cu, 30, 30)
    with pytest.raises(ValueError, match="dout must have shape"):
        ea.attn_bwd_varlen(q, k, v, q, _t(HQ, 40, dtype=torch.float32), _t(39, HQ, D), cu, cu, 30, 30)


def test_kvcache_rejections():
    q = _t(B, 4, HQ, D)
    kc, vc = _t(B, 64, HKV, D), _t(B, 64, HKV, D)
    lens = torch.full((B,), 10, dtype=torch.int32)
    with pytest.raises(ValueError, match="seqused_k is not accepted"):
        ea.attn_fwd_kvcache(q, kc, vc, lens, seqused_k=lens)
    with pytest.raises(ValueError, match="cache_seqlens must have shape"):
        ea.attn_fwd_kvcache(q, kc, vc, torch.full((B + 1,), 10, dtype=torch.int32))
    with pytest.raises(ValueError, match="v_cache must have shape"):
        ea.attn_fwd_kvcache(q, kc, _t(B, 32, HKV, D), lens)
    with pytest.raises(ValueError, match="block_table must be int32"):
        ea.attn_fwd_kvcache(q, kc, vc, lens, block_table=torch.zeros((B, 1), dtype=torch.int64))


def test_side_tensors():
    from exact_attention_36_amd import _lib
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="sinks must be contiguous fp32"):
        _lib.make_params(q, k, sinks=torch.zeros(HQ, dtype=torch.float64))
    with pytest.raises(ValueError, match="seqused_q must be contiguous int32"):
        _lib.make_params(q, k, nseq=B, seqused_q=torch.zeros(B + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="alibi_slopes must be contiguous fp32"):
        _lib.make_params(q, k, nseq=B, alibi_slopes=torch.zeros(HQ + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        _lib.make_params(q, k, sinks=torch.zeros(HQ, dtype=torch.float32))
