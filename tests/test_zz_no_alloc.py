"""attn_bwd_noalloc (the backward on the library's fixed device scratch)
against attn_bwd with a caller workspace, through the C ABI: two calls in a
row on one GPU, the second smaller than the first, each required to equal
attn_bwd bit for bit (same kernels, same inputs) and the oracle's tolerance
is then met by construction.  The second call runs on scratch that still
holds the first call's row statistics."""
import ctypes

import numpy as np
import pytest
import torch

import exact_attention_36_amd as ea
from exact_attention_36_amd import _lib, synth
from _helpers import dev_tensor

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bwd_both(B, S, hq, hkv, d, sinks, causal, window, gd):
    inp = synth.batched_inputs(B * 1000 + S, B, S, S, hq, hkv, d, grads=True, sinks=sinks)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    s_dev = torch.from_numpy(inp["sinks"]).cuda() if sinks else None
    o, lse = ea.attn_fwd(q, k, v, causal=causal, window=window, sinks=s_dev)
    lib = ea.load_library()
    p = _lib.make_params(q, k, causal, window, s_dev, nseq=B)
    code = _lib.ATTN_FP32 if gd == torch.float32 else _lib.ATTN_BF16
    outs = []
    for noalloc in (False, True):
        dq = torch.empty(q.shape, dtype=gd, device="cuda")
        dk = torch.empty(k.shape, dtype=gd, device="cuda")
        dv = torch.empty(v.shape, dtype=gd, device="cuda")
        ds = torch.empty(hq, dtype=torch.float32, device="cuda") if sinks else None
        P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        args = [ctypes.byref(p), B, S, S, P(q), P(k), P(v), P(o), P(lse), P(do), P(dq), P(dk), P(dv), P(ds), code]
        if noalloc:
            st = lib.attn_bwd_noalloc(*args, _stream())
        else:
            n = lib.attn_bwd_workspace_size(ctypes.byref(p), B, S, S, code)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            st = lib.attn_bwd(*args, P(ws), n, _stream())
        assert st == 0, _lib.last_error()
        outs.append((dq, dk, dv, ds))
    torch.cuda.synchronize()
    return outs


def test_noalloc_backward_equals_workspace_backward_twice():
    # first call: GQA 8/2, sinks, causal + window, fp32 gradients
    ref, got = _bwd_both(2, 300, 8, 2, 128, True, True, (100, 0), torch.float32)
    for name, a, b in zip(("dq", "dk", "dv", "dsinks"), ref, got):
        assert torch.equal(a, b), name
    # second call, smaller: MHA, no sinks, D = 64, bf16 gradients, on scratch the first call left behind
    ref, got = _bwd_both(1, 70, 2, 2, 64, False, False, (-1, -1), torch.bfloat16)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name


def test_noalloc_binding_and_limit():
    inp = synth.batched_inputs(5, 1, 96, 96, 4, 4, 128, grads=True)
    q, k, v, do = (dev_tensor(inp[n]) for n in ("q", "k", "v", "dout"))
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    a = ea.attn_bwd(q, k, v, o, lse, do, causal=True)
    b = _lib.attn_bwd_noalloc(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    # a call whose workspace would exceed the scratch is refused before any launch
    lib = ea.load_library()
    big = _lib.attn_params()
    big.dtype, big.head_dim, big.heads_q, big.heads_kv = _lib.ATTN_BF16, 128, 64, 64
    fake = ctypes.c_void_p(0x1000)
    st = lib.attn_bwd_noalloc(ctypes.byref(big), 64, 8192, 8192, *([fake] * 9), None, _lib.ATTN_BF16, None)
    assert st == _lib.ATTN_ENOTSUP and "fixed scratch" in _lib.last_error()
