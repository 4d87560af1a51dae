"""The C ABI on the CPU: the library loads, exports every function that
include/attn.h declares, and rejects bad arguments on the host (status code
and message) before launching anything.  No call here reaches a GPU."""
import ctypes
import os
import re

import pytest

import exact_attention_36_amd as ea
from exact_attention_36_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ea.load_library()
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert ea.version() == 100


def _params(**kw):
    p = _lib.attn_params()
    p.dtype, p.head_dim, p.heads_q, p.heads_kv = _lib.ATTN_BF16, 128, 4, 2
    p.softmax_scale, p.causal, p.window_left, p.window_right, p.sinks = 0.0, 1, -1, -1, None
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _fwd(p, B=1, sq=16, sk=16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=None, nws=0):
    return ea.load_library().attn_fwd(ctypes.byref(p) if p is not None else None, B, sq, sk, q, k, v, o,
                                      lse, ws, nws, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=7), _lib.ATTN_EINVAL, "dtype"),
    (dict(head_dim=0), _lib.ATTN_EINVAL, "multiple of 8"),
    (dict(head_dim=100), _lib.ATTN_EINVAL, "multiple of 8"),
    (dict(head_dim=512), _lib.ATTN_EINVAL, "multiple of 8"),
    (dict(heads_q=6, heads_kv=4), _lib.ATTN_EINVAL, "divide"),
    (dict(heads_kv=0), _lib.ATTN_EINVAL, ">= 1"),
    (dict(window_left=-2), _lib.ATTN_EINVAL, "window"),
    (dict(window_right=-5), _lib.ATTN_EINVAL, "window"),
    (dict(causal=2), _lib.ATTN_EINVAL, "causal"),
    (dict(num_sinks=-1), _lib.ATTN_EINVAL, "num_sinks"),
    (dict(num_sinks=65), _lib.ATTN_EINVAL, "num_sinks"),
    (dict(sinks_shared=2), _lib.ATTN_EINVAL, "sinks_shared"),
    (dict(softcap=-1.0), _lib.ATTN_EINVAL, "softcap"),
    (dict(softcap=float("inf")), _lib.ATTN_EINVAL, "softcap"),
    (dict(softcap=float("nan")), _lib.ATTN_EINVAL, "softcap"),
    (dict(alibi_per_batch=3), _lib.ATTN_EINVAL, "alibi_per_batch"),
])
def test_fwd_rejects_bad_params(kw, status, needle):
    assert _fwd(_params(**kw)) == status
    assert needle in ea.last_error()


def test_fwd_rejects_bad_shapes_and_pointers():
    assert _fwd(None) == _lib.ATTN_EINVAL
    assert "NULL" in ea.last_error()
    assert _fwd(_params(), B=0) == _lib.ATTN_EINVAL
    assert _fwd(_params(), sq=0) == _lib.ATTN_EINVAL
    assert _fwd(_params(), sk=-3) == _lib.ATTN_EINVAL
    assert _fwd(_params(), q=None) == _lib.ATTN_EINVAL
    assert _fwd(_params(), lse=None) == _lib.ATTN_EINVAL
    assert _fwd(_params(), sq=1 << 24) == _lib.ATTN_ENOTSUP
    assert "offset" in ea.last_error()


def test_fwd_split_workspace_is_checked():
    p = _params(heads_q=64, heads_kv=8)
    lib = ea.load_library()
    need = lib.attn_fwd_workspace_size(ctypes.byref(p), 2, 16, 32768)
    assert need > 0  # decode shape: keys are split among workgroups
    assert _fwd(p, B=2, sq=16, sk=32768, ws=None, nws=0) == _lib.ATTN_EINVAL
    assert "workspace" in ea.last_error()
    assert _fwd(p, B=2, sq=16, sk=32768, ws=FAKE, nws=need - 1) == _lib.ATTN_EINVAL
    # a long prefill does not split
    assert lib.attn_fwd_workspace_size(ctypes.byref(p), 4, 2048, 2048) == 0


def test_bwd_rejects_bad_arguments():
    lib = ea.load_library()
    p = _params()
    args = lambda **o: [o.get(n, FAKE) for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv")]
    call = lambda p, gd=_lib.ATTN_BF16, ds=None, ws=None, nws=0, **o: lib.attn_bwd(
        ctypes.byref(p), 1, 16, 16, *args(**o), ds, gd, ws, nws, None)
    assert call(p, gd=_lib.ATTN_FP16) == _lib.ATTN_EINVAL
    assert "grad_dtype" in ea.last_error()
    assert call(p, dout=None) == _lib.ATTN_EINVAL
    ps = _params(sinks=0x2000)
    assert call(ps, ds=None) == _lib.ATTN_EINVAL
    assert "dsinks" in ea.last_error()
    need = lib.attn_bwd_workspace_size(ctypes.byref(p), 1, 16, 16, _lib.ATTN_BF16)
    assert need >= 2 * 16 * 4 * 4  # D_i and the sink-adjusted lse per (row, q head)
    assert call(p, ws=FAKE, nws=need - 1) == _lib.ATTN_EINVAL
    assert "workspace" in ea.last_error()
    assert call(p, ws=None, nws=0) == _lib.ATTN_EINVAL


def test_kvcache_rejects_bad_arguments():
    lib = ea.load_library()
    p = _params()
    call = lambda q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, bt=None, nb=0, page=0, cap=64, o=FAKE, lse=FAKE, sq=4: \
        lib.attn_fwd_kvcache(ctypes.byref(p), 2, sq, q, kc, vc, sl, bt, nb, page, cap, o, lse, None, 0, None)
    assert call(sl=None) == _lib.ATTN_EINVAL
    assert "cache_seqlens" in ea.last_error()
    assert call(cap=0) == _lib.ATTN_EINVAL            # no block table: the slot capacity is needed
    assert call(bt=FAKE, nb=0, page=256) == _lib.ATTN_EINVAL
    assert call(bt=FAKE, nb=4, page=100) == _lib.ATTN_EINVAL   # pages hold whole 64-key tiles
    assert "page_block_size" in ea.last_error()
    assert call(sq=0) == _lib.ATTN_EINVAL
    assert call(bt=FAKE, nb=1 << 20, page=1 << 10) == _lib.ATTN_ENOTSUP
    # the workspace query follows the same cache arguments
    assert lib.attn_fwd_kvcache_workspace_size(ctypes.byref(p), 2, 4, None, 0, 0, 0) == 0
    assert lib.attn_fwd_kvcache_workspace_size(ctypes.byref(p), 2, 4, FAKE, 128, 256, 0) > 0


def test_varlen_rejects_bad_arguments():
    lib = ea.load_library()
    p = _params()
    call = lambda n=2, tq=10, tk=10, cq=FAKE, ck=FAKE, mq=8, mk=8: lib.attn_fwd_varlen(
        ctypes.byref(p), n, tq, tk, cq, ck, mq, mk, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert call(n=0) == _lib.ATTN_EINVAL
    assert call(cq=None) == _lib.ATTN_EINVAL
    assert call(tq=-1) == _lib.ATTN_EINVAL
    assert call(mq=-1) == _lib.ATTN_EINVAL
    assert call(mk=1 << 26) == _lib.ATTN_ENOTSUP
    assert lib.attn_bwd_varlen(ctypes.byref(_params(dtype=5)), 2, 10, 10, FAKE, FAKE, 8, 8, *([FAKE] * 9),
                               None, 0, None, 0, None) == _lib.ATTN_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load_library()


def test_append_and_rotary_reject_bad_arguments():
    lib = ea.load_library()
    p = _params(dtype=_lib.ATTN_BF16, head_dim=64)
    def app(**kw):
        a = dict(B=1, sn=1, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, out=None, bt=None, nb=0, page=0, cap=16,
                 cos=None, sin=None, rd=0, inter=1, nro=0)
        a.update(kw)
        return lib.attn_kvcache_append(ctypes.byref(p), a["B"], a["sn"], a["kn"], a["vn"], a["kc"], a["vc"], a["lens"],
                                       a["out"], a["bt"], a["nb"], a["page"], a["cap"], a["cos"], a["sin"], a["rd"],
                                       a["inter"], a["nro"], None)
    assert app(sn=0) == _lib.ATTN_EINVAL
    assert app(kn=None) == _lib.ATTN_EINVAL
    assert app(lens=None) == _lib.ATTN_EINVAL
    assert app(cap=0) == _lib.ATTN_EINVAL
    assert app(bt=FAKE, nb=0, page=64) == _lib.ATTN_EINVAL
    assert app(bt=FAKE, nb=4, page=0) == _lib.ATTN_EINVAL
    assert app(cos=FAKE, sin=FAKE, rd=24, nro=8) == _lib.ATTN_EINVAL  # not a multiple of 16
    assert "rotary_dim" in ea.last_error()
    assert app(cos=FAKE, sin=FAKE, rd=80, nro=8) == _lib.ATTN_EINVAL  # above the head dim
    assert app(cos=FAKE, sin=None, rd=32, nro=8) == _lib.ATTN_EINVAL
    assert app(cos=FAKE, sin=FAKE, rd=32, nro=0) == _lib.ATTN_EINVAL
    assert app(cos=FAKE, sin=FAKE, rd=32, nro=8, inter=2) == _lib.ATTN_EINVAL
    def rot(**kw):
        a = dict(B=1, S=1, H=1, x=FAKE, out=FAKE, pos=FAKE, per=1, cos=FAKE, sin=FAKE, rd=32, inter=0, nro=4)
        a.update(kw)
        return lib.attn_rotary(ctypes.byref(p), a["B"], a["S"], a["H"], a["x"], a["out"], a["pos"], a["per"], a["cos"],
                               a["sin"], a["rd"], a["inter"], a["nro"], None)
    assert rot(H=0) == _lib.ATTN_EINVAL
    assert rot(pos=None) == _lib.ATTN_EINVAL
    assert rot(per=3) == _lib.ATTN_EINVAL
    assert rot(rd=0) == _lib.ATTN_EINVAL


def test_thirty_two_bit_limits_are_rejected():
    """Sizes past the kernels' 32-bit index arithmetic: the fast division of a
    sequence's packed rows by the group size (exact for queries * G^2 < 2^32)
    and the backward's row-statistics descriptor (query rows x q heads < 2^29)."""
    lib = ea.load_library()
    # G = 128, D = 8: the byte-offset check passes, the group division does not
    p = _params(heads_q=128, heads_kv=1, head_dim=8)
    assert _fwd(p, sq=300000, sk=16) == _lib.ATTN_ENOTSUP
    assert "group division" in ea.last_error()
    assert _fwd(p, sq=200000, sk=16, lse=None) == _lib.ATTN_EINVAL  # within range: fails on the NULL lse instead
    p = _params(heads_q=64, heads_kv=64, head_dim=8, causal=0)
    args = [FAKE] * 9
    st = lib.attn_bwd(ctypes.byref(p), 16, 600000, 16, *args, None, _lib.ATTN_BF16, FAKE, 1 << 40, None)
    assert st == _lib.ATTN_ENOTSUP
    assert "row-statistics" in ea.last_error()


def test_noalloc_backward_refuses_oversize_and_bad_arguments():
    """attn_bwd_noalloc checks its arguments like attn_bwd and refuses, on the
    host, a call whose workspace would not fit the fixed scratch."""
    lib = ea.load_library()
    args = [FAKE] * 9
    p = _params(heads_q=64, heads_kv=64)
    assert lib.attn_bwd_noalloc(ctypes.byref(p), 64, 8192, 8192, *args, None, _lib.ATTN_BF16, None) == \
        _lib.ATTN_ENOTSUP
    assert "fixed scratch" in ea.last_error()
    assert lib.attn_bwd_noalloc(ctypes.byref(_params()), 1, 16, 16, *args, None, _lib.ATTN_FP16, None) == \
        _lib.ATTN_EINVAL
    assert lib.attn_bwd_noalloc(ctypes.byref(_params()), 0, 16, 16, *args, None, _lib.ATTN_BF16, None) == \
        _lib.ATTN_EINVAL
    assert lib.attn_bwd_noalloc(ctypes.byref(_params(sinks=0x2000)), 1, 16, 16, *args, None, _lib.ATTN_BF16,
                                None) == _lib.ATTN_EINVAL
