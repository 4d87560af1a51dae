"""The benchmark's read-probe library (libattn36_probe.so, built beside the
attention library): it loads, exports its two entry points, and refuses
sizes its kernels do not cover before touching the GPU."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "exact_attention_36_amd", "libattn36_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PATH):
        pytest.fail("libattn36_probe.so is not built (run __graft_entry__.build())")
    # torch first, as in bench.py: the library then binds to the HIP runtime
    # torch has loaded instead of loading a second one
    import torch  # noqa: F401
    return ctypes.CDLL(PATH)


def test_exports(probe):
    assert hasattr(probe, "probe_read_dma") and hasattr(probe, "probe_read_regs")


@pytest.mark.parametrize("B,S,H,ns", [(0, 4096, 8, 2), (2, 4096, 8, 3), (2, 4000, 8, 2), (2, 4096, 0, 2),
                                      (1, 1 << 22, 8, 2)])
def test_bad_sizes_refused(probe, B, S, H, ns):
    null = ctypes.c_void_p(0)
    assert probe.probe_read_dma(null, null, B, S, H, ns, 1, null, null) == 1
    assert probe.probe_read_regs(null, null, B, S, H, ns, null, null) == 1


def _xor_chunks(*tensors):
    """xor of every 16-byte chunk of the tensors, as two uint64 words"""
    import numpy as np
    out = np.zeros(2, dtype=np.uint64)
    for t in tensors:
        a = t.detach().cpu().contiguous().view(-1).numpy().view(np.uint64).reshape(-1, 2)
        out ^= np.bitwise_xor.reduce(a, axis=0)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["dma_default", "dma_nt", "regs"])
def test_probe_reads_every_byte_once(probe, kind):
    """The xor of the probe's sink equals the xor of all 16-byte chunks of K
    and V: every byte was read (and folded in) exactly once."""
    import torch
    B, S, H, ns = 2, 1024, 3, 2
    print("probe", kind, B, S, H, ns, flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    k = torch.randint(-2**15, 2**15, (B, S, H, 128), dtype=torch.int32, device="cuda", generator=g).to(torch.int16)
    v = torch.randint(-2**15, 2**15, (B, S, H, 128), dtype=torch.int32, device="cuda", generator=g).to(torch.int16)
    sink = torch.zeros(B * H * ns * 256 * 4, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    if kind == "regs":
        rc = probe.probe_read_regs(p(k), p(v), B, S, H, ns, p(sink), st)
    else:
        rc = probe.probe_read_dma(p(k), p(v), B, S, H, ns, int(kind == "dma_nt"), p(sink), st)
    assert rc == 0
    torch.cuda.synchronize()
    assert (_xor_chunks(sink) == _xor_chunks(k, v)).all()
