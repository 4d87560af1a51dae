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
    return ctypes.CDLL(PATH)


def test_exports(probe):
    assert hasattr(probe, "probe_read_dma") and hasattr(probe, "probe_read_regs")


@pytest.mark.parametrize("B,S,H,ns", [(0, 4096, 8, 2), (2, 4096, 8, 3), (2, 4000, 8, 2), (2, 4096, 0, 2),
                                      (1, 1 << 22, 8, 2)])
def test_bad_sizes_refused(probe, B, S, H, ns):
    null = ctypes.c_void_p(0)
    assert probe.probe_read_dma(null, null, B, S, H, ns, 1, null, null) == 1
    assert probe.probe_read_regs(null, null, B, S, H, ns, null, null) == 1
