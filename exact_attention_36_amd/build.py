"""Build libattn36.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shlex
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libattn36.so")
# the benchmark's HBM read-rate reference (not part of the attention library)
PROBE_SOURCE = "read_probe.hip"
PROBE_PATH = os.path.join(PKG, "libattn36_probe.so")
SOURCES = ["attn_api.cpp", "attn_timing.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_cache.hip", "attn_noalloc.hip",
           "attn_sched.hip",
           # one translation unit per score variant, compiled in parallel
           "attn_fwd_cap.hip", "attn_fwd_alibi.hip", "attn_fwd_cap_alibi.hip",
           "attn_bwd_cap.hip", "attn_bwd_alibi.hip", "attn_bwd_cap_alibi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n%s\n%s%s" % (" ".join(shlex.quote(c) for c in cmd),
                                                        r.stdout, r.stderr))


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libattn36.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(os.cpu_count() or 4, 16, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    _run([HIPCC, *FLAGS, "-shared", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    tmp = PROBE_PATH + ".tmp%d" % os.getpid()
    _run([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp])
    os.replace(tmp, PROBE_PATH)
    if verbose:
        print("built", LIB_PATH, "and", PROBE_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
