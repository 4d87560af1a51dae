"""Benchmark: one step = the fused attention forward plus backward on the
causal prefill workload B=4, Hq=Hkv=16, S=2048, D=128, bf16 (seeded synthetic
N(0,1) inputs resident in HBM), through the C ABI.

Prints one JSON line.  `value` is fwd+bwd algorithmic TFLOP/s (14 * D * visible
(query, key) pairs per step: 4*D forward, 10*D backward) at the median of the
K timed steps, each timed with HIP events after a 512 MB read that flushes
the MALL (min, p90 and the unflushed "warm" steps are reported beside it).
`roofline` reports the kernel with the most time per step (found in a pass
with every launch timed), whose launches in the timed region are bracketed by
HIP events on the library's stream.  `config_lines` measures the other
workloads the same way -- the tiny forward (config 1, µs per call), GQA with a
window and sinks (config 3) and the packed batch (config 4), forward and
backward against the MFMA and HBM rooflines -- and `decode` the decode-shaped
forward (config 5) as K/V HBM GB/s, contiguous and paged.  `cpu_baseline`
times the fp64 CPU oracle on whole (batch, head) slices of the workload,
checks the GPU's outputs of the timed steps against those slices, and samples
query rows of the other configs.  `--workload decode` runs only the decode
shape; `--workload sweep`, `headdims`, `variants` and `configs` (the five
parity workloads) print one line per shape; `--workload latency` times the
launch-bound shape eagerly and as graph replays.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published

WORKLOAD = dict(name="causal prefill fwd+bwd B4 H16 S2048 D128 bf16", B=4, S=2048, HQ=16, HKV=16,
                D=128, causal=True, window=(-1, -1))


def visible_pairs(B, sq, sk, hq, causal, window):
    """Number of (query, key) pairs the mask keeps, summed over batch and q heads."""
    import numpy as np
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    diag = i + sk - sq
    keep = np.ones((sq, sk), bool)
    if causal:
        keep &= j <= diag
    if window[0] >= 0:
        keep &= j >= diag - window[0]
    if window[1] >= 0:
        keep &= j <= diag + window[1]
    return int(keep.sum()) * B * hq


_FWD = ["exact_attention_36_amd/csrc/attn_fwd_kernels.h", "exact_attention_36_amd/csrc/attn_fwd.hip"]
_BWD = ["exact_attention_36_amd/csrc/attn_bwd_kernels.h", "exact_attention_36_amd/csrc/attn_bwd.hip"]
KERNEL_SOURCES = {"fwd": _FWD, "fwd_decode": _FWD, "bwd_dkdv": _BWD, "bwd_dq": _BWD}
COMMON_SOURCES = ["exact_attention_36_amd/csrc/attn_device.h", "exact_attention_36_amd/csrc/attn_common.h",
                  "exact_attention_36_amd/csrc/attn_kernels.h", "exact_attention_36_amd/csrc/attn_api.cpp"]


def kernel_source_hash(kernel: str) -> str:
    """sha256 over the source files a kernel is built from."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(kernel: str):
    """HBM bytes per launch of `kernel` from its committed counter summary, or None.

    profiles/counters_<kernel>.txt holds `key: value` lines: the FETCH_SIZE and
    WRITE_SIZE readings per dispatch, each scaled by the factor a plain copy
    kernel of known size gave in the same run, and the hash of the kernel
    sources they were measured with; if the sources changed since, the
    counters no longer describe this kernel and the result is None.
    """
    path = os.path.join(ROOT, "profiles", "counters_%s.txt" % kernel)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


def copy_calibration():
    """A plain elementwise copy of known size (read 256 MiB, write 256 MiB),
    run before the steps so that a counter run sees it beside the kernels."""
    import torch
    n = 128 << 20  # bf16 elements
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


DECODE = dict(name="decode / chunked-prefill fwd B32 s_q16 s_kv32768 Hq64 Hkv8 D128 bf16 causal", B=32, SQ=16,
              SK=32768, HQ=64, HKV=8, D=128)
DECODE_BATCHED = dict(name="batched decode fwd B128 s_q1 s_kv8192 Hq64 Hkv8 D128 bf16 causal (keys not split)",
                      B=128, SQ=1, SK=8192, HQ=64, HKV=8, D=128)
FLUSH_BYTES = 512 << 20  # twice the 256 MB MALL (last-level cache)
SPIN_CYCLES = 200000     # torch.cuda._sleep before a timed call in the flush check


class Flusher:
    """Reads a 512 MB buffer (a reduction kernel on the current stream),
    which evicts the tiles the previous repetition left in the MALL.  The
    buffer is written once, here; the per-repetition flush only reads it, so
    the MALL is left holding clean lines and the timed kernel that follows
    pays for no write-back of the flush's own data (a 512 MB write before
    each repetition evicts as well but slows the next kernel by that
    write-back: `--workload flush` measures both)."""

    def __init__(self):
        import torch
        self.buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
        self.sink = torch.empty((), dtype=torch.int64, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


class WriteFlusher:
    """The alternative flush: a 512 MB write (fill kernel) before each
    repetition; kept for the comparison in `--workload flush`."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.i = 0

    def __call__(self):
        self.i = (self.i + 1) & 0xFF
        self.buf.fill_(self.i)


def time_each(fn, reps, flush=None):
    """Per-repetition milliseconds of fn() from HIP events on the current
    stream (the library's stream); with `flush`, the MALL flush runs before
    each repetition, outside its events."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def summary(ts):
    """median, min and p90 (nearest rank) of a list of milliseconds."""
    a = sorted(ts)
    n = len(a)
    med = a[n // 2] if n % 2 else 0.5 * (a[n // 2 - 1] + a[n // 2])
    p90 = a[min(n - 1, max(0, -(-9 * n // 10) - 1))]
    return {"median": round(med, 5), "min": round(a[0], 5), "p90": round(p90, 5), "n": n}


def run_decode(steps, warmup, flush=None):
    """The decode-shaped forward (split-KV split kernel + combine): per call
    milliseconds (HIP events around the whole call, median of `steps`, the
    MALL flushed before each unless flush is None) and the K/V bytes it must
    stream from HBM, as GB/s and a fraction of the 8 TB/s peak."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    d = DECODE
    q, k, v = synth.device_normal(5, [(d["B"], d["SQ"], d["HQ"], d["D"]), (d["B"], d["SK"], d["HKV"], d["D"]),
                                      (d["B"], d["SK"], d["HKV"], d["D"])])
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    call = lambda: ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)  # noqa: E731
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    st = summary(time_each(call, steps, flush))
    warm = summary(time_each(call, steps))
    kv_bytes = 2 * d["B"] * d["SK"] * d["HKV"] * d["D"] * 2
    gbps = kv_bytes / (st["median"] * 1e-3) / 1e9
    pairs = visible_pairs(d["B"], d["SQ"], d["SK"], d["HQ"], True, (-1, -1))
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    # A batched decode with enough (sequence, kv head) work tiles not to split
    # the keys: the same 4.3 GB of K/V, each tile read by one workgroup, no
    # combine kernel.
    b = DECODE_BATCHED
    q, k, v = synth.device_normal(6, [(b["B"], b["SQ"], b["HQ"], b["D"]), (b["B"], b["SK"], b["HKV"], b["D"]),
                                      (b["B"], b["SK"], b["HKV"], b["D"])])
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    call = lambda: ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)  # noqa: E731
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    st_b = summary(time_each(call, steps, flush))
    kv_b = 2 * b["B"] * b["SK"] * b["HKV"] * b["D"] * 2
    gb_b = kv_b / (st_b["median"] * 1e-3) / 1e9
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"workload": d["name"], "ms_per_call": st, "kv_bytes": kv_bytes, "kv_GBps": round(gbps, 1),
            "hbm_peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4),
            "warm_ms_per_call": warm, "warm_kv_GBps": round(kv_bytes / (warm["median"] * 1e-3) / 1e9, 1),
            "traffic": traffic_from_profile("fwd_decode"), "traffic_unit": "bytes per split-kernel launch",
            "tflops": round(4.0 * d["D"] * pairs / (st["median"] * 1e-3) / 1e12, 2),
            "batched_unsplit": {"workload": b["name"], "ms_per_call": st_b, "kv_bytes": kv_b,
                                "kv_GBps": round(gb_b, 1), "frac": round(gb_b / HBM_PEAK_GBS, 4)}}


def run_kvcache(steps, warmup, flush=None, page=256):
    """The decode shape served from a paged KV cache (attn_fwd_kvcache): every
    slot full (cache_seqlens = 32768), pages of `page` rows dealt to the slots
    in a seeded random order; time per call and K/V GB/s as run_decode."""
    import numpy as np
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    d = DECODE
    npg = d["SK"] // page
    q, k, v = synth.device_normal(5, [(d["B"], d["SQ"], d["HQ"], d["D"]), (d["B"] * npg, page, d["HKV"], d["D"]),
                                      (d["B"] * npg, page, d["HKV"], d["D"])])
    table = torch.from_numpy(np.random.default_rng(5).permutation(d["B"] * npg).astype(np.int32)
                             .reshape(d["B"], npg)).cuda()
    lens = torch.full((d["B"],), d["SK"], dtype=torch.int32, device="cuda")
    o, lse = ea.attn_fwd_kvcache(q, k, v, lens, block_table=table, causal=True)
    call = lambda: ea.attn_fwd_kvcache(q, k, v, lens, block_table=table, causal=True, out=o, lse=lse)  # noqa: E731
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    st = summary(time_each(call, steps, flush))
    kv_bytes = 2 * d["B"] * d["SK"] * d["HKV"] * d["D"] * 2
    gbps = kv_bytes / (st["median"] * 1e-3) / 1e9
    # The cache update of a decode step: the SQ new keys/values of every slot
    # written at its used length (keys rotated, rotary over all D dims) and q
    # rotated -- attn_kvcache_append + attn_rotary, timed together with events.
    kn, vn = synth.device_normal(6, [(d["B"], d["SQ"], d["HKV"], d["D"])] * 2)
    ang = torch.arange(d["SK"], device="cuda", dtype=torch.float64)[:, None] * \
        (10000.0 ** (-torch.arange(0, d["D"], 2, device="cuda", dtype=torch.float64) / d["D"]))[None, :]
    cos, sin = torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()
    lens0 = lens - d["SQ"]
    grown = torch.empty_like(lens)
    qr = torch.empty_like(q)

    def update():
        ea.attn_kvcache_append(kn, vn, k, v, lens0, block_table=table, rotary_cos=cos, rotary_sin=sin,
                               rotary_interleaved=False, seqlens_out=grown)
        ea.attn_rotary(q, lens0, cos, sin, interleaved=False, per_token=True, out=qr)
    for _ in range(warmup):
        update()
    torch.cuda.synchronize()
    upd = summary(time_each(update, steps))
    upd_bytes = 2 * (2 * kn.numel() * 2 + q.numel() * 2)  # k, v new rows and q: read once, written once
    del q, k, v, o, lse, table, kn, vn, qr
    torch.cuda.empty_cache()
    return {"workload": d["name"] + " paged KV cache (pages of %d rows, shuffled)" % page,
            "ms_per_call": st, "kv_bytes": kv_bytes, "kv_GBps": round(gbps, 1),
            "hbm_peak_GBps": HBM_PEAK_GBS, "frac": round(gbps / HBM_PEAK_GBS, 4),
            "update": {"what": "append %d new keys/values per slot (keys rotated) + rotate q; eager calls, "
                               "three small launches: launch-bound (warm)" % d["SQ"],
                       "ms": upd, "bytes": upd_bytes,
                       "GBps": round(upd_bytes / (upd["median"] * 1e-3) / 1e9, 1)}}


def run_sweep(steps, warmup):
    """Context sweep shaped like the jax-flash-attn3 README table: S = 512 ... 16384,
    B = 16384 / S, H = 16, D = 128, bf16, causal and not; forward and fwd+bwd
    TFLOP/s from the library's own kernel timing (HIP events)."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    rows = []
    for causal in (False, True):
        for S in (512, 1024, 2048, 4096, 8192, 16384):
            B, H, D = 16384 // S, 16, 128
            q, k, v, do = synth.device_normal(S, [(B, S, H, D)] * 4)
            o, lse = ea.attn_fwd(q, k, v, causal=causal)
            for _ in range(warmup):
                ea.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
                ea.attn_bwd(q, k, v, o, lse, do, causal=causal)
            torch.cuda.synchronize()
            ea.attn_timing_enable(True)
            for _ in range(steps):
                ea.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
                ea.attn_bwd(q, k, v, o, lse, do, causal=causal)
            torch.cuda.synchronize()
            t = {n: ea.attn_timing_read(n)[1] / steps for n in ea._lib.KERNELS}
            ea.attn_timing_enable(False)
            fwd_ms = t["fwd"] + t["fwd_combine"]
            bwd_ms = t["bwd_dsink"] + t["bwd_dq"] + t["bwd_dkdv"]
            pairs = visible_pairs(B, S, S, H, causal, (-1, -1))
            rows.append({"S": S, "B": B, "causal": causal, "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                         "fwd_tflops": round(4.0 * D * pairs / (fwd_ms * 1e-3) / 1e12, 1),
                         "fwdbwd_tflops": round(14.0 * D * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1)})
            print(json.dumps(rows[-1]), flush=True)
            del q, k, v, do, o, lse
    return rows


def run_headdims(steps, warmup):
    """Head-dim sweep on the causal prefill shape (B=4, H=16, S=2048, bf16):
    D = 32 ... 256.  A head dim runs on the 64-, 128- or 256-wide kernels, the
    next width up, with zero tile columns, so `tflops` counts the flops of the
    real head dim and `tile_tflops` those the MFMA pipe executes at the tile
    width."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    B, S, H = 4, 2048, 16
    pairs = visible_pairs(B, S, S, H, True, (-1, -1))
    rows = []
    for D in (32, 48, 64, 80, 96, 112, 128, 160, 192, 224, 256):
        q, k, v, do = synth.device_normal(D, [(B, S, H, D)] * 4)
        o, lse = ea.attn_fwd(q, k, v, causal=True)
        for _ in range(warmup):
            ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
            ea.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        ea.attn_timing_enable(True)
        for _ in range(steps):
            ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
            ea.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        t = {n: ea.attn_timing_read(n)[1] / steps for n in ea._lib.KERNELS}
        ea.attn_timing_enable(False)
        fwd_ms = t["fwd"] + t["fwd_combine"]
        bwd_ms = t["bwd_dsink"] + t["bwd_dq"] + t["bwd_dkdv"]
        tile = 64 if D <= 64 else 128 if D <= 128 else 256
        rows.append({"D": D, "tile_D": tile, "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                     "fwd_tflops": round(4.0 * D * pairs / (fwd_ms * 1e-3) / 1e12, 1),
                     "tflops": round(14.0 * D * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1),
                     "tile_tflops": round(14.0 * tile * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1)})
        print(json.dumps(rows[-1]), flush=True)
        del q, k, v, do, o, lse
    return rows


def run_variants(steps, warmup):
    """Score variants on the causal prefill shape (B=4, H=16, S=2048, D=128,
    bf16): plain, soft cap 50, ALiBi (geometric slopes), both, and 4 sinks per
    head; forward and backward ms and TFLOP/s (14*D flops per visible pair)."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    B, S, H, D = 4, 2048, 16, 128
    pairs = visible_pairs(B, S, S, H, True, (-1, -1))
    q, k, v, do = synth.device_normal(11, [(B, S, H, D)] * 4)
    slopes = torch.from_numpy(synth.alibi_slopes(H)).cuda()
    sinks4 = torch.from_numpy(synth.sink_table(11, H, 4)).cuda()
    rows = []
    for name, kw in (("plain", {}), ("softcap50", dict(softcap=50.0)), ("alibi", dict(alibi_slopes=slopes)),
                     ("softcap50_alibi", dict(softcap=50.0, alibi_slopes=slopes)), ("sinks4", dict(sinks=sinks4))):
        o, lse = ea.attn_fwd(q, k, v, causal=True, **kw)
        for _ in range(warmup):
            ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse, **kw)
            ea.attn_bwd(q, k, v, o, lse, do, causal=True, **kw)
        torch.cuda.synchronize()
        ea.attn_timing_enable(True)
        for _ in range(steps):
            ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse, **kw)
            ea.attn_bwd(q, k, v, o, lse, do, causal=True, **kw)
        torch.cuda.synchronize()
        t = {n: ea.attn_timing_read(n)[1] / steps for n in ea._lib.KERNELS}
        ea.attn_timing_enable(False)
        fwd_ms = t["fwd"] + t["fwd_combine"]
        bwd_ms = t["bwd_dsink"] + t["bwd_dq"] + t["bwd_dkdv"]
        rows.append({"variant": name, "fwd_ms": round(fwd_ms, 4), "bwd_dq_ms": round(t["bwd_dq"], 4),
                     "bwd_dkdv_ms": round(t["bwd_dkdv"], 4), "bwd_ms": round(bwd_ms, 4),
                     "fwd_tflops": round(4.0 * D * pairs / (fwd_ms * 1e-3) / 1e12, 1),
                     "tflops": round(14.0 * D * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 1)})
        print(json.dumps(rows[-1]), flush=True)
    return rows


def run_stream(steps, warmup):
    """Practical HBM read rates on this machine for the decode shape's bytes
    (4.295 GB: the K and V of the decode shape), each repetition after the
    MALL flush, timed with HIP events.  First the read probes of
    libattn36_probe.so, which read K and V [32, 32768, 8, 128] in the split-KV
    forward's order (workgroup = sequence, kv head and split, 64-key tiles)
    with no arithmetic: global -> LDS DMA in a two-deep ring with the default
    cache policy and with the non-temporal hint, and plain 16-byte register
    loads with the hint.  Then torch's own streaming kernels over the same
    bytes: a sum (reads only), a copy (read + write) and an add (two reads,
    one write).  References for the decode's K/V rate, not kernels of the
    attention library."""
    import ctypes
    import torch
    d = DECODE
    flush = Flusher()
    rows = []

    def emit(name, fn, nbytes):
        for _ in range(warmup):
            fn()
        st = summary(time_each(fn, steps, flush))
        rows.append({"stream": name, "bytes": nbytes, "ms": st,
                     "GBps": round(nbytes / (st["median"] * 1e-3) / 1e9, 1),
                     "frac_of_8TBps": round(nbytes / (st["median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        print(json.dumps(rows[-1]), flush=True)

    probe_path = os.path.join(ROOT, "exact_attention_36_amd", "libattn36_probe.so")
    if not os.path.exists(probe_path):
        raise SystemExit("libattn36_probe.so is not built: run __graft_entry__.build() first")
    probe = ctypes.CDLL(probe_path)
    shape = (d["B"], d["SK"], d["HKV"], d["D"])
    k = torch.empty(shape, dtype=torch.bfloat16, device="cuda").normal_()
    v = torch.empty(shape, dtype=torch.bfloat16, device="cuda").normal_()
    kv_bytes = 2 * k.numel() * 2
    ns = 2  # the split count the attention forward picks for this shape
    sink = torch.empty(d["B"] * d["HKV"] * ns * 256 * 4, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def call(rc):
        if rc != 0:
            raise RuntimeError("read probe failed with code %d" % rc)

    for name, fn in (
            ("probe: DMA to LDS, default policy (K/V read)",
             lambda: call(probe.probe_read_dma(ptr(k), ptr(v), d["B"], d["SK"], d["HKV"], ns, 0, ptr(sink), stream))),
            ("probe: DMA to LDS, non-temporal (K/V read)",
             lambda: call(probe.probe_read_dma(ptr(k), ptr(v), d["B"], d["SK"], d["HKV"], ns, 1, ptr(sink), stream))),
            ("probe: register loads, non-temporal (K/V read)",
             lambda: call(probe.probe_read_regs(ptr(k), ptr(v), d["B"], d["SK"], d["HKV"], ns, ptr(sink), stream)))):
        emit(name, fn, kv_bytes)
    del k, v, sink
    torch.cuda.empty_cache()

    n = 2 * d["B"] * d["SK"] * d["HKV"] * d["D"]  # elements of K and V, bf16
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    emit("torch sum (read)", lambda: x.sum(dtype=torch.float32), 2 * n)
    y = torch.empty_like(x)
    emit("torch copy (read + write)", lambda: y.copy_(x), 4 * n)
    del y
    a, b = x[: n // 2], x[n // 2:]
    z = torch.empty_like(a)
    emit("torch add (2 reads + write)", lambda: torch.add(a, b, out=z), 6 * n // 2)
    del z, x
    torch.cuda.empty_cache()
    return rows


def run_flush_check(steps, warmup):
    """What the MALL flush does to the timed call after it.  Three callers:
    a decode-shaped forward over 67 MB of K/V (s_kv = 512: it fits in the
    256 MB MALL, so it runs faster warm), the full decode shape (4.3 GB of
    K/V, far larger than the MALL) and the causal prefill forward; each timed
    with no flush (warm), after the 512 MB read flush and after a 512 MB
    write.  A flush that evicts shows as the small decode slowing down; one
    that leaves write-backs behind shows as the large decode slowing down.
    In every mode a spin kernel runs just before the call (see below)."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    d = DECODE
    flushes = {"none": None, "read": Flusher(), "write": WriteFlusher()}
    w = WORKLOAD
    shapes = [("decode B32 s_q16 s_kv512 Hq64 Hkv8 D128 (K/V 67 MB)", d["B"], d["SQ"], 512, d["HQ"], d["HKV"]),
              ("decode B32 s_q16 s_kv32768 Hq64 Hkv8 D128 (K/V 4.3 GB)", d["B"], d["SQ"], d["SK"], d["HQ"], d["HKV"]),
              ("causal prefill fwd B4 H16 S2048 D128", w["B"], w["S"], w["S"], w["HQ"], w["HKV"])]
    for name, B, sq, sk, hq, hkv in shapes:
        q, k, v = synth.device_normal(5, [(B, sq, hq, d["D"]), (B, sk, hkv, d["D"]), (B, sk, hkv, d["D"])])
        o, lse = ea.attn_fwd(q, k, v, causal=True)
        call = lambda: ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)  # noqa: E731
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        res = {}
        for _ in range(2):  # two alternations; the second is reported
            for fname, f in flushes.items():
                # a spin kernel after the flush (or alone) keeps the GPU busy
                # while the host queues the call, so that no mode is timed
                # with the host's launch latency in it
                def pre(f=f):
                    if f is not None:
                        f()
                    torch.cuda._sleep(SPIN_CYCLES)
                res[fname] = summary(time_each(call, steps, pre))
        print(json.dumps({"workload": "flush check", "caller": name, "kv_bytes": 2 * k.numel() * 2,
                          "ms_per_call": res}), flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()


def run_latency(steps, warmup):
    """Launch-bound shape (B=1, H=2, S=128, D=64, bf16, non-causal forward):
    µs per call issued eagerly through the binding, per call of a HIP graph
    that holds 20 calls (torch.cuda.graph; the library allocates nothing and
    never synchronises, so it captures as is), and per replay of a graph that
    holds one call (the graph launch's own cost)."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    q, k, v = synth.device_normal(1, [(1, 128, 2, 64)] * 3)
    o, lse = ea.attn_fwd(q, k, v)
    n = max(steps, 100) * 10
    for _ in range(warmup * 10):
        ea.attn_fwd(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        ea.attn_fwd(q, k, v, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ea.attn_fwd(q, k, v, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    def graph_of(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                ea.attn_fwd(q, k, v, out=o, lse=lse)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        reps = n // calls
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * calls)
    graph20_us = graph_of(20)
    graph1_us = graph_of(1)
    row = {"workload": "fwd B1 H2 S128 D64 bf16 non-causal", "calls": n, "eager_us_per_call": round(eager_us, 2),
           "graph20_us_per_call": round(graph20_us, 2), "graph1_us_per_replay": round(graph1_us, 2)}
    print(json.dumps(row), flush=True)
    return row


def compulsory_bytes(qt, kvt, rows, bwd):
    """HBM bytes a pass must move, each tensor once: forward Q K V in, O and
    the fp32 LSE out; backward Q K V O dO and LSE in, dQ dK dV out."""
    return (4 * qt + 4 * kvt + 4 * rows) if bwd else (2 * qt + 2 * kvt + 4 * rows)


def roof(flop, nbytes, st):
    """Rates of one timed pass (`st` from summary()) against the MFMA and HBM
    rooflines: the attainable time is max(flop / 2.5 PFLOP/s, bytes / 8 TB/s)."""
    ms = st["median"]
    t_mfma = flop / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms": st, "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_bytes": int(nbytes), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "attainable_ms": round(max(t_mfma, t_hbm), 5), "frac_of_attainable": round(max(t_mfma, t_hbm) / ms, 4)}


def config3_inputs():
    """GQA 32/8, S = 8192, B = 2, window (127, 0), fp32 sinks [32]."""
    import numpy as np
    import torch
    from exact_attention_36_amd import synth
    q, k, v, do = synth.device_normal(3, [(2, 8192, 32, 128), (2, 8192, 8, 128), (2, 8192, 8, 128), (2, 8192, 32, 128)])
    sinks = torch.from_numpy(np.random.default_rng(3).standard_normal(32).astype(np.float32)).cuda()
    return q, k, v, do, sinks


def config4_inputs():
    """Packed batch: 64 sequence lengths of the packed-workload recipe (seed 4,
    the same lengths as the parity tests), tensors drawn on the device."""
    import numpy as np
    import torch
    from exact_attention_36_amd import synth
    L = synth.packed_lengths(np.random.default_rng(4))
    cu = synth.cu_seqlens(L)
    T = int(cu[-1])
    q, k, v, do = synth.device_normal(4, [(T, 16, 128), (T, 4, 128), (T, 4, 128), (T, 16, 128)])
    return q, k, v, do, torch.from_numpy(cu).cuda(), L


def run_config_lines(steps, warmup, flush):
    """Configs 1, 3 and 4 (config 2 is the headline step, config 5 the decode
    line): forward and backward each timed `steps` times (MALL flushed before
    each), median / min / p90 and rates against the rooflines."""
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    out = {}

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        return summary(time_each(fn, steps, flush))

    q, k, v = synth.device_normal(1, [(1, 128, 2, 64)] * 3)
    o, lse = ea.attn_fwd(q, k, v)
    st = timed(lambda: ea.attn_fwd(q, k, v, out=o, lse=lse))
    out["config1"] = {"workload": "fwd B1 H2 S128 D64 bf16 non-causal (launch-bound: µs per eager call)",
                      "us_per_call": {k_: (round(v_ * 1e3, 2) if k_ != "n" else v_) for k_, v_ in st.items()}}
    del q, k, v, o, lse

    q, k, v, do, sinks = config3_inputs()
    kw = dict(causal=True, window=(127, 0), sinks=sinks)
    o, lse = ea.attn_fwd(q, k, v, **kw)
    pairs = visible_pairs(2, 8192, 8192, 32, True, (127, 0))
    qt, kvt, rows = q.numel() * 2, k.numel() * 2, 2 * 32 * 8192
    sf = timed(lambda: ea.attn_fwd(q, k, v, out=o, lse=lse, **kw))
    sb = timed(lambda: ea.attn_bwd(q, k, v, o, lse, do, **kw))
    out["config3"] = {"workload": "GQA 32/8 causal window (127,0) sinks B2 S8192 D128 bf16 fwd+bwd",
                      "fwd": roof(4.0 * 128 * pairs, compulsory_bytes(qt, kvt, rows, False), sf),
                      "bwd": roof(10.0 * 128 * pairs, compulsory_bytes(qt, kvt, rows, True), sb)}
    del q, k, v, do, sinks, o, lse
    torch.cuda.empty_cache()

    q, k, v, do, cu, L = config4_inputs()
    mx = int(L.max())
    o, lse = ea.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True)
    pairs = 16 * sum(int(x) * (int(x) + 1) // 2 for x in L)
    qt, kvt, rows = q.numel() * 2, k.numel() * 2, 16 * q.shape[0]
    sf = timed(lambda: ea.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True, out=o, lse=lse))
    sb = timed(lambda: ea.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, causal=True))
    out["config4"] = {"workload": "packed 65536 tokens in 64 sequences (8 empty) GQA 16/4 D128 bf16 causal fwd+bwd",
                      "fwd": roof(4.0 * 128 * pairs, compulsory_bytes(qt, kvt, rows, False), sf),
                      "bwd": roof(10.0 * 128 * pairs, compulsory_bytes(qt, kvt, rows, True), sb)}
    del q, k, v, do, o, lse
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _max_err(got, ref):
    import numpy as np
    e = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(e.max()), float(e.mean())


def cpu_baseline(inp, w, gpu_out, seconds_target=10.0):
    """The fp64 oracle (unchanged) on the host's cores.

    Headline: whole (batch, head) slices of the benchmarked workload, forward
    and backward, for about `seconds_target` seconds, as TFLOP/s (14 * D flops
    per visible pair, the GPU's convention); the same slices of the GPU's own
    outputs from the timed steps are compared with them (max-abs and mean-abs
    errors of O, dQ, dK, dV, LSE).  Per other config: a seeded sample of query
    rows (their O, LSE, D and dQ), with seconds, rows/s and visible pairs/s,
    and the full-config fwd+bwd time extrapolated from that rate (rows plus
    key columns: two passes over the visible pairs)."""
    import numpy as np
    import oracle
    from exact_attention_36_amd import synth
    D, S = w["D"], w["S"]
    scale = synth.default_scale(D)
    host = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    go = {n: host(t) for n, t in gpu_out.items()}
    done_pairs, t_used, slices, worst = 0, 0.0, 0, {}
    for b in range(w["B"]):
        for h in range(w["HQ"]):
            sl = lambda a, hh=h: np.ascontiguousarray(a[b:b + 1, :, hh:hh + 1, :])  # noqa: E731
            p = oracle.batched(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), scale, causal=w["causal"],
                               window=w["window"], dout=sl(inp["dout"]))
            t0 = time.perf_counter()
            ref = oracle.full(p, grads=True)
            t_used += time.perf_counter() - t0
            done_pairs += visible_pairs(1, S, S, 1, w["causal"], w["window"])
            slices += 1
            for name, got, r in (("o", go["o"][b, :, h], ref["o"][:, 0]), ("dq", go["dq"][b, :, h], ref["dq"][:, 0]),
                                 ("dk", go["dk"][b, :, h], ref["dk"][:, 0]), ("dv", go["dv"][b, :, h], ref["dv"][:, 0]),
                                 ("lse", go["lse"][b, h], ref["lse"][0])):
                mx, mn = _max_err(got, r)
                m0 = worst.get(name, (0.0, 0.0))
                worst[name] = (max(m0[0], mx), max(m0[1], mn))
            if t_used >= seconds_target:
                break
        if t_used >= seconds_target:
            break
    flops = 14.0 * D * done_pairs
    ok = all(worst[n][0] <= (1e-3 if n == "lse" else 2e-2 + 2 ** -5) and (n == "lse" or worst[n][1] <= 2e-3)
             for n in worst)
    res = {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": "%d full (batch, head) slices of the %dx%d causal workload, fwd+bwd (O, LSE, dQ, dK, dV), "
                     "%.1f s" % (slices, S, S, t_used),
           "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
           "threads_used": oracle.num_threads(),
           "full_config_seconds_extrapolated": round(14.0 * D * visible_pairs(w["B"], S, S, w["HQ"], w["causal"],
                                                                              w["window"]) / (flops / t_used), 1),
           "gpu_output_check": {"slices": slices, "max_abs": {n: float("%.3g" % v[0]) for n, v in worst.items()},
                                "mean_abs": {n: float("%.3g" % v[1]) for n, v in worst.items()},
                                "within_tolerance": bool(ok),
                                "tolerance": "max-abs 2e-2 (+ half a bf16 ulp, at most 2^-5, for |x| >= 4), "
                                             "mean-abs 2e-3, LSE 1e-3"}}
    res["configs"] = oracle_config_rates()
    return res


def oracle_config_rates(rows_per_config=192, seed=1000):
    """Seeded samples of query rows of configs 1, 3, 4 and 5 through the oracle
    (forward and backward row quantities), with the rate and the full-config
    fwd+bwd time extrapolated from it."""
    import numpy as np
    import torch
    import oracle
    from exact_attention_36_amd import synth
    rng = np.random.default_rng(seed)
    res = {}

    def sample(name, p, seq_pool, hq, lq_of, full_pairs, vis_of):
        n = rows_per_config
        seqs = rng.choice(np.asarray(seq_pool), n)
        heads = rng.integers(0, hq, n)
        rows = np.array([rng.integers(0, max(1, lq_of(s_))) for s_ in seqs])
        pairs = sum(vis_of(int(s_), int(r_)) for s_, r_ in zip(seqs, rows))
        t0 = time.perf_counter()
        oracle.rows(p, seqs, heads, rows, grads=True)
        dt = time.perf_counter() - t0
        rate = pairs / dt
        res[name] = {"rows": n, "seconds": round(dt, 3), "rows_per_s": round(n / dt, 1),
                     "visible_pairs_per_s": round(rate, 1),
                     "full_fwd_bwd_seconds_extrapolated": round(2.0 * full_pairs / rate, 1)}

    hb = synth.host_bits
    # config 1: everything, timed as a whole
    inp = synth.batched_inputs(1, 1, 128, 128, 2, 2, 64, grads=True)
    p = oracle.batched(inp["q"], inp["k"], inp["v"], synth.default_scale(64), dout=inp["dout"])
    t0 = time.perf_counter()
    oracle.full(p)
    dt = time.perf_counter() - t0
    res["config1"] = {"rows": 256, "seconds": round(dt, 4), "full_fwd_bwd_seconds": round(dt, 4)}
    # config 3: batch entry 0 (its rows see 128 keys)
    q, k, v, do, sinks = config3_inputs()
    p = oracle.batched(hb(q[:1]), hb(k[:1]), hb(v[:1]), synth.default_scale(128), causal=True, window=(127, 0),
                       dout=hb(do[:1]), sinks=sinks.cpu().numpy())
    sample("config3", p, [0], 32, lambda s_: 8192, visible_pairs(2, 8192, 8192, 32, True, (127, 0)),
           lambda s_, r_: min(r_ + 1, 128))
    del q, k, v, do, sinks
    # config 4: the packed batch
    q, k, v, do, cu, L = config4_inputs()
    cuh = cu.cpu().numpy()
    p = oracle.varlen(hb(q), hb(k), hb(v), cuh, cuh, synth.default_scale(128), causal=True, dout=hb(do))
    live = np.flatnonzero(L > 0)
    sample("config4", p, live, 16, lambda s_: int(L[s_]), 16 * sum(int(x) * (int(x) + 1) // 2 for x in L),
           lambda s_, r_: (r_ + 1) if L[s_] > 0 else 0)
    del q, k, v, do, cu, live
    torch.cuda.empty_cache()
    # config 5: batch entry 0 of the decode shape
    d = DECODE
    q, k, v = synth.device_normal(5, [(d["B"], d["SQ"], d["HQ"], d["D"]), (d["B"], d["SK"], d["HKV"], d["D"]),
                                      (d["B"], d["SK"], d["HKV"], d["D"])])
    dout = synth.device_normal(55, [(1, d["SQ"], d["HQ"], d["D"])])[0]
    p = oracle.batched(hb(q[:1]), hb(k[:1]), hb(v[:1]), synth.default_scale(128), causal=True, dout=hb(dout))
    sample("config5", p, [0], d["HQ"], lambda s_: d["SQ"], visible_pairs(d["B"], d["SQ"], d["SK"], d["HQ"], True, (-1, -1)),
           lambda s_, r_: d["SK"] - d["SQ"] + r_ + 1)
    del q, k, v, dout
    torch.cuda.empty_cache()
    return res


def read_power_clock():
    """One `amd-smi metric -p -c` reading: socket power (W) and the mean of the
    per-XCD shader clocks (MHz), or None where the tool is missing."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    clks = [float(m) for m in re.findall(r"^\s*CLK:\s*([0-9.]+)\s*MHz", txt, re.M)]
    # the GFX_i blocks come first; other clock domains follow under their own names
    gfx = []
    for block in re.split(r"\n\s*(?=GFX_\d+:|MEM_\d+:|VCLK_\d+:|DCLK_\d+:|[A-Z]+_\d+:)", txt):
        if block.strip().startswith("GFX_"):
            m = re.search(r"^\s*CLK:\s*([0-9.]+)\s*MHz", block, re.M)
            if m:
                gfx.append(float(m.group(1)))
    if not pw or not (gfx or clks):
        return None
    return float(pw.group(1)), sum(gfx) / len(gfx) if gfx else None


def run_configs(steps, warmup, only=None):
    """Kernel times of the five parity workloads, one JSON line each, from the
    library's HIP-event timing: the tiny non-causal forward (B=1, H=2, S=128,
    D=64), causal prefill (B=4, H=16, S=2048), GQA 32/8 with window (127, 0)
    and sinks (B=2, S=8192), the packed batch (65536 tokens in 64 sequences,
    GQA 16/4, causal) and the decode shape (B=32, s_q=16, s_kv=32768, GQA
    64/8).  TFLOP/s count 4·D flops per visible pair forward, 10·D backward."""
    import numpy as np
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    names = list(ea._lib.KERNELS)

    def timed(fn, reps):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ea.attn_timing_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        r = {n: ea.attn_timing_read(n) for n in names}
        ea.attn_timing_enable(False)
        return {n: (ms / reps) for n, (c, ms) in r.items()}

    def line(name, D, pairs, tf, tb=None, kv_bytes=None):
        # packed calls may first build their grids' schedule tables ("order")
        f = tf["fwd"] + tf["fwd_combine"] + tf.get("order", 0.0)
        r = {"workload": name, "fwd_ms": round(f, 4), "fwd_tflops": round(4.0 * D * pairs / (f * 1e-3) / 1e12, 1)}
        if kv_bytes:
            r["kv_GBps"] = round(kv_bytes / (f * 1e-3) / 1e9, 1)
        if tb:
            b = tb["bwd_dsink"] + tb["bwd_dq"] + tb["bwd_dkdv"] + tb.get("order", 0.0)
            r.update(bwd_ms=round(b, 4), dq_ms=round(tb["bwd_dq"], 4), dkdv_ms=round(tb["bwd_dkdv"], 4),
                     dsink_ms=round(tb["bwd_dsink"], 4), order_ms=round(tf.get("order", 0.0) + tb.get("order", 0.0), 4),
                     bwd_tflops=round(10.0 * D * pairs / (b * 1e-3) / 1e12, 1),
                     fwdbwd_tflops=round(14.0 * D * pairs / ((f + b) * 1e-3) / 1e12, 1))
        print(json.dumps(r), flush=True)

    batched = [
        ("fwd B1 H2 S128 D64 non-causal", 1, 128, 128, 2, 2, 64, False, (-1, -1), False, False),
        ("causal prefill B4 H16 S2048 D128", 4, 2048, 2048, 16, 16, 128, True, (-1, -1), False, True),
        ("GQA 32/8 window (127,0) sinks B2 S8192 D128", 2, 8192, 8192, 32, 8, 128, True, (127, 0), True, True),
        ("decode B32 s_q16 s_kv32768 GQA 64/8 D128 causal", 32, 16, 32768, 64, 8, 128, True, (-1, -1), False, False),
    ]
    for cfg, (name, B, sq, sk, hq, hkv, D, causal, win, sinks, bwd) in zip((1, 2, 3, 5), batched):
        if only is not None and cfg != only:
            continue
        q, k, v, do = synth.device_normal(sq + hq, [(B, sq, hq, D), (B, sk, hkv, D), (B, sk, hkv, D), (B, sq, hq, D)])
        s = torch.from_numpy(np.random.default_rng(3).standard_normal(hq).astype(np.float32)).cuda() if sinks else None
        o, lse = ea.attn_fwd(q, k, v, causal=causal, window=win, sinks=s)
        tf = timed(lambda: ea.attn_fwd(q, k, v, causal=causal, window=win, sinks=s, out=o, lse=lse), steps)
        tb = timed(lambda: ea.attn_bwd(q, k, v, o, lse, do, causal=causal, window=win, sinks=s), steps) if bwd else None
        kv = 2 * B * sk * hkv * D * 2 if sq < 64 else None
        line(name, D, visible_pairs(B, sq, sk, hq, causal, win), tf, tb, kv)
        del q, k, v, do, o, lse
    if only is not None and only != 4:
        return
    w = synth.packed_workload(seed=4)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    q, k, v, do = (dev(w[n]) for n in ("q", "k", "v", "dout"))
    cu = torch.from_numpy(w["cu_q"]).cuda()
    mx = int(w["lengths"].max())
    o, lse = ea.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True)
    tf = timed(lambda: ea.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True, out=o, lse=lse), steps)
    tb = timed(lambda: ea.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, causal=True), steps)
    pairs = 16 * sum(int(L) * (int(L) + 1) // 2 for L in w["lengths"])
    line("packed 65536 tokens 64 seqs GQA 16/4 D128 causal", 128, pairs, tf, tb)


def run_power(seconds):
    """Socket power and shader clock while the workload's forward, backward
    and whole step each run back to back for `seconds` (sampled after the
    first 2 s), next to each phase's call rate."""
    import threading
    import numpy as np
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth
    w = WORKLOAD
    inp = synth.batched_inputs(2, w["B"], w["S"], w["S"], w["HQ"], w["HKV"], w["D"], grads=True)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    o, lse = ea.attn_fwd(q, k, v, causal=w["causal"], window=w["window"])
    phases = {
        "fwd": lambda: ea.attn_fwd(q, k, v, causal=w["causal"], window=w["window"], out=o, lse=lse),
        "bwd": lambda: ea.attn_bwd(q, k, v, o, lse, do, causal=w["causal"], window=w["window"]),
        "step": lambda: (ea.attn_fwd(q, k, v, causal=w["causal"], window=w["window"], out=o, lse=lse),
                         ea.attn_bwd(q, k, v, o, lse, do, causal=w["causal"], window=w["window"])),
    }
    res = []
    for name, fn in phases.items():
        samples, stop = [], threading.Event()

        def sampler():
            if stop.wait(2.0):
                return
            while not stop.is_set():
                r = read_power_clock()
                if r:
                    samples.append(r)
                stop.wait(0.5)

        th = threading.Thread(target=sampler)
        th.start()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            n += 20
        dt = time.perf_counter() - t0
        stop.set()
        th.join()
        pw = [s[0] for s in samples]
        ck = [s[1] for s in samples if s[1] is not None]
        res.append({"phase": name, "calls": n, "ms_per_call": round(dt / n * 1e3, 4),
                    "socket_power_w": round(sum(pw) / len(pw), 1) if pw else None,
                    "gfx_clock_mhz": round(sum(ck) / len(ck), 1) if ck else None, "samples": len(samples)})
        print(json.dumps(res[-1]), flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the other workloads (configs 1, 3, 4 and the decode shape)")
    ap.add_argument("--workload", choices=("step", "decode", "sweep", "headdims", "variants", "latency", "power", "configs",
                                           "stream", "flush"), default="step",
                    help="step: the fwd+bwd line (default, also measures the decode shape); "
                         "decode: only the decode-shaped forward (for profiling it alone); "
                         "sweep: context sweep over S = 512..16384 (one JSON line per shape); configs: kernel times of the five "
                         "parity workloads; "
                         "headdims: causal prefill at D = 32..256 (one JSON line per head dim); "
                         "variants: causal prefill with soft cap / ALiBi / 4 sinks (one line each); "
                         "latency: launch-bound forward, eager calls vs HIP graph replays; "
                         "power: socket power and shader clock (amd-smi) under the step's kernels; "
                         "stream: read probes in the decode's access order and torch's sum / copy / add over the decode "
                         "shape's 4.3 GB (practical HBM rates); "
                         "flush: calls timed warm, after the read flush and after a 512 MB write")
    ap.add_argument("--seconds", type=float, default=10.0, help="duration of each --workload power phase")
    ap.add_argument("--config", type=int, choices=(1, 2, 3, 4, 5), default=None,
                    help="with --workload configs: run only this workload (1..5 in the order listed there)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 256 MiB elementwise copy first (reference for HBM counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the attention kernels run on a single device and this "
              "library has no multi-GPU path (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import exact_attention_36_amd as ea
    from exact_attention_36_amd import synth

    if args.workload == "sweep":
        run_sweep(args.steps, args.warmup)
        return
    if args.workload == "headdims":
        run_headdims(args.steps, args.warmup)
        return
    if args.workload == "variants":
        run_variants(args.steps, args.warmup)
        return
    if args.workload == "latency":
        run_latency(args.steps, args.warmup)
        return
    if args.workload == "configs":
        if args.copy_calibration:
            copy_calibration()
        run_configs(args.steps, args.warmup, args.config)
        return
    if args.workload == "power":
        run_power(args.seconds)
        return
    if args.workload == "stream":
        run_stream(args.steps, args.warmup)
        return
    if args.workload == "flush":
        run_flush_check(args.steps, args.warmup)
        return
    if args.workload == "decode":
        if args.copy_calibration:
            copy_calibration()
        flush = Flusher()
        dec = run_decode(args.steps, args.warmup, flush)
        dec["paged"] = run_kvcache(args.steps, args.warmup, flush)
        print(json.dumps({"metric": "decode-shaped forward, K/V HBM GB/s, 1 MI355X", "value": dec["kv_GBps"],
                          "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": dec["ms_per_call"]["median"], "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded N(0,1) rounded to bf16",
                          "config": {"workload": dec["workload"]}, "decode": dec}))
        return

    w = WORKLOAD
    B, S, HQ, HKV, D = w["B"], w["S"], w["HQ"], w["HKV"], w["D"]
    inp = synth.batched_inputs(2, B, S, S, HQ, HKV, D, grads=True)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration()
    flush = Flusher()
    last = {}

    def step():
        o, lse = ea.attn_fwd(q, k, v, causal=w["causal"], window=w["window"])
        dq, dk, dv, _ = ea.attn_bwd(q, k, v, o, lse, do, causal=w["causal"], window=w["window"])
        last.update(o=o, lse=lse, dq=dq, dk=dk, dv=dv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Per-kernel breakdown, from a pass of its own (MALL flushed before each
    # step) with every launch bracketed by HIP events; the events inflate the
    # kernels a little, so their sum is reported beside the same pass's step
    # time.  The timed region below brackets only the dominant kernel.
    ea.attn_timing_enable(True)
    bd_steps = summary(time_each(step, args.steps, flush))
    kern = {}
    for name in ea._lib.KERNELS:
        n, tot = ea.attn_timing_read(name)
        if n:
            kern[name] = (n, tot)
    ea.attn_timing_enable(False)
    dom = max(kern, key=lambda n: kern[n][1])  # dominant kernel: most total time

    # Timed region: exactly K steps, the MALL flushed before each (outside the
    # step's events), the dominant kernel's launches timed live with HIP events
    # on the library's stream (the step's own stream).
    ea.attn_timing_enable(True, kernels=[dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold = time_each(step, args.steps, flush)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_l, tot = ea.attn_timing_read(dom)
    ea.attn_timing_enable(False)
    avg_ms = tot / n_l
    st = summary(cold)
    ms = st["median"]
    warm = summary(time_each(step, args.steps))
    fwd_only = summary(time_each(lambda: ea.attn_fwd(q, k, v, causal=w["causal"], window=w["window"]),
                                 args.steps, flush))

    pairs = visible_pairs(B, S, S, HQ, w["causal"], w["window"])
    fwd_flop, bwd_flop = 4.0 * D * pairs, 10.0 * D * pairs
    tflops = (fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12
    # MFMA work each kernel is built to do: the forward 2 products per visible
    # pair, the key-major dK/dV kernel 4 (S, dP, dV, dK), the query-major dQ
    # kernel 3 (S, dP, dQ); the step's value keeps the 4:10 convention.
    flop_of = {"fwd": fwd_flop, "bwd_dkdv": 8.0 * D * pairs, "bwd_dq": 6.0 * D * pairs}
    # compulsory HBM bytes per launch (each tensor read or written once)
    qt, kvt, rows = B * S * HQ * D * 2, B * S * HKV * D * 2, B * HQ * S
    algo_bytes = {"fwd": 2 * qt + 2 * kvt + 4 * rows,              # Q K V in, O and lse out
                  "bwd_dq": 4 * qt + 2 * kvt + 12 * rows,          # Q O dO K V, lse in; dQ, D, lse' out
                  "bwd_dkdv": 2 * qt + 4 * kvt + 8 * rows}         # Q dO K V, D, lse' in; dK dV out
    roof_ = None
    if dom in flop_of:
        ach = flop_of[dom] / (avg_ms * 1e-3) / 1e12
        roof_ = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                 "traffic": traffic_from_profile(dom), "traffic_unit": "bytes per launch",
                 "algorithmic_bytes": algo_bytes[dom], "avg_launch_ms": round(avg_ms, 5)}
    kms = {n: round(t / args.steps, 5) for n, (c, t) in kern.items()}
    fwd_tf = fwd_flop / (fwd_only["median"] * 1e-3) / 1e12
    out = {
        "metric": "attention fwd+bwd TFLOPS (and % of MFMA bf16 peak), 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) q, k, v, dout rounded to bf16",
        "config": {"workload": w["name"], "batch": B, "seq_len": S, "heads_q": HQ, "heads_kv": HKV,
                   "head_dim": D, "causal": w["causal"], "parallelism": "single GPU"},
        "timing": "per-step HIP events, MALL (512 MB) flushed before each step outside its events; value and "
                  "ms_per_step use the median over the K timed steps",
        "ms_per_step_stats": st,
        "warm": {"what": "the same steps without the flush (K/V may hit the 256 MB MALL)", "ms_per_step": warm,
                 "value": round((fwd_flop + bwd_flop) / (warm["median"] * 1e-3) / 1e12, 2)},
        "pct_mfma_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "fwd": {"ms": fwd_only, "tflops": round(fwd_tf, 2), "frac_of_mfma_peak": round(fwd_tf / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels_ms_per_step": kms,
        "kernels_breakdown": {"what": "a pass of its own with every launch bracketed by HIP events (they add a few "
                                      "µs per launch); kernel means beside that pass's median step",
                              "kernels_sum_ms": round(sum(kms.values()), 5), "step_ms": bd_steps},
        "roofline": roof_,
        "wall_s": round(wall, 3),
    }
    if not args.no_decode:
        out["config_lines"] = run_config_lines(args.steps, 2, flush)
        out["decode"] = run_decode(args.steps, 2, flush)
        out["decode"]["paged"] = run_kvcache(args.steps, 2, flush)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, last)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
