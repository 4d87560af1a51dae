"""Host-side logic of bench.py, on the CPU: the visible-pair count that turns
kernel times into TFLOP/s, the counter-summary reader behind the roofline's
`traffic` field (its value only while the kernel sources match the hash the
counters were taken with), and the refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs_brute(B, sq, sk, hq, causal, window):
    n = 0
    for i in range(sq):
        diag = i + sk - sq  # bottom-right alignment
        for j in range(sk):
            ok = (not causal or j <= diag) and (window[0] < 0 or j >= diag - window[0]) and \
                 (window[1] < 0 or j <= diag + window[1])
            n += ok
    return n * B * hq


@pytest.mark.parametrize("sq,sk,causal,window", [
    (7, 7, False, (-1, -1)), (7, 7, True, (-1, -1)), (5, 11, True, (-1, -1)), (11, 5, True, (-1, -1)),
    (9, 9, True, (3, 0)), (9, 13, False, (2, 4)), (13, 9, False, (0, 0)), (6, 6, True, (0, -1)),
])
def test_visible_pairs_matches_brute_force(sq, sk, causal, window):
    assert bench.visible_pairs(2, sq, sk, 3, causal, window) == _pairs_brute(2, sq, sk, 3, causal, window)


def test_visible_pairs_closed_forms():
    S = 2048
    assert bench.visible_pairs(4, S, S, 16, True, (-1, -1)) == 4 * 16 * S * (S + 1) // 2
    assert bench.visible_pairs(1, S, S, 1, False, (-1, -1)) == S * S


def _fake_root(tmp_path):
    for p in set(sum(bench.KERNEL_SOURCES.values(), [])) | set(bench.COMMON_SOURCES):
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def test_traffic_only_while_sources_match(tmp_path, monkeypatch):
    root = _fake_root(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.traffic_from_profile("fwd") is None  # no summary
    h = bench.kernel_source_hash("fwd")
    (root / "profiles" / "counters_fwd.txt").write_text(
        "# header: lines with ':' after '#' are ignored\nkernel: fwd\nhbm_bytes_per_launch: 12345\n"
        "source_sha256: %s\n" % h)
    assert bench.traffic_from_profile("fwd") == 12345
    assert bench.traffic_from_profile("fwd_decode") is None
    with open(root / bench.KERNEL_SOURCES["fwd"][0], "a") as f:
        f.write("\n// edited\n")
    assert bench.kernel_source_hash("fwd") != h
    assert bench.traffic_from_profile("fwd") is None  # stale counters are not reported


def test_committed_counter_summaries_parse():
    for k in bench.KERNEL_SOURCES:
        path = os.path.join(ROOT, "profiles", "counters_%s.txt" % k)
        if not os.path.exists(path):
            continue
        rec = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
        assert int(float(rec["hbm_bytes_per_launch"])) > 0
        assert len(rec["source_sha256"].strip()) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    assert r.stdout == ""


def test_summary_statistics():
    """median of an even count is the mean of the middle two; p90 is the
    nearest-rank 90th percentile; min is the smallest."""
    s = bench.summary([5.0, 1.0, 3.0, 2.0])
    assert s["median"] == 2.5 and s["min"] == 1.0 and s["p90"] == 5.0 and s["n"] == 4
    s = bench.summary([float(x) for x in range(1, 31)])  # 1..30
    assert s["median"] == 15.5 and s["p90"] == 27.0 and s["min"] == 1.0
    assert bench.summary([7.0])["p90"] == 7.0


def test_roofline_fields():
    """attainable time is the larger of the MFMA-bound and HBM-bound times."""
    st = {"median": 0.1, "min": 0.1, "p90": 0.1, "n": 1}
    r = bench.roof(2.5e11, 8e8, st)          # 0.1 ms at 2.5 PF; 8e8 B at 8 TB/s = 0.1 ms
    assert abs(r["frac_of_mfma_peak"] - 1.0) < 1e-9 and abs(r["frac_of_attainable"] - 1.0) < 1e-9
    r = bench.roof(2.5e10, 1.6e9, st)        # HBM-bound: 0.2 ms attainable against 0.1 measured
    assert r["bound"] == "hbm" and abs(r["attainable_ms"] - 0.2) < 1e-12
    # compulsory bytes: forward Q K V in, O and lse out; backward Q K V O dO lse in, dQ dK dV out
    assert bench.compulsory_bytes(10, 3, 2, False) == 2 * 10 + 2 * 3 + 8
    assert bench.compulsory_bytes(10, 3, 2, True) == 4 * 10 + 4 * 3 + 8
