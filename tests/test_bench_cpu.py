"""The benchmark's host-side contract (CPU only): the one-GPU guard and the
use of committed counter summaries for the roofline's `traffic` field."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""                       # no JSON line for a refused run


def test_library_digest_is_stable():
    d = bench.library_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", d) and d == bench.library_digest()


def test_measured_traffic_uses_only_rows_of_the_current_sources(tmp_path, monkeypatch):
    d = bench.library_digest()
    f = tmp_path / "traffic.md"
    f.write_text(
        "| kernel | src digest | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB | HBM bytes/dispatch |\n"
        "|---|---|---|---|---|---|---|\n"
        f"| `k_a<true, 1>` | {d} | 10 | 1.0 | 1.0 | 1.0 | 1000 |\n"
        f"| `k_a_reduce<true, 1>` | {d} | 10 | 1.0 | 1.0 | 1.0 | 24 |\n"
        "| `k_b<true>` | 0000000000000000 | 10 | 1.0 | 1.0 | 1.0 | 5000 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k_a<true, 1>") == 1000
    assert bench.measured_traffic("k_a<true, 1> + k_a_reduce<true, 1>") == 1024
    assert bench.measured_traffic("k_b<true>") is None            # taken on other sources
    assert bench.measured_traffic("k_c<0>") is None               # no row


def test_committed_traffic_summary_has_the_decode_kernels():
    text = open(bench.TRAFFIC_FILE).read()
    rows = [l for l in text.splitlines() if l.startswith("| `")]
    names = {l.split("|")[1].strip().strip("`") for l in rows}
    assert any(n.startswith("k_w4a16_decode<") for n in names)
    assert all(len(l.strip().strip("|").split("|")) == 7 for l in rows)
    assert "FETCH_SIZE" in text and "WRITE_SIZE" in text and "Calibration" in text


def test_w4_codes_reads_the_packed_layout_like_the_oracle():
    """The benchmark's host-side reader of packed weights (used for its
    tensor-level metrics) against the oracle's unpack and dequantization."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, 512)) * 0.02).astype(np.float32)
    for asym in (False, True):
        qw, sc, z = oracle.w4_pack(w, 128, asym)
        u, deq = bench.w4_codes(qw, sc, z, np)
        u_ref, _, _ = oracle.w4_unpack(qw, sc, z, 48, 512)
        assert np.array_equal(u, u_ref)
        assert np.array_equal(deq, oracle.w4_dequant(qw, sc, z, 48, 512))
