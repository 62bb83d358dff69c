"""Host-side logic of bench.py (CPU only): the algorithmic work it credits,
the counter-note parsers and their source-hash guard, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import swa_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("L,s,r,pos0", [(1, 0, 1, 0), (300, 4, 28, 0), (257, 0, 1000, 0), (200, 70, 40, 0),
                                        (130, 4, 100, 4096), (64, 3, 5, 77)])
def test_key_count_sum_is_the_sum_of_key_set_sizes(L, s, r, pos0):
    """The credited pairs are exactly the oracle's enumerated key sets."""
    want = sum(len(oracle.key_set(t, s, r)) for t in range(pos0, pos0 + L))
    assert bench.key_count_sum(L, s, r, pos0) == want


@pytest.mark.parametrize("L,s,r,dil", [(300, 4, 28, 2), (200, 0, 17, 3), (150, 10, 9, 7), (90, 4, 5, 100)])
def test_dilated_key_count_sum_is_the_sum_of_dilated_key_sets(L, s, r, dil):
    want = sum(len(oracle.key_set(t, s, r, dil)) for t in range(L))
    assert bench.dilated_key_count_sum(L, s, r, dil) == want


def test_main_workload_flops():
    """4 d flops per (query, key) pair of U(t): 4.124e11 for GQA 32/8,
    d = 128, L = 8192, s = 0, r = 4096 (25,167,872 pairs per head)."""
    w = si.WORKLOADS[2]
    assert bench.key_count_sum(w.L, w.s, w.r) == 25167872
    assert bench.prefill_flops(w) == 4.0 * 128 * 25167872 * 32
    assert abs(bench.prefill_flops(w) - 4.124e11) / 4.124e11 < 1e-3


def _note(tmp_path, body, sha):
    p = tmp_path / "note.md"
    p.write_text(body + "\nkernel_sources_sha256: %s\n" % sha)
    return str(p)


def test_note_parsers_follow_the_kernel_source_hash(tmp_path, monkeypatch):
    sha = bench.kernel_sources_sha256()
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", _note(tmp_path, "traffic_bytes_per_launch: 123456", sha))
    assert bench.recorded_traffic() == 123456
    monkeypatch.setattr(bench, "MFMA_NOTE", _note(tmp_path, "mfma_busy_frac: 0.5", sha))
    assert bench.recorded_mfma_busy() == 0.5
    monkeypatch.setattr(bench, "SCLK_NOTE", _note(tmp_path, "sclk_ghz_timed: 2.0", sha))
    assert bench.recorded_sclk() == 2.0
    stale = "0" * 64
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", _note(tmp_path, "traffic_bytes_per_launch: 123456", stale))
    monkeypatch.setattr(bench, "MFMA_NOTE", _note(tmp_path, "mfma_busy_frac: 0.5", stale))
    monkeypatch.setattr(bench, "SCLK_NOTE", _note(tmp_path, "sclk_ghz_timed: 2.0", stale))
    assert bench.recorded_traffic() is None and bench.recorded_mfma_busy() is None and bench.recorded_sclk() is None
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic() is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
