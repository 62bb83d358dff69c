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


def test_main_step_flops():
    """The main step credits the 32 chunks' pairs: 8.659e12 flops for
    H = 32, d = 128, L = 131072, s + r = 4096 (528,484,352 pairs per head);
    chunk 0 (no cache) has half a full chunk's pairs plus the growing rows."""
    w = si.WORKLOADS[5]
    assert bench.MAIN_WID == 5
    assert bench.key_count_sum(w.L, w.s, w.r) == 528484352
    assert bench.chunk_flops(w, 0, w.L) == 4.0 * 128 * 528484352 * 32
    assert abs(bench.chunk_flops(w, 0, w.L) - 8.659e12) / 8.659e12 < 1e-3
    parts = sum(bench.chunk_flops(w, p, p + w.chunk) for p in range(0, w.L, w.chunk))
    assert parts == bench.chunk_flops(w, 0, w.L)
    assert bench.chunk_flops(w, 4096, 8192) == 4.0 * 128 * 4096 * 4096 * 32


def test_backward_and_decode_work():
    w = si.WORKLOADS[2]
    assert bench.backward_flops(w) == 10.0 * 128 * 25167872 * 32
    w4 = si.WORKLOADS[4]
    assert bench.decode_step_bytes(w4) == 1075052544


def _note(tmp_path, monkeypatch, family, workload, kind, body, sha):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    p = tmp_path / ("%s_%s_%s.md" % (family, workload, kind))
    p.write_text(body + "\nkernel_sources_sha256: %s\n" % sha)


def test_note_parser_follows_the_kernel_source_hash(tmp_path, monkeypatch):
    for fam in bench.KERNEL_SOURCES:
        sha = bench.kernel_sources_sha256(fam)
        _note(tmp_path, monkeypatch, fam, "wl", "traffic", "traffic_bytes_per_launch: 123456", sha)
        assert bench.recorded(fam, "wl", "traffic", "traffic_bytes_per_launch") == 123456
        _note(tmp_path, monkeypatch, fam, "wl", "mfma", "mfma_busy_frac: 0.5", "0" * 64)
        assert bench.recorded(fam, "wl", "mfma", "mfma_busy_frac") is None
        assert bench.recorded(fam, "other", "traffic", "traffic_bytes_per_launch") is None


def test_committed_notes_parse():
    """Every counter note under profiles/ carries the figure its kind
    promises where the bench reads it (a `key: value` line), and was taken
    on the committed kernel sources (the bench's roofline would otherwise
    show null for it)."""
    keys = {"traffic": "traffic_bytes_per_launch", "mfma": "mfma_busy_frac", "sclk": "sclk_ghz_timed"}
    n = 0
    for f in os.listdir(bench.PROFILES):
        m = __import__("re").match(r"(prefill_pp_kernel|decode_split_kernel|backward)_(.+)_(traffic|mfma|sclk)\.md$", f)
        if not m:
            continue
        assert bench.recorded(m.group(1), m.group(2), m.group(3), keys[m.group(3)]) is not None, f
        n += 1
    assert n >= 7


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_global_key_count_sum_is_the_sum_of_key_set_sizes():
    for L, s, r, G in [(300, 4, 28, [2, 50, 51, 299]), (200, 0, 16, [0, 7, 100]), (90, 70, 10, [3, 80])]:
        want = sum(len(oracle.key_set(t, s, r, globals_=G)) for t in range(L))
        assert bench.global_key_count_sum(L, s, r, G) == want


def test_note_hash_ignores_comments_only():
    """A counter note stays valid across comment edits, not across code edits."""
    a = "int f(int x) { // the row\n  return x + 1; /* next\n tile */ }\n"
    b = "int f(int x) {\n  // another comment\n  return x + 1;   }\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
