"""Host logic of the benchmark (no GPU): the one-GPU guard, the roofline
fractions and the digest check that decides whether stored HBM counter
readings still describe the kernels being timed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_effective_bandwidth_and_roofline_fractions():
    # 8 GB moved in one second is exactly the HBM peak
    assert bench.effective_gbps(8e9, 1.0) == pytest.approx(8.0)
    assert bench.roof_fraction("hbm", 4e9, 0, 1.0) == pytest.approx(4.0 / bench.HBM_PEAK_GBS)
    # half the dense bf16 matrix-core rate
    assert bench.roof_fraction("mfma", 0, bench.BF16_MFMA_PEAK / 2, 1.0) == pytest.approx(0.5)
    # fixed-order arithmetic counts one FMA (two flops) per code and column
    fl = 2 * bench.FP32_VALU_FMA_PER_S * 0.25
    assert bench.roof_fraction("alu", 0, fl, 1.0) == pytest.approx(0.25)


def test_source_digest_is_stable_and_hex():
    a, b = bench.source_digest(), bench.source_digest()
    assert a == b and len(a) == 16 and int(a, 16) >= 0


def test_digest_ignores_comments_but_not_code():
    src = 'int a = 1; // one\n/* two\n lines */ const char *s = "x // y";\n'
    same = '// a new note\nint a = 1;   /* changed */\nconst char *s = "x // y";\n'
    assert bench.strip_comments(src) == bench.strip_comments(same)
    assert bench.strip_comments(src) != bench.strip_comments(src.replace("a = 1", "a = 2"))
    assert bench.strip_comments(src) != bench.strip_comments(src.replace("x // y", "x // z"))  # in a string


def test_digest_covers_the_header_and_the_compile_flags(monkeypatch):
    flags = bench.build_flags()
    assert "-ffp-contract=off" in flags and "--offload-arch=gfx950" in flags
    assert not any(f.startswith("-I") for f in flags)   # paths differ between checkouts
    base = bench.source_digest()
    monkeypatch.setattr(bench, "build_flags", lambda: flags + ["-ffast-math"])
    assert bench.source_digest() != base
    monkeypatch.setattr(bench, "build_flags", lambda: flags)
    real_open = open

    def header_changed(path, *a, **k):
        if str(path).endswith(os.path.join("include", "qmv.h")):
            import io
            with real_open(path, *a, **k) as f:
                return io.StringIO(f.read() + "\nint qmv_extra_declaration;\n")
        return real_open(path, *a, **k)
    monkeypatch.setattr("builtins.open", header_changed)
    assert bench.source_digest() != base


def test_stored_traffic_follows_the_digest(tmp_path, monkeypatch):
    rec = {"source_digest": "0123456789abcdef", "hbm_bytes_per_launch": 12345}
    (tmp_path / "t.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("t.json", "0123456789abcdef") == 12345
    assert bench.stored_traffic("t.json", "fedcba9876543210") is None
    assert bench.stored_traffic("missing.json", "0123456789abcdef") is None



def test_headline_bytes_are_the_lm_head_stream():
    # packed int2 weights (K/4 bytes a row), fp16 row scales, fp16
    # activations, and the index + maximum written per activation row
    assert bench.argmax_bytes(1) == 262144 * 1536 // 4 + 262144 * 2 + 1536 * 2 + 8 == 101_190_664
    assert bench.argmax_bytes(4) - bench.argmax_bytes(1) == 3 * (1536 * 2 + 8)


def test_gather_counts_each_distinct_expert_once():
    import numpy as np
    E, N, K = 32, 5760, 2880
    eb = N * K // 2 + N * (K // 32)
    ids = np.array([[0, 1, 2, 3], [3, 2, 1, 0]], np.int32)  # two rows, the same four experts
    assert bench.gather_bytes(ids, E, N, K, 2, 4) == 4 * eb + 2 * K * 2 + 2 * 4 * 4 + 2 * 4 * N * 4
    ids2 = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], np.int32)
    assert bench.gather_bytes(ids2, E, N, K, 2, 4) - bench.gather_bytes(ids, E, N, K, 2, 4) == 4 * eb
    # an id outside [0, E) reads no expert
    assert bench.gather_bytes(np.array([[0, 40]], np.int32), E, N, K, 1, 2) == eb + K * 2 + 2 * 4 + 2 * N * 4


def test_timed_rotation_continues_after_the_warmup(monkeypatch):
    seen = []
    monkeypatch.setattr(bench, "graph_of", lambda calls: [c() for c in calls] and calls)
    monkeypatch.setattr(bench, "time_graph", lambda g: 1.0)
    sec = bench.run_case(lambda i: (lambda: seen.append(i)), steps=7, warmup=3)
    assert seen == list(range(10))   # warmup 0..2, timed 3..9: no copy is re-read back to back
    assert sec == 1.0 / 7


def test_warmup_replays_until_the_minimum_load_time(monkeypatch):
    """min_warm_s replays the warmup graph (steps 0 .. W-1 each time, so the
    rotation still continues into the timed calls) until that much GPU time
    has passed; the timed graph is replayed exactly once."""
    replays = []
    monkeypatch.setattr(bench, "graph_of", lambda calls: ("warm" if len(calls) == 3 else "timed", calls))
    monkeypatch.setattr(bench, "time_graph", lambda g: replays.append(g[0]) or (0.004 if g[0] == "warm" else 0.5))
    sec = bench.run_case(lambda i: (lambda: None), steps=5, warmup=3, min_warm_s=0.01)
    assert replays == ["warm", "warm", "warm", "timed"]   # 4 + 4 + 4 ms >= 10 ms
    assert sec == 0.5 / 5
    replays.clear()
    bench.run_case(lambda i: (lambda: None), steps=5, warmup=3)
    assert replays == ["warm", "timed"]                     # the headline: exactly W warmup calls


def test_default_run_is_bounded():
    a = bench.parse([])
    assert a.gpus == 1 and (a.steps + a.warmup) * 40e-6 < 60 and a.warmup < a.steps
