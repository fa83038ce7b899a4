"""Host logic of bench.py that needs no GPU: the one-GPU contract, the
kernel-source hash that keeps stored traffic figures tied to the kernels
they were measured on, and the traffic lookup itself."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_source_tokens_ignore_comments_and_layout_only():
    src = "int f(int x) {\n  // doubles x\n  return 2 * x; /* plain */\n}\n"
    same = "int f(int x) { return 2 * x; }  // another comment\n"
    other = "int f(int x) { return 3 * x; }\n"
    assert bench._code_tokens(src) == bench._code_tokens(same)
    assert bench._code_tokens(src) != bench._code_tokens(other)


def test_kernel_source_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)


def test_traffic_is_reported_only_for_the_measured_kernels(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"w_now": {"kernel_source_hash": h, "bytes_per_launch": 123},
                             "w_old": {"kernel_source_hash": "0" * 16, "bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w_now") == 123
    assert bench.measured_traffic("w_old") is None  # kernels changed since the counters were taken
    assert bench.measured_traffic("w_missing") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic("w_now") is None


def test_committed_traffic_figures_carry_the_counter_scales():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    entries = {k: v for k, v in t.items() if not k.startswith("_")}
    assert entries
    for name, e in entries.items():
        # bytes = FETCH_SIZE KiB x read scale + WRITE_SIZE KiB x write scale, x 1024
        want = (e["fetch_kib_per_step"] * e["read_scale"] + e["write_kib_per_step"] * e["write_scale"]) * 1024
        assert abs(e["bytes_per_launch"] - want) <= 0.001 * want + 1024, name
