"""CPU: bench.py's command-line contract that needs no GPU. A request for more
than one GPU is refused with a message and exit status 2 before anything touches
a device, and the committed counter figures are read back as bench.py reports
them."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    import glob

    files = glob.glob(bench.TRAFFIC_FILE.format("*"))
    assert files, "no committed counter summary"
    for path in files:
        with open(path) as f:
            rec = json.load(f)
        assert path == bench.TRAFFIC_FILE.format(rec["workload"])
        got = bench.measured_traffic(rec["workload"])
        if rec["kernel_sha"] == bench.kernel_sha():
            assert got == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        else:
            assert got is None
    assert bench.measured_traffic("no-such-workload") is None


def test_roofline_bound_follows_the_ridge():
    import mk_inputs

    large = bench.roofline_of(mk_inputs.BY_NAME["large"], 1000.0)
    assert large["bound"] == "mfma" and large["unit"] == "TFLOP/s"
    assert abs(large["achieved"] - 2 * 8192 ** 3 / 1e-3 / 1e12) < 0.1
    mlp = bench.roofline_of(mk_inputs.BY_NAME["mlp"], 1000.0)
    assert mlp["bound"] == "hbm" and mlp["unit"] == "GB/s"
    assert abs(mlp["frac"] - mlp["achieved"] / bench.HBM_PEAK_GBPS) < 1e-4


def test_kernel_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)
    assert len(bench.kernel_sha()) == 16
