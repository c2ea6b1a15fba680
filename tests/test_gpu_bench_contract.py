"""bench.py end to end on the GPU, briefly: one JSON line with the contract's
keys, a roofline object and (for the default workload) the oracle's CPU
baseline, for the forward, the frame-wise and the attention workloads."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert KEYS <= set(d), KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= set(rf)
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    return d


def test_bench_default_line():
    d = _bench("--cpu-seconds", "1")
    assert d["config"]["workload"] == "rollout_h16_d128" and d["roofline"]["bound"] == "hbm"
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "tokens/s"


@pytest.mark.parametrize("workload,bound", [("frame_stream_h16_d64", "hbm"), ("attn_chunk_h16_d64", "mfma")])
def test_bench_other_entry_points(workload, bound):
    d = _bench("--workload", workload, "--no-cpu")
    assert d["config"]["workload"] == workload and d["roofline"]["bound"] == bound
