"""Host-side logic of bench.py that needs no GPU: the algorithmic byte counts
behind the roofline figure, the traffic summaries it reads from profiles/ and
the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS  # noqa: E402


def test_algorithmic_bytes_of_the_streaming_chunk():
    # B=1, H=16, T=2640, d=64, bf16 inputs: q, k, v, alpha, beta read once,
    # out written once, the fp32 state read and written once: 27.7 MB with
    # fp32 outputs, 22.3 MB with bf16 outputs
    wl = WORKLOADS["stream_chunk_h16_d64"]
    tokheads = 16 * 2640
    per_token = 2 * 64 * 2 + 64 * 2 + 2 * 2
    state = 16 * 64 * 64 * 4
    assert bench.algorithmic_bytes(wl, 4, True) == tokheads * (per_token + 64 * 4) + 2 * state == 27726848
    assert bench.algorithmic_bytes(wl, 2, True) == tokheads * (per_token + 64 * 2) + 2 * state
    assert round(bench.algorithmic_bytes(wl, 2, True) / 1e6, 1) == 22.3
    # no incoming state: the state is written only; an output gate is read once
    assert bench.algorithmic_bytes(wl, 4, False) == 27726848 - state
    assert bench.algorithmic_bytes(wl, 4, True, True) == 27726848 + tokheads * 64 * 2
    assert bench.algorithmic_flops(wl) == 6 * tokheads * 64 * 64


def test_traffic_is_read_only_for_matching_sources():
    assert bench.read_traffic("0" * 16, "stream_chunk_h16_d64") is None
    assert bench.read_traffic(bench.kernel_source_hash(), "no_such_workload") is None


def test_committed_traffic_profile_matches_the_sources():
    # the counter summaries under profiles/ were taken on the current kernels
    t = bench.read_traffic(bench.kernel_source_hash(), "stream_chunk_h16_d64")
    assert t is not None, "profiles/ holds counters of other kernel sources: capture them again"
    assert 1.0 <= t / bench.algorithmic_bytes(WORKLOADS["stream_chunk_h16_d64"], 4, True) < 4.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
