"""Host-side checks of bench.py: its one-GPU contract and the causal pair
count behind its FLOP figures (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import cpa_oracle  # noqa: E402
from sequence_attention_cpa_amd.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["tiny", "12k", "128k", "1m"])
def test_causal_pairs_match_the_zigzag_closed_form(name):
    """Every zigzag rank meets 2N C^2 + C visible (query, key) pairs per head:
    the count bench.py turns into useful FLOP (4 D per pair)."""
    w = WORKLOADS[name]
    pos = cpa_oracle.zigzag_layout(w.L, w.N)
    want = 2 * w.N * w.C * w.C + w.C
    for r in sorted({0, w.N // 2, w.N - 1}):
        got = sum(bench.causal_pairs(pos[r], pos[j]) for j in range(w.N))
        assert got == want, f"{name} rank {r}: {got} pairs, closed form {want}"


def test_causal_pairs_of_a_contiguous_split():
    """Under a contiguous split rank r meets r Lr^2 + Lr (Lr + 1) / 2 pairs: the
    imbalance bench.py reports next to the zigzag's."""
    import numpy as np

    L, N = 4096, 4
    Lr = L // N
    pos = np.arange(L, dtype=np.int64).reshape(N, Lr)
    for r in range(N):
        got = sum(bench.causal_pairs(pos[r], pos[j]) for j in range(N))
        assert got == r * Lr * Lr + Lr * (Lr + 1) // 2


def test_traffic_comes_from_the_committed_counters_of_the_same_kernel_and_workload():
    """The roofline's traffic figure is the profiled 128k launch's, taken on
    the attention source as it stands; other workloads report none."""
    import json
    with open(bench.PMC_FILES["global"]) as f:
        d = json.load(f)
    got = bench.pmc_traffic("global", "128k")
    if d.get("kernel_sha") == bench.kernel_sha():
        assert got == d["traffic_bytes_per_launch"] > 0
        assert d["traffic_bytes_per_launch"] == (d["read_bytes_per_launch"]
                                                 + d["write_bytes_per_launch"])
    else:
        assert got is None
    for other in ("12k", "1m", "128k_qkv"):
        assert bench.pmc_traffic("global", other) is None
