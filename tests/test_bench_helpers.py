"""bench.py's host-side helpers: its count of the entries that take part
(the throughput numerator) equals the oracle's on workloads with invalid
entries, a masked tail, SWA entries and several tokens per sequence."""

from __future__ import annotations

import pytest

import bench
import oracle
from synth import make_custom, make_workload


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_valid_entries_match_the_oracle_on_the_workloads(ci):
    w = make_workload(ci)
    assert bench._valid_entries(w) == oracle.decode_workload(w)[2]


@pytest.mark.parametrize("s_q", [1, 2])
def test_valid_entries_match_the_oracle_with_masked_tails(s_q):
    w = make_custom(B=4, H=16, topk=200, swa=24, seq_lens=[3000, 150, 900, 40], seed=91,
                    invalid_frac=0.07, valid_len_range=(60, 220), s_q=s_q)
    assert bench._valid_entries(w) == oracle.decode_workload(w)[2]


def test_more_than_one_gpu_is_refused_with_a_message():
    """The path and its benchmark are single-GPU: --gpus N > 1 exits with a
    message (before touching a GPU)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""
