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
