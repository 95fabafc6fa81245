"""The seeded input generator: the same seed gives the same bytes, and each
workload follows its stated recipe (sizes, invalid fraction, SWA placement,
scale-code range, padding, unused table entries, valid_len range)."""

from __future__ import annotations

import numpy as np
import pytest

from synth import CONFIGS, make_workload, workload_digest


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_same_seed_same_bytes(ci):
    a, b = make_workload(ci), make_workload(ci)
    assert workload_digest(a) == workload_digest(b)
    assert workload_digest(make_workload(ci, seed=7)) != workload_digest(a)


def _row_bytes(w, b, slot):
    bs = w.block_size
    page = int(w.block_table[b // w.s_q, slot // bs])
    off = slot % bs
    return (w.kv[page, off * 576:(off + 1) * 576],
            w.kv[page, bs * 576 + off * 8: bs * 576 + off * 8 + 8])


@pytest.mark.parametrize("ci", [0, 1, 2, 4])
def test_recipe(ci):
    c = CONFIGS[ci]
    w = make_workload(ci)
    assert (w.B, w.H, w.topk, w.swa) == (c["B"], c["H"], c["topk"], c["swa"])
    assert w.q.shape == (w.B, w.H, 512) and w.sink.shape == (w.H,)
    assert w.sm_scale == float(np.float32(512 ** -0.5))
    main = w.topk_idx[:, :w.topk]
    for b in range(w.B):
        L = int(w.seq_lens[b])
        n = min(w.topk, L)
        # Exactly round(p * topk) main positions are -1 on top of any the
        # sequence is too short to fill; the rest are distinct slots < L.
        live = main[b][main[b] >= 0]
        assert len(np.unique(live)) == len(live) and np.all(live < L)
        n_inv = int(np.floor(c["invalid_frac"] * w.topk + 0.5))
        assert (main[b] < 0).sum() >= n_inv
        assert len(live) >= n - n_inv
        # SWA: the last swa positions of the sequence, ascending.
        np.testing.assert_array_equal(w.topk_idx[b, w.topk:], np.arange(L - w.swa, L))
        # Pages: one per 64 slots, the rest of the table -1.
        pages = -(-L // w.block_size)
        assert np.all(w.block_table[b, :pages] >= 0) and np.all(w.block_table[b, pages:] == -1)
        # Rows that take part: scale codes in [120, 130], pad byte 0.
        for slot in live[:8]:
            _, sc = _row_bytes(w, b, int(slot))
            assert np.all((sc[:7] >= 120) & (sc[:7] <= 130)) and sc[7] == 0
    if c["valid_len"] is None:
        assert w.valid_len is None
    else:
        lo, hi = c["valid_len"]
        assert np.all((w.valid_len >= lo) & (w.valid_len <= hi))
    if c["seq_len"][0] == "loguniform":
        assert np.all((w.seq_lens >= c["seq_len"][1]) & (w.seq_lens <= c["seq_len"][2]))
    else:
        assert np.all(w.seq_lens == c["seq_len"][1])
    # Every page is used by one sequence only (a shuffled pool); the slack
    # pages no table names hold nothing but 0xFF poison.
    used = w.block_table[w.block_table >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < w.num_blocks
    slack = np.setdiff1d(np.arange(w.num_blocks), used)
    assert len(slack) > 0 and np.all(w.kv[slack] == 0xFF)
