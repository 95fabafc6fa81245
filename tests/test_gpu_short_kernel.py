"""The short-split decode kernel (splits of at most 128 entries) in each of
its variants, against the fp64 oracle to the decode tolerance
(|d out| <= 2e-2 + 1e-2 |out_ref|, |d lse| <= 1e-3, infinities equal), and
against the pipelined kernel on the same plan (DSV4_DECODE_PIPELINED).

Variants: heads per workgroup 16, 32 and 64 (QK cut into k halves, one
(row block, head block) pair per wave, two row blocks per wave); one or two
64-row super-tiles per split with a ragged last split; block table or global
slots; with and without the scrub flag; a masked tail (valid_len) and SWA
entries.  The plan must pick the short-split kernel and the expected head
grouping for every case, so a selector change cannot silently move these
cases to the other kernel.
"""

import numpy as np
import pytest

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


# (B, H, topk, swa, S, expected heads per group)
CASES = [
    (1, 16, 120, 0, 1, 16),       # one split, two super-tiles, ragged second
    (2, 16, 200, 56, 4, 16),      # 64 entries a split: one super-tile
    (3, 32, 256, 64, 3, 16),      # 107 -> 128-entry chunks, two super-tiles, two head groups
    (64, 64, 192, 64, 2, 32),     # 128 entries a split, 32-head groups
    (128, 64, 192, 64, 2, 64),    # 64-head groups (grid 256)
    (2, 128, 96, 32, 1, 16),      # H = 128 in 16-head groups, one split
]


def _plan(w, S, flags=0, use_bt=True):
    gh = _gh()
    return dsv4.dsv4_sparse_decode_plan(gh.make_desc(w, use_bt=use_bt, flags=flags), S)


@pytest.mark.parametrize("B,H,topk,swa,S,hg", CASES)
@pytest.mark.parametrize("use_bt", [True, False])
def test_short_kernel_against_oracle_and_pipelined(B, H, topk, swa, S, hg, use_bt):
    gh = _gh()
    w = make_custom(B=B, H=H, topk=topk, swa=swa, seq_lens=[4096 + 37 * b for b in range(B)],
                    seed=900 + B + H + S, invalid_frac=0.04,
                    valid_len_range=(topk // 3, topk) if swa else None)
    plan = _plan(w, S, use_bt=use_bt)
    assert plan.partial_kernel == dsv4.DSV4_KERNEL_SHORT
    assert plan.heads_per_group == hg
    assert _plan(w, S, flags=dsv4.DSV4_DECODE_PIPELINED).partial_kernel == \
        dsv4.DSV4_KERNEL_PIPELINED
    print(f"short kernel B={B} H={H} Kt={topk + swa} S={S} hg={hg} bt={use_bt}", flush=True)
    dw = gh.DeviceWorkload(w)
    idx = dw.idx
    if not use_bt:
        import torch
        slots = oracle.convert_req_index_to_global(
            token_indices=w.topk_idx, block_table=w.block_table,
            max_blocks_per_req=w.max_blocks_per_seq, block_size=w.block_size, invalid_fill=-1)
        idx = torch.from_numpy(slots).cuda()
    out, lse = gh.gpu_decode(dw, num_splits=S, use_bt=use_bt, topk_idx=idx)
    ro, rl, _ = oracle.decode_workload(w, num_splits=S)
    gh.assert_decode_close(out, lse, ro, rl, f"short B={B} H={H} S={S}")
    po, pl = gh.gpu_decode(dw, num_splits=S, use_bt=use_bt, topk_idx=idx,
                           flags=dsv4.DSV4_DECODE_PIPELINED)
    gh.assert_decode_close(out, lse, po, pl, "short against pipelined")


@pytest.mark.parametrize("B,H,topk,swa,S,hg", [CASES[0], CASES[2], CASES[4]])
def test_short_kernel_scrub(B, H, topk, swa, S, hg):
    """Poisoned taking-part rows with the scrub flag give the bytes the same
    pool gives with those elements encoded as zeros."""
    gh = _gh()
    from synth import poison_rows
    w = make_custom(B=B, H=H, topk=topk, swa=swa, seq_lens=[4096 + 37 * b for b in range(B)],
                    seed=950 + B, invalid_frac=0.04)
    assert _plan(w, S, flags=dsv4.DSV4_DECODE_SCRUB).partial_kernel == dsv4.DSV4_KERNEL_SHORT
    valid = [int(s) for s in w.topk_idx[0, :8] if s >= 0][:4]
    kv_bad, kv_zero = poison_rows(w, 0, valid, seed=7)
    dw = gh.DeviceWorkload(w)
    import torch
    got = gh.gpu_decode(dw, num_splits=S, kv=torch.from_numpy(kv_bad).cuda(),
                        flags=dsv4.DSV4_DECODE_SCRUB)
    want = gh.gpu_decode(dw, num_splits=S, kv=torch.from_numpy(kv_zero).cuda(),
                         flags=dsv4.DSV4_DECODE_SCRUB)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert np.isfinite(got[0]).all()
