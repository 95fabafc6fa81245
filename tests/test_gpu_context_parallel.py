"""Context-parallel sharding, shown on one GPU: the index list is cut into n
shares (each GPU's part of the KV sequence); each share is decoded alone
without the sink into a normalised output and its lse, exactly the split
contract; the n results merged by dsv4_combine_splits with the sink must
match the oracle's decode of the whole list.  On n GPUs the merge's input
arrives by an all-gather; here the shares run one after another."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_workload

pytestmark = pytest.mark.gpu


def _share_decode(dw, cols, topk, swa, out, lse):
    """Decodes entries [cols, cols + topk + swa) of every index row."""
    from tests import gpu_helpers as gh
    w = dw.w
    kw = dict(batch=w.B, num_heads=w.H, topk=topk, swa=swa, block_size=w.block_size,
              num_blocks=w.num_blocks, page_stride=w.page_stride, sm_scale=w.sm_scale,
              max_blocks_per_seq=w.max_blocks_per_seq,
              block_table_stride=w.block_table.shape[1], topk_idx_stride=w.Kt)
    plan = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**kw), 0)
    ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
          if plan.workspace_bytes else None)
    desc = dsv4.make_desc(workspace=ws, **kw)
    dsv4.dsv4_sparse_decode(desc, dw.q, dw.kv, dw.bt, dw.idx[:, cols:], None, None, out, lse, 0)
    return gh


@pytest.mark.parametrize("ci,n", [(2, 2), (2, 4), (2, 8), (1, 4)])
def test_shares_merged_by_the_combine_match_the_full_decode(ci, n):
    from tests import gpu_helpers as gh
    print(f"context parallel workload {ci} n={n}", flush=True)
    w = make_workload(ci)
    assert w.valid_len is None
    dw = gh.DeviceWorkload(w)
    m = w.topk // n
    shares = [(i * m, m, 0) for i in range(n)]
    if w.swa:
        shares.append((w.topk, 0, w.swa))          # the SWA entries: one more share
    P = len(shares)
    part_out = torch.empty((w.B, w.H, P, 512), dtype=torch.bfloat16, device="cuda")
    part_lse = torch.empty((w.B, w.H, P), dtype=torch.float32, device="cuda")
    for i, (cols, topk, swa) in enumerate(shares):
        out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        _share_decode(dw, cols, topk, swa, out, lse)
        part_out[:, :, i] = out
        part_lse[:, :, i] = lse
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    dsv4.dsv4_combine_splits(w.B, w.H, P, part_out, part_lse, dw.sink, out, lse, None)
    torch.cuda.synchronize()
    ref_out, ref_lse, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(),
                           ref_out, ref_lse, f"context parallel ci={ci} n={n}")
