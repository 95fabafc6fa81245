"""Measurement aids on the GPU (include/dsv4_diag.h): the short-split
kernel's stamped variant gives the same bytes as the decode's first stage,
and ten ordered stamps per workgroup."""

import numpy as np
import pytest
import torch

import sparse_mla_attention_block_amd as dsv4
from synth import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_short_timeline_matches_the_partial_stage(ci):
    from tests import gpu_helpers as gh
    w = make_workload(ci)
    dw = gh.DeviceWorkload(w)
    desc = gh.make_desc(w)
    plan = dsv4.dsv4_sparse_decode_plan(desc, w.num_splits)
    assert plan.partial_kernel == dsv4.DSV4_KERNEL_SHORT
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws)
    outs = []
    for stamped in (False, True):
        out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        if stamped:
            stamps = torch.zeros(plan.grid_partial * 10, dtype=torch.int64, device="cuda")
            dsv4.dsv4_short_timeline(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out, lse,
                                     w.num_splits, stamps)
        else:
            dsv4.dsv4_sparse_decode_partial(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out,
                                            lse, w.num_splits)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone(), ws.clone()))
    (o0, l0, w0), (o1, l1, w1) = outs
    if plan.num_splits == 1:
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    else:
        assert torch.equal(w0, w1)                         # partials and their lse
    t = stamps.view(-1, 10).cpu().numpy().astype(np.int64)
    t = t[t[:, 1] > 0]
    assert t.shape[0] == w.B * plan.num_splits * plan.head_groups
    assert np.all(np.diff(t[:, 1:9], axis=1) >= 0)        # shader-clock stamps in order
    assert np.all(t[:, 9] >= t[:, 0])
