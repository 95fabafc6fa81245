"""The HIP path against the hand-worked fixtures in tests/golden/: the
two-row decode (closed-form outputs and lse, with no sink and with a sink logit of 1, every
byte of the pool that takes no part is NaN) and the hand-worked conversion
(bit-exact)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import sparse_mla_attention_block_amd as dsv4
from tests import golden_fixtures as gf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["no_sink", "sink_one"])
@pytest.mark.parametrize("S", [1, 2])
def test_hip_decode_reproduces_the_hand_worked_decode(case, S):
    from tests import gpu_helpers as gh
    print(f"golden decode {case} S={S}", flush=True)
    fx = gf.load("decode_two_rows.json")
    inp = gf.decode_inputs(fx)
    g = inp["geometry"]
    dev = torch.device("cuda")
    kw = dict(batch=g["B"], num_heads=g["H"], topk=g["topk"], swa=g["swa"],
              block_size=g["block_size"], num_blocks=g["num_blocks"],
              page_stride=g["page_stride"], sm_scale=g["sm_scale"],
              max_blocks_per_seq=inp["max_blocks_per_seq"],
              block_table_stride=inp["block_table"].shape[1])
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(dsv4.make_desc(**kw), S)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev) if nbytes else None
    desc = dsv4.make_desc(workspace=ws, **kw)
    q = torch.from_numpy(inp["q"].view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(inp["kv"]).to(dev)
    bt = torch.from_numpy(inp["block_table"]).to(dev)
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    sink = (None if case == "no_sink"
            else torch.full((g["H"],), fx[case]["sink_value"], dtype=torch.float32, device=dev))
    out = torch.full((g["B"], g["H"], 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((g["B"], g["H"]), float("nan"), dtype=torch.float32, device=dev)
    dsv4.dsv4_sparse_decode(desc, q, kv, bt, idx, None, sink, out, lse, S)
    torch.cuda.synchronize()
    ref_out, ref_lse = gf.decode_expected(fx, case)
    gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(),
                           ref_out, ref_lse, f"golden {case} S={S}")


@pytest.mark.parametrize("fill", [0, -1])
def test_hip_conversion_reproduces_the_hand_worked_conversion(fill):
    from tests import gpu_helpers as gh
    print(f"golden conversion fill={fill}", flush=True)
    fx = gf.load("convert_hand_worked.json")
    got = gh.gpu_convert(token_indices=np.array(fx["token_indices"], dtype=np.int32),
                         block_table=np.array(fx["block_table"], dtype=np.int32),
                         max_blocks_per_req=fx["max_blocks_per_req"],
                         block_size=fx["block_size"],
                         req_id=np.array(fx["req_id"], dtype=np.int32), invalid_fill=fill)
    want = fx["expected"]["fill_0" if fill == 0 else "fill_minus_1"]
    np.testing.assert_array_equal(got, np.array(want, dtype=np.int32))
