"""The allocation-free decode (dsv4_sparse_decode_noalloc) on the GPU.

Two calls in a row through the C ABI, the second with a smaller input, each
checked bit for bit against dsv4_sparse_decode with a caller's workspace
(the same kernels, so the same bytes) and against the fp64 oracle to the
decode tolerance; the first call leaves its partials in the library's
scratch, which the second must not read.  Then a one-split call (no scratch
needed) and a request too large for the scratch, which must be refused on
the host with a clear error.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, make_workload

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _both(w, S, flags=0):
    gh = _gh()
    dw = gh.DeviceWorkload(w)
    desc = gh.make_desc(w, flags=flags)
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    assert nbytes <= dsv4.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            dsv4.dsv4_sparse_decode_noalloc(gh.make_desc(w, flags=flags), dw.q, dw.kv, dw.bt,
                                            dw.idx, dw.vl, dw.sink, out, lse, S)
        else:
            dsv4.dsv4_sparse_decode(gh.make_desc(w, workspace=ws, flags=flags), dw.q, dw.kv,
                                    dw.bt, dw.idx, dw.vl, dw.sink, out, lse, S)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs, nbytes


def test_noalloc_decode_matches_the_workspace_decode():
    gh = _gh()
    cases = [
        ("short_batch, selector plan", make_workload(1), 0),
        ("smaller batch, 3 splits", make_custom(B=2, H=32, topk=300, swa=20,
                                                seq_lens=[4000, 700], seed=500,
                                                invalid_frac=0.03, valid_len_range=(150, 300)), 3),
        ("tiny, one split", make_workload(0), 1),
    ]
    sizes = []
    for what, w, S in cases:
        print(f"noalloc: {what}", flush=True)
        ((o_ref, l_ref), (o, l)), nbytes = _both(w, S)
        sizes.append(nbytes)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), what
        assert torch.equal(l, l_ref), what
        ro, rl, _ = oracle.decode_workload(w)
        gh.assert_decode_close(o.float().double().cpu().numpy(), l.double().cpu().numpy(),
                               ro, rl, what)
    assert sizes[0] > sizes[1] > 0 and sizes[2] == 0


def test_noalloc_with_balanced_splits():
    """DSV4_DECODE_BALANCE sizes the scratch use by the split slots; the
    result matches the workspace decode bit for bit, twice in a row (the
    second call smaller, with fewer tokens)."""
    gh = _gh()
    flags = dsv4.DSV4_DECODE_BALANCE | dsv4.DSV4_DECODE_PIPELINED
    for B, seed in ((6, 520), (3, 521)):
        w = make_custom(B=B, H=64, topk=512, swa=64, seq_lens=[4000 + 500 * b for b in range(B)],
                        seed=seed, invalid_frac=0.03, valid_len_range=(20, 512))
        plan = dsv4.dsv4_sparse_decode_plan(gh.make_desc(w, flags=flags), 4)
        assert plan.balanced_splits == 4 and plan.num_splits == 5
        print(f"noalloc balanced B={B}", flush=True)
        ((o_ref, l_ref), (o, l)), _ = _both(w, 4, flags)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(l, l_ref)
        ro, rl, _ = oracle.decode_workload(w)
        gh.assert_decode_close(o.float().double().cpu().numpy(), l.double().cpu().numpy(),
                               ro, rl, f"noalloc balanced B={B}")


def test_noalloc_refuses_a_decode_larger_than_its_scratch():
    gh = _gh()
    w = make_workload(0)
    dw = gh.DeviceWorkload(w)
    desc = dsv4.make_desc(batch=256, num_heads=128, topk=2048, swa=0, block_size=64,
                          num_blocks=w.num_blocks, page_stride=w.page_stride, sm_scale=w.sm_scale)
    assert dsv4.dsv4_sparse_decode_workspace_bytes(desc, 64) > dsv4.NOALLOC_SCRATCH_BYTES
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsv4.Dsv4Error) as e:
        dsv4.dsv4_sparse_decode_noalloc(desc, dw.q, dw.kv, None, dw.idx, None, None, out, None, 64)
    assert e.value.status == dsv4.DSV4_ERR_WORKSPACE_TOO_SMALL
    assert "allocation-free" in str(e.value) and "DSV4_NOALLOC_SCRATCH_BYTES" in str(e.value)
