"""Decode that also writes the global slots (dsv4_sparse_decode_with_slots).

The slots are checked bit for bit against the oracle's conversion of the same
index rows (req_id[t] = t // s_q, fill -1, every column including the masked
tail), and out/lse bit for bit against dsv4_sparse_decode with the same
arguments (the same arithmetic, in a kernel that also writes the slots).
All paths of the entry point run: the conversion inside the short-split
kernel, inside the pipelined kernel (at most 1024 index columns a split), and
a conversion launch before the pipelined kernel (more columns a split).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, make_workload

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _run(w, S, idx_pad=0, expect_kernel=None, flags=0):
    """Decodes w with slots and without; returns (slots, (out, lse) with
    slots, (out, lse) without, plan), out as int16 bits, the slots from a
    buffer prefilled with a sentinel."""
    gh = _gh()
    dw = gh.DeviceWorkload(w)
    Kt = w.Kt
    idx_host = w.topk_idx
    if idx_pad:
        junk = np.full((w.B, idx_pad), 7, dtype=np.int32)
        idx_host = np.concatenate([w.topk_idx, junk], axis=1)
    idx = torch.from_numpy(np.ascontiguousarray(idx_host)).cuda()
    kw = dict(batch=w.B, num_heads=w.H, topk=w.topk, swa=w.swa, block_size=w.block_size,
              num_blocks=w.num_blocks, page_stride=w.page_stride, sm_scale=w.sm_scale,
              max_blocks_per_seq=w.max_blocks_per_seq,
              block_table_stride=w.block_table.shape[1], topk_idx_stride=Kt + idx_pad,
              tokens_per_seq=w.s_q, flags=flags)
    plan = dsv4.dsv4_sparse_decode_plan(dsv4.make_desc(**kw), S)
    if expect_kernel is not None:
        assert plan.partial_kernel == expect_kernel
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    desc = dsv4.make_desc(workspace=ws, **kw)
    slots = torch.full((w.B, Kt), SENTINEL, dtype=torch.int32, device="cuda")
    outs = []
    for with_slots in (True, False):
        out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        if with_slots:
            dsv4.dsv4_sparse_decode_with_slots(desc, dw.q, dw.kv, dw.bt, idx, dw.vl, dw.sink,
                                               out, lse, S, slots)
        else:
            dsv4.dsv4_sparse_decode(desc, dw.q, dw.kv, dw.bt, idx, dw.vl, dw.sink, out, lse, S)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    return slots.cpu().numpy(), outs[0], outs[1], plan


def _want_slots(w):
    req = (np.arange(w.B) // w.s_q).astype(np.int32)
    return oracle.convert_req_index_to_global(
        token_indices=w.topk_idx, block_table=w.block_table,
        max_blocks_per_req=w.max_blocks_per_seq, block_size=w.block_size, width=w.Kt,
        req_id=req, num_reqs=w.block_table.shape[0], invalid_fill=-1)


def _check(w, S, what, idx_pad=0, expect_kernel=None, flags=0):
    print(f"with_slots {what} S={S}", flush=True)
    slots, (o1, l1), (o2, l2), plan = _run(w, S, idx_pad, expect_kernel, flags)
    want = _want_slots(w)
    assert not (slots == SENTINEL).any(), f"{what}: unwritten slots"
    assert np.array_equal(slots, want), f"{what}: {(slots != want).sum()} slots differ"
    assert np.array_equal(o1, o2), f"{what}: out differs from dsv4_sparse_decode"
    assert np.array_equal(l1.view(np.int32), l2.view(np.int32)), f"{what}: lse differs"
    return plan, o1, l1


@pytest.mark.parametrize("ci,kernel", [(0, 1), (1, 1), (2, 1), (3, 0), (4, 0)])
def test_workloads_at_the_selector_plan(ci, kernel):
    """All five workloads: the short-split kernel for the first three, the
    pipelined kernel for the large batch and the ragged batch (whose masked
    tails are converted too), each writing the slots itself."""
    w = make_workload(ci)
    _check(w, w.num_splits, w.name, expect_kernel=kernel)


@pytest.mark.parametrize("ci,S", [(2, 1), (4, 2)])
def test_conversion_launch_when_a_split_has_over_1024_columns(ci, S):
    """The pipelined kernel writes the slots itself for at most 1024 index
    columns a split; past that (one split over 2048 columns, two over 2176)
    a conversion launch precedes the decode."""
    w = make_workload(ci)
    assert (w.Kt + S - 1) // S > 1024
    _check(w, S, f"{w.name} S={S} (conversion launch)", expect_kernel=dsv4.DSV4_KERNEL_PIPELINED)


@pytest.mark.parametrize("ci,S", [(1, 8), (1, 5), (2, 16), (2, 64), (0, 1)])
def test_forced_splits_in_the_short_kernel(ci, S):
    """Column ranges per split of several sizes, ragged last range."""
    w = make_workload(ci)
    _check(w, S, f"{w.name} S={S}", expect_kernel=dsv4.DSV4_KERNEL_SHORT)


@pytest.mark.parametrize("H,S", [(16, 4), (32, 3), (64, 5), (128, 4)])
def test_masked_tail_and_head_groups(H, S):
    """valid_len below topk: the conversion still covers columns
    [valid_len, topk); only head group 0 writes, every group decodes."""
    w = make_custom(B=3, H=H, topk=256, swa=64, seq_lens=[3000, 900, 200], seed=300 + H,
                    invalid_frac=0.05, valid_len_range=(40, 256))
    plan, o, l = _check(w, S, f"tail H={H}", expect_kernel=dsv4.DSV4_KERNEL_SHORT)
    gh = _gh()
    ro, rl, _ = oracle.decode_workload(w, num_splits=S)
    out = o.view(np.uint16).astype(np.uint32) << 16
    gh.assert_decode_close(out.view(np.float32).astype(np.float64), l.astype(np.float64), ro, rl,
                           f"tail H={H}")


@pytest.mark.parametrize("s_q,S", [(2, 3), (3, 4)])
@pytest.mark.parametrize("kernel", [1, 0])
def test_multi_token_rows_read_their_sequence(s_q, S, kernel):
    """Token t reads table row t // s_q, in the short-split kernel's own
    conversion and in the conversion launch before the pipelined kernel."""
    w = make_custom(B=3, H=64, topk=256, swa=64, seq_lens=[4000, 700, 300], seed=410 + s_q,
                    invalid_frac=0.03, valid_len_range=(100, 256), s_q=s_q)
    flags = 0 if kernel == dsv4.DSV4_KERNEL_SHORT else dsv4.DSV4_DECODE_PIPELINED
    _check(w, S, f"s_q={s_q} kernel={kernel}", expect_kernel=kernel, flags=flags)


@pytest.mark.parametrize("S,kernel", [(4, 1), (1, 1), (4, 0)])
def test_bad_entries_and_index_stride(S, kernel):
    """Negative indices, blocks past the table, negative and huge page
    entries (a slot past INT32_MAX, a page past the pool that the decode
    masks but the conversion still converts), and index rows with a stride
    beyond topk + swa whose extra columns hold junk."""
    w = make_custom(B=2, H=16, topk=96, swa=32, seq_lens=[700, 400], seed=77, block_size=4,
                    invalid_frac=0.1)
    bt = w.block_table.copy()
    idx = w.topk_idx.copy()
    bt[0, 1] = -3                      # negative page entry
    bt[0, 2] = 1 << 28                 # slot fits in int32, page past the pool
    bt[1, 0] = 1 << 30                 # slot past INT32_MAX
    idx[0, :4] = [4, 8, 9, 5]          # blocks 1, 2, 2, 1
    idx[1, :3] = [0, 2, 3]             # block 0
    idx[0, 10] = -7
    idx[1, 11] = w.max_blocks_per_seq * 4 + 1   # block past the table
    w = dataclasses.replace(w, block_table=bt, topk_idx=idx)
    flags = 0 if kernel == dsv4.DSV4_KERNEL_SHORT else dsv4.DSV4_DECODE_PIPELINED
    plan, o, l = _check(w, S, f"bad entries kernel={kernel}", idx_pad=5, expect_kernel=kernel,
                        flags=flags)
    want = _want_slots(w)
    assert want[0, 0] == -1 and want[0, 2] == (1 << 28) * 4 + 1 and want[1, 0] == -1
