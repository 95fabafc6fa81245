"""Dual-cache decode on the GPU: SWA entries resolve in a second pool with
its own pages, block table and block size (rows that only SWA entries name
are poison in the first pool).  Compared with the oracle to the decode
tolerance (|d out| <= 2e-2 + 1e-2 |out_ref|, |d lse| <= 1e-3), and bitwise
with the single-pool decode of the workload the pools were split from, run
on the same (pipelined) partial kernel: dual-pool decodes always use it,
while a single pool with short splits would otherwise take the short-split
kernel, whose rounding differs."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, make_workload, split_swa_pool

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _dual(w, S, *, global_slots=False, idx=None):
    gh = _gh()
    sp = w.swa_pool
    kv1 = torch.from_numpy(w.kv).cuda()
    kv2 = torch.from_numpy(sp["kv"]).cuda()
    bt1 = None if global_slots else torch.from_numpy(w.block_table).cuda()
    bt2 = None if global_slots else torch.from_numpy(sp["block_table"]).cuda()
    main = dsv4.make_pool(kv1, bt1, block_size=w.block_size, max_blocks_per_seq=w.max_blocks_per_seq)
    swa = dsv4.make_pool(kv2, bt2, block_size=sp["block_size"],
                         max_blocks_per_seq=sp["max_blocks_per_seq"])
    desc = gh.make_desc(w)
    n = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws)
    q = torch.from_numpy(w.q.view(np.int16)).cuda().view(torch.bfloat16)
    ti = torch.from_numpy(w.topk_idx if idx is None else idx).cuda()
    vl = torch.from_numpy(w.valid_len).cuda() if w.valid_len is not None else None
    sink = torch.from_numpy(w.sink).cuda() if w.sink is not None else None
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_decode_dual(desc, q, main, swa, ti, vl, sink, out, lse, S)
    torch.cuda.synchronize()
    return out.float().double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("bs2,S", [(16, 1), (16, 4), (1, 3), (64, 0), (128, 2)])
def test_dual_cache_matches_oracle_and_single_pool(bs2, S):
    gh = _gh()
    w = make_custom(B=3, H=64, topk=256, swa=96, seq_lens=[6000, 1500, 300], seed=250 + bs2,
                    invalid_frac=0.03, valid_len_range=(100, 256))
    w2 = split_swa_pool(w, block_size=bs2, seed=251, page_pad=8 * (bs2 % 3))
    print(f"dual cache bs2={bs2} S={S}", flush=True)
    out, lse = _dual(w2, S)
    ro, rl, _ = oracle.decode_workload(w2, num_splits=S)
    gh.assert_decode_close(out, lse, ro, rl, f"dual bs2={bs2} S={S}")
    single = gh.gpu_decode(gh.DeviceWorkload(w), num_splits=S, flags=dsv4.DSV4_DECODE_PIPELINED)
    assert np.array_equal(out, single[0]) and np.array_equal(lse, single[1])


def test_dual_cache_multi_token():
    gh = _gh()
    w = split_swa_pool(make_custom(B=2, H=32, topk=128, swa=64, seq_lens=[2000, 700], seed=260,
                                   s_q=2, valid_len_range=(60, 128)), block_size=32, seed=261)
    out, lse = _dual(w, 2)
    ro, rl, _ = oracle.decode_workload(w, num_splits=2)
    gh.assert_decode_close(out, lse, ro, rl, "dual multi-token")


def test_dual_cache_over_global_slots():
    """Without block tables: main indices are slots of the first pool, SWA
    indices slots of the second."""
    gh = _gh()
    w = split_swa_pool(make_custom(B=2, H=32, topk=128, swa=32, seq_lens=[3000, 900], seed=270,
                                   valid_len_range=(64, 128)), block_size=16, seed=271)
    sp = w.swa_pool
    idx = w.topk_idx.copy()
    for b in range(w.B):
        for k in range(idx.shape[1]):
            i = int(w.topk_idx[b, k])
            if i < 0:
                continue
            bt, bs = (w.block_table, w.block_size) if k < w.topk else (sp["block_table"],
                                                                      sp["block_size"])
            idx[b, k] = int(bt[b, i // bs]) * bs + i % bs
    out, lse = _dual(w, 2, global_slots=True, idx=idx)
    ro, rl, _ = oracle.decode_workload(w, num_splits=2)
    gh.assert_decode_close(out, lse, ro, rl, "dual global slots")


def test_dual_cache_at_full_size():
    """The ragged workload (32 tokens, H=128, top-k 2048 + SWA 128) with its
    SWA rows in a block-16 pool, in the selector's launch configuration."""
    gh = _gh()
    w = split_swa_pool(make_workload(4), block_size=16, seed=280)
    print("dual cache full size", flush=True)
    out, lse = _dual(w, 0)
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, "dual full size")
