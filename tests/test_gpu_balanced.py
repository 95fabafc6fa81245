"""Balanced splits (DSV4_DECODE_BALANCE) on the GPU: the pipelined kernel
gives each token a split count that follows its length, read from valid_len
at run time.  Every case is compared with the fp64 oracle to the decode
tolerance (|d out| <= 2e-2 + 1e-2 |out_ref|, |d lse| <= 1e-3, infinities
equal).  The split counts themselves are pinned through the partials: slot s
of token b's row holds lse = -inf exactly when s >= n_b, with n_b computed
here from the rule the header states (the fewest tiles per split T whose
counts n_b = max(1, ceil(eff_b / 32T)) fit the budget B*S and the slots).
"""

import math

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


def expected_counts(w, budget, slots):
    """n_b per query token by the header's rule (host mirror for the check)."""
    vl = (np.full(w.B // w.s_q, w.topk) if w.valid_len is None
          else np.clip(w.valid_len.astype(np.int64), 0, w.topk))
    eff = np.repeat(vl, w.s_q) + w.swa
    kt = w.topk + w.swa
    lo = max(1, math.ceil(eff.max() / (32 * slots)))
    hi = math.ceil(math.ceil(kt / budget) / 32)
    for T in range(lo, hi + 1):
        n = np.maximum(1, -(-eff // (32 * T)))
        if n.sum() <= w.B * budget:
            return n, T
    raise AssertionError("no tile count fits the budget")


def _partials(dw, S, flags):
    """Runs the first stage alone; returns (plan, part_lse [B, H, slots])."""
    gh = _gh()
    w = dw.w
    desc = gh.make_desc(w, flags=flags)
    plan = dsv4.dsv4_sparse_decode_plan(desc, S)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws, flags=flags)
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws.fill_(0x7F)                       # NaN-free garbage: every slot must be written
    dsv4.dsv4_sparse_decode_partial(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out, lse, S)
    torch.cuda.synchronize()
    _, pl = dsv4.workspace_split_views(ws, w.B, w.H, plan.num_splits)
    return plan, pl.double().cpu().numpy()


def _check_slots(w, plan, pl):
    n, _ = expected_counts(w, plan.balanced_splits, plan.num_splits)
    for b in range(w.B):
        assert np.all(np.isneginf(pl[b, :, n[b]:])), f"token {b}: slots past n_b={n[b]} not empty"
        assert not np.isnan(pl[b, :, :n[b]]).any()
        assert np.all(np.isfinite(pl[b, :, :n[b]]) | np.isneginf(pl[b, :, :n[b]]))
    return n


def _balanced_case(w, S, extra_flags=0, expect_on=True):
    gh = _gh()
    flags = dsv4.DSV4_DECODE_BALANCE | extra_flags
    dw = gh.DeviceWorkload(w)
    plan = dsv4.dsv4_sparse_decode_plan(gh.make_desc(w, flags=flags), S)
    uni = dsv4.dsv4_sparse_decode_plan(gh.make_desc(w, flags=extra_flags), S)
    print(f"balanced B={w.B} H={w.H} Kt={w.Kt} S={S} plan slots={plan.num_splits} "
          f"budget={plan.balanced_splits}", flush=True)
    if expect_on:
        assert plan.balanced_splits == uni.num_splits >= 2
        assert plan.num_splits == min(64, uni.num_splits + -(-uni.num_splits // 4))
        assert plan.grid_partial == uni.grid_partial
    else:
        assert plan.balanced_splits == 0 and plan.num_splits == uni.num_splits
    out, lse = gh.gpu_decode(dw, num_splits=S, flags=flags)
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, "balanced decode")
    out2, lse2 = gh.gpu_decode(dw, num_splits=S, flags=flags, partial_then_combine=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "two-stage form differs"
    n = None
    if expect_on:
        plan_p, pl = _partials(dw, S, flags)
        n = _check_slots(w, plan_p, pl)
    return dw, plan, n


def test_ragged_workload_balanced():
    """The ragged batch (32 tokens, H = 128, valid lengths 1078-2041 + 128
    SWA): longer tokens take more splits than the budget, shorter fewer."""
    w = make_workload(4)
    _, plan, n = _balanced_case(w, 0)
    assert n.max() > plan.balanced_splits > n.min()
    _, T = expected_counts(w, plan.balanced_splits, plan.num_splits)
    uniform_tiles = math.ceil(math.ceil((w.valid_len.max() + w.swa) / plan.balanced_splits) / 32)
    assert T < uniform_tiles, (T, uniform_tiles)


@pytest.mark.parametrize("B,H,topk,swa,S,vl", [
    (6, 64, 512, 64, 4, [0, 512, 100, 31, 400, 257]),     # empty main list, full, short
    (3, 128, 1024, 0, 0, [1024, 40, 600]),               # selector's S, no SWA
    (5, 32, 384, 32, 7, [384, 384, 384, 384, 384]),      # equal lengths
    (2, 64, 256, 0, 2, [0, 0]),                          # nothing to attend
    (4, 64, 640, 32, 3, [-7, 100000, 320, 1]),           # lengths clamped to [0, topk]
])
def test_balanced_small_cases(B, H, topk, swa, S, vl):
    w = make_custom(B=B, H=H, topk=topk, swa=swa, seq_lens=[5000 + 321 * b for b in range(B)],
                    seed=1300 + B * H + S, invalid_frac=0.05)
    w.valid_len = np.asarray(vl, dtype=np.int32)
    _balanced_case(w, S, dsv4.DSV4_DECODE_PIPELINED)


def test_balanced_without_valid_len_is_uniform():
    """No valid_len: every token has topk + swa entries, so every token gets
    the budget's split count and the spare slot stays empty."""
    w = make_custom(B=4, H=64, topk=1024, swa=128, seq_lens=[9000, 8000, 7000, 6000], seed=1320,
                    invalid_frac=0.02)
    assert w.valid_len is None
    _, plan, n = _balanced_case(w, 4, dsv4.DSV4_DECODE_PIPELINED)
    assert np.all(n == 4)


def test_balanced_multi_token():
    """s_q = 2: the two query tokens of a sequence share its length."""
    w = make_custom(B=3, H=64, topk=512, swa=64, seq_lens=[6000, 3000, 900], seed=1330, s_q=2,
                    valid_len_range=(50, 512), invalid_frac=0.03)
    _, _, n = _balanced_case(w, 4, dsv4.DSV4_DECODE_PIPELINED)
    assert np.array_equal(n[0::2], n[1::2])


@pytest.mark.parametrize("B,on", [(64, True), (65, False)])
def test_balanced_batch_limit(B, on):
    """At most 64 tokens (one wave's lanes); past that the flag is ignored."""
    w = make_custom(B=B, H=16, topk=256, swa=0, seq_lens=[3000 + 7 * b for b in range(B)],
                    seed=1340 + B, valid_len_range=(1, 256))
    _balanced_case(w, 4, dsv4.DSV4_DECODE_PIPELINED, expect_on=on)


def test_balanced_ignored_on_short_kernel_plans():
    """The flag applies to the pipelined kernel only: a plan that picks the
    short-split kernel keeps uniform splits (and the same bytes)."""
    gh = _gh()
    w = make_custom(B=2, H=64, topk=256, swa=0, seq_lens=[4000, 2000], seed=1350,
                    valid_len_range=(10, 256))
    plan = dsv4.dsv4_sparse_decode_plan(gh.make_desc(w, flags=dsv4.DSV4_DECODE_BALANCE), 4)
    assert plan.partial_kernel == dsv4.DSV4_KERNEL_SHORT and plan.balanced_splits == 0
    dw = gh.DeviceWorkload(w)
    a = gh.gpu_decode(dw, num_splits=4, flags=dsv4.DSV4_DECODE_BALANCE)
    b = gh.gpu_decode(dw, num_splits=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_balanced_with_slots_and_determinism():
    """dsv4_sparse_decode_with_slots under the flag converts in a launch of
    its own; its output equals the plain balanced decode bit for bit, and
    two runs agree bit for bit."""
    gh = _gh()
    w = make_custom(B=4, H=64, topk=1024, swa=64, seq_lens=[8000, 5000, 3000, 2500], seed=1360,
                    valid_len_range=(100, 1024), invalid_frac=0.05)
    flags = dsv4.DSV4_DECODE_BALANCE | dsv4.DSV4_DECODE_PIPELINED
    dw = gh.DeviceWorkload(w)
    a = gh.gpu_decode(dw, num_splits=4, flags=flags)
    b = gh.gpu_decode(dw, num_splits=4, flags=flags)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    desc = gh.make_desc(w, flags=flags)
    n = dsv4.dsv4_sparse_decode_workspace_bytes(desc, 4)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws, flags=flags)
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    slots = torch.full((w.B, w.Kt), -7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_sparse_decode_with_slots(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out, lse,
                                       4, slots)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().double().cpu().numpy(), a[0])
    assert np.array_equal(lse.double().cpu().numpy(), a[1])
    want = oracle.convert_req_index_to_global(
        token_indices=w.topk_idx, block_table=w.block_table,
        max_blocks_per_req=w.max_blocks_per_seq, block_size=w.block_size, invalid_fill=-1)
    assert np.array_equal(slots.cpu().numpy(), want)


def test_balanced_dual_pool():
    """SWA entries in a second pool: the pool of an entry still follows its
    position in the token's effective list."""
    gh = _gh()
    w = make_custom(B=3, H=64, topk=512, swa=96, seq_lens=[6000, 1500, 700], seed=1370,
                    invalid_frac=0.03, valid_len_range=(30, 512))
    w2 = split_swa_pool(w, block_size=16, seed=1371)
    sp = w2.swa_pool
    flags = dsv4.DSV4_DECODE_BALANCE | dsv4.DSV4_DECODE_PIPELINED
    kv1, bt1 = torch.from_numpy(w2.kv).cuda(), torch.from_numpy(w2.block_table).cuda()
    kv2, bt2 = torch.from_numpy(sp["kv"]).cuda(), torch.from_numpy(sp["block_table"]).cuda()
    main = dsv4.make_pool(kv1, bt1, block_size=w2.block_size,
                          max_blocks_per_seq=w2.max_blocks_per_seq)
    swa = dsv4.make_pool(kv2, bt2, block_size=sp["block_size"],
                         max_blocks_per_seq=sp["max_blocks_per_seq"])
    desc = gh.make_desc(w2, flags=flags)
    plan = dsv4.dsv4_sparse_decode_plan(desc, 4)
    assert plan.balanced_splits == 4
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w2, workspace=ws, flags=flags)
    dw = gh.DeviceWorkload(w2)
    out = torch.full((w2.B, w2.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w2.B, w2.H), float("nan"), dtype=torch.float32, device="cuda")
    print("balanced dual pool", flush=True)
    dsv4.dsv4_sparse_decode_dual(desc, dw.q, main, swa, dw.idx, dw.vl, dw.sink, out, lse, 4)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.decode_workload(w2)
    gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl,
                           "balanced dual pool")
