"""Sparse FP8 MLA decode on the GPU against the fp64 oracle.

Every comparison is element by element on the whole output: |d out| <=
2e-2 + 1e-2 |out_ref| on the bf16 output and |d lse| <= 1e-3, infinities
equal.  The five workloads run at full size in the launch configuration the
benchmark uses (the selector's split count), plus forced split counts and
edge cases on smaller shapes that still span several tiles and a ragged
tail.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_custom, make_workload, poison_rows
import sparse_mla_attention_block_amd as dsv4

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _ref(w, **kw):
    out, lse, _ = oracle.decode_workload(w, **kw)
    return out, lse


def _check(w, what, **gpu_kw):
    gh = _gh()
    print(f"decode {what}: B={w.B} H={w.H} topk={w.topk} swa={w.swa} bs={w.block_size} "
          f"S={gpu_kw.get('num_splits', w.num_splits)}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, **gpu_kw)
    ro, rl = _ref(w)
    gh.assert_decode_close(out, lse, ro, rl, what)
    return dw, out, lse, ro, rl


@pytest.mark.parametrize("ci", range(5))
def test_workload_full_size(ci):
    """At the benchmark's plan: the selector's split count, with the split
    count chosen per row (balanced splits) where the configuration asks for
    it (the ragged batch)."""
    w = make_workload(ci)
    flags = dsv4.DSV4_DECODE_BALANCE if w.per_row_splits else 0
    _check(w, f"workload {ci} {w.name}", flags=flags)


def test_ragged_workload_with_uniform_splits():
    """The ragged batch at the selector's uniform plan as well."""
    w = make_workload(4)
    assert w.per_row_splits
    _check(w, "workload 4 ragged, uniform splits")


@pytest.mark.parametrize("S", [4, 2, 3])
def test_short_batch_at_the_short_work_cap(S):
    """The short-context batch (B=4, H=64, 512 + 128 entries) at the split
    counts the pages' short-work cap of 4 allows (vLLM PR #52212 page,
    implementation item 2), at full size; the selector itself picks more
    splits for this shape."""
    w = make_workload(1)
    _check(w, f"short_batch S={S}", num_splits=S)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 32, 64])
def test_forced_split_counts(S):
    w = make_custom(B=3, H=64, topk=300, swa=37, seq_lens=[5000, 400, 90], seed=10 + S,
                    invalid_frac=0.03, valid_len_range=(150, 300))
    _check(w, f"S={S}", num_splits=S)


@pytest.mark.parametrize("H", [16, 32, 48, 64, 96, 128])
def test_head_counts(H):
    w = make_custom(B=2, H=H, topk=200, swa=20, seq_lens=[3000, 700], seed=20 + H,
                    invalid_frac=0.05, valid_len_range=(100, 200))
    _check(w, f"H={H}", num_splits=0)
    _check(w, f"H={H} S=1", num_splits=1)


@pytest.mark.parametrize("H,hg", [(32, 32), (48, 48), (64, 64), (80, 16), (96, 48), (128, 64)])
def test_every_head_group_variant(H, hg):
    """A batch of 256 tokens keeps the largest head group, so each kernel
    variant (16, 32, 48, 64 heads per workgroup) runs on a full-size grid."""
    import sparse_mla_attention_block_amd as dsv4
    rng = np.random.default_rng(40 + H)
    w = make_custom(B=256, H=H, topk=48, swa=16, seq_lens=list(rng.integers(64, 400, 256)),
                    seed=40 + H, invalid_frac=0.05, valid_len_range=(20, 48))
    plan = dsv4.dsv4_sparse_decode_plan(_gh().make_desc(w), 0)
    assert (plan.heads_per_group, plan.num_splits) == (hg, 1)
    _check(w, f"H={H} hg={hg}", num_splits=0)


@pytest.mark.parametrize("bs,pad", [(1, 0), (1, 8), (16, 0), (64, 64)])
def test_block_sizes_and_page_strides(bs, pad):
    w = make_custom(B=2, H=64, topk=150, swa=16, seq_lens=[2000, 321], seed=30 + bs + pad,
                    block_size=bs, page_pad=pad, invalid_frac=0.04)
    _check(w, f"bs={bs} pad={pad}", num_splits=3)


def test_without_sink_and_without_lse():
    gh = _gh()
    w = make_custom(B=2, H=32, topk=100, swa=0, seq_lens=[900, 900], seed=41, with_sink=False,
                    invalid_frac=0.1)
    for S in (1, 4):
        _check(w, f"no sink S={S}", num_splits=S)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=4, want_lse=False)
    assert np.isnan(lse).all()                       # lse = NULL: never written
    ro, _ = _ref(w)
    assert np.all(np.abs(out - ro) <= gh.OUT_ATOL + gh.OUT_RTOL * np.abs(ro))


@pytest.mark.parametrize("S", [1, 5])
@pytest.mark.parametrize("with_sink", [True, False])
def test_empty_and_all_invalid_rows(S, with_sink):
    gh = _gh()
    w = make_custom(B=4, H=16, topk=64, swa=8, seq_lens=[500, 500, 500, 500], seed=50,
                    with_sink=with_sink, valid_len_range=(0, 64))
    w.topk_idx[0, :] = -1                            # nothing at all
    w.topk_idx[1, :64] = -1                          # SWA only
    w.valid_len[2] = 0                               # main masked by valid_len
    w.valid_len[3] = -7                              # clamps to 0
    dw, out, lse, ro, rl = _check(w, f"empty rows S={S} sink={with_sink}", num_splits=S)
    assert np.all(out[0] == 0.0)
    if with_sink:
        assert np.allclose(lse[0], w.sink, atol=1e-6)
    else:
        assert np.all(np.isneginf(lse[0]))


def test_valid_len_beyond_topk_and_null():
    gh = _gh()
    w = make_custom(B=2, H=64, topk=100, swa=30, seq_lens=[800, 800], seed=60,
                    valid_len_range=(0, 1))
    w.valid_len[:] = [500, 100]                      # both mean "no masking"
    dw, out, lse, _, _ = _check(w, "valid_len >= topk", num_splits=2)
    out2, lse2 = gh.gpu_decode(dw, num_splits=2, valid_len=None)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("scale", [8.0, 30.0])
def test_large_logits_rescale_stably(scale):
    w = make_custom(B=1, H=64, topk=512, swa=0, seq_lens=[4096], seed=70, invalid_frac=0.02)
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).float() * scale
    w.q = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for S in (1, 8):
        _check(w, f"q x{scale} S={S}", num_splits=S)


@pytest.mark.parametrize("sink_value", [25.0, -25.0])
def test_dominant_or_negligible_sink(sink_value):
    w = make_custom(B=2, H=64, topk=128, swa=0, seq_lens=[2000, 2000], seed=80)
    w.sink[:] = sink_value
    for S in (1, 4):
        _check(w, f"sink={sink_value} S={S}", num_splits=S)


def test_duplicates_count_twice():
    w = make_custom(B=2, H=64, topk=96, swa=32, seq_lens=[3000, 96], seed=90)
    w.topk_idx[0, 10:20] = w.topk_idx[0, 0]
    _check(w, "duplicates", num_splits=3)


def test_poisoned_rows_are_never_read_bitwise():
    """Masked-tail entries re-pointed at 0xFF rows or past the block table
    give bit-identical output to the clean run."""
    gh = _gh()
    w = make_custom(B=2, H=64, topk=256, swa=64, seq_lens=[6000, 3000], seed=100,
                    invalid_frac=0.05, valid_len_range=(120, 200))
    dw = gh.DeviceWorkload(w)
    for S in (1, 4):
        clean = gh.gpu_decode(dw, num_splits=S)
        ti = w.topk_idx.copy()
        for b in range(w.B):
            used = set(int(x) for x in ti[b] if x >= 0)
            free = [s for s in range(int(w.seq_lens[b])) if s not in used]
            vl = int(w.valid_len[b])
            for k in range(vl, w.topk):
                ti[b, k] = free.pop() if k % 3 else w.max_blocks_per_seq * w.block_size + k
        dirty = gh.gpu_decode(dw, num_splits=S, topk_idx=torch.from_numpy(ti).cuda())
        assert np.array_equal(clean[0], dirty[0]) and np.array_equal(clean[1], dirty[1])


def _used_slots(w, b, n):
    vl = w.topk if w.valid_len is None else int(w.valid_len[b])
    return [int(x) for x in w.topk_idx[b, :vl] if x >= 0][:n]


@pytest.mark.parametrize("S", [1, 4])
def test_scrub_reads_non_finite_elements_as_zero(S):
    """With the scrub flag, a pool holding FP8 NaN bytes, a NaN scale code and
    NaN/-inf RoPE values in taking-part rows gives bit for bit what the pool
    with those elements encoded as finite zeros gives without it, and
    matches the oracle's scrub mode."""
    gh = _gh()
    w = make_custom(B=3, H=64, topk=256, swa=64, seq_lens=[5000, 700, 3000], seed=130,
                    invalid_frac=0.03, valid_len_range=(150, 256))
    pair = None
    for b in range(w.B):
        pair = poison_rows(w, b, _used_slots(w, b, 6), seed=131 + b, base=pair)
    kv_p, kv_c = pair
    w.kv = kv_c
    dw = gh.DeviceWorkload(w)
    kv_pd = torch.from_numpy(kv_p).cuda()
    print(f"scrub S={S}", flush=True)
    clean = gh.gpu_decode(dw, num_splits=S)
    scrubbed = gh.gpu_decode(dw, num_splits=S, kv=kv_pd, flags=dsv4.DSV4_DECODE_SCRUB)
    assert np.array_equal(clean[0], scrubbed[0]) and np.array_equal(clean[1], scrubbed[1])
    also = gh.gpu_decode(dw, num_splits=S, flags=dsv4.DSV4_DECODE_SCRUB)
    assert np.array_equal(clean[0], also[0]) and np.array_equal(clean[1], also[1])
    w.kv = kv_p
    ro, rl, _ = oracle.decode_workload(w, num_splits=S, scrub=True)
    gh.assert_decode_close(scrubbed[0], scrubbed[1], ro, rl, "scrub vs oracle")


def test_deterministic_bitwise():
    gh = _gh()
    w = make_workload(1)
    dw = gh.DeviceWorkload(w)
    a = gh.gpu_decode(dw)
    b = gh.gpu_decode(dw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_stage_entry_points_match_the_fused_call():
    gh = _gh()
    w = make_workload(2)
    dw = gh.DeviceWorkload(w)
    a = gh.gpu_decode(dw)
    b = gh.gpu_decode(dw, partial_then_combine=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_global_slots_after_conversion_match_block_table_path():
    """convert (fill -1) then decode without a table == decode with the table."""
    gh = _gh()
    import sparse_mla_attention_block_amd as dsv4
    w = make_workload(4)
    dw = gh.DeviceWorkload(w)
    a = gh.gpu_decode(dw)
    gslots = torch.empty_like(dw.idx)
    dsv4.dsv4_convert_req_index_to_global(None, w.B, dw.bt, w.block_table.shape[1],
                                          w.max_blocks_per_seq, dw.idx, w.Kt, w.B, w.Kt,
                                          w.block_size, None, -1, gslots)
    b = gh.gpu_decode(dw, use_bt=False, topk_idx=gslots)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_side_stream_and_no_overrun():
    """Runs on a non-default stream; guard bytes around out/lse stay intact."""
    import sparse_mla_attention_block_amd as dsv4
    gh = _gh()
    w = make_custom(B=3, H=64, topk=200, swa=10, seq_lens=[1000, 1000, 1000], seed=110)
    dw = gh.DeviceWorkload(w)
    S = 3
    desc = gh.make_desc(w)
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    guard = 4096
    ws_full = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = ws_full[guard:guard + nbytes]
    desc = gh.make_desc(w, workspace=ws)
    n = w.B * w.H * 512
    out_full = torch.full((n + 2 * 2048,), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_full = torch.full((w.B * w.H + 2 * 256,), 7.0, dtype=torch.float32, device="cuda")
    out = out_full[2048:2048 + n].view(w.B, w.H, 512)
    lse = lse_full[256:256 + w.B * w.H].view(w.B, w.H)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        dsv4.dsv4_sparse_decode(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out, lse, S, st)
    st.synchronize()
    assert torch.all(out_full[:2048] == 7.0) and torch.all(out_full[2048 + n:] == 7.0)
    assert torch.all(lse_full[:256] == 7.0) and torch.all(lse_full[256 + w.B * w.H:] == 7.0)
    assert torch.all(ws_full[:guard] == 0x5A) and torch.all(ws_full[guard + nbytes:] == 0x5A)
    ro, rl = _ref(w)
    gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(), ro,
                           rl, "side stream")


def test_gather_floor_loads_exactly_the_taking_part_rows():
    """The gather floor folds every word of every taking-part row once per head
    group; with one head group the XOR over all its output words equals the
    XOR of those rows' 576 data bytes and 8 scale bytes, read on the host."""
    import sparse_mla_attention_block_amd as dsv4
    gh = _gh()
    w = make_custom(B=3, H=16, topk=300, swa=20, seq_lens=[4000, 900, 64], seed=61,
                    invalid_frac=0.1, valid_len_range=(100, 300))
    dw = gh.DeviceWorkload(w)
    desc = gh.make_desc(w)
    plan = dsv4.dsv4_sparse_decode_plan(desc, 3)
    assert plan.head_groups == 1
    words = torch.full((plan.grid_partial * plan.block_partial,), -1, dtype=torch.int32,
                       device="cuda")
    print("gather floor: B=3 H=16 S=3", flush=True)
    dsv4.dsv4_gather_floor(desc, dw.kv, dw.bt, dw.idx, dw.vl, 3, words)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32))
    want = np.uint32(0)
    kv = w.kv
    for b in range(w.B):
        vl = min(max(int(w.valid_len[b]), 0), w.topk)
        cols = list(range(vl)) + list(range(w.topk, w.topk + w.swa))
        for c in cols:
            i = int(w.topk_idx[b, c])
            if i < 0 or i // w.block_size >= w.max_blocks_per_seq:
                continue
            pg = int(w.block_table[b, i // w.block_size])
            if pg < 0 or pg >= w.num_blocks:
                continue
            off = i % w.block_size
            data = kv[pg, off * 576:(off + 1) * 576]
            sc = kv[pg, w.block_size * 576 + off * 8: w.block_size * 576 + off * 8 + 8]
            want ^= np.bitwise_xor.reduce(np.concatenate([data, sc]).view(np.uint32))
    assert got == want


@pytest.mark.parametrize("S", [1, 3])
def test_very_long_index_list(S):
    """16384 main entries: at S = 1 one workgroup walks 512 tiles, so the
    32-tile resolution ring is refilled 30 times."""
    w = make_custom(B=1, H=16, topk=16384, swa=64, seq_lens=[200000], seed=210 + S,
                    invalid_frac=0.01)
    _check(w, f"topk=16384 S={S}", num_splits=S)


def test_many_tokens_with_short_lists():
    rng = np.random.default_rng(220)
    w = make_custom(B=2048, H=16, topk=32, swa=8, seq_lens=list(rng.integers(20, 200, 2048)),
                    seed=220, invalid_frac=0.1, valid_len_range=(0, 32))
    _check(w, "B=2048 short lists", num_splits=0)


def test_block_size_128():
    w = make_custom(B=3, H=32, topk=400, swa=40, seq_lens=[7000, 1300, 129], seed=230,
                    block_size=128, invalid_frac=0.02, valid_len_range=(200, 400))
    _check(w, "bs=128", num_splits=0)
    _check(w, "bs=128 S=5", num_splits=5)


def test_multi_token_over_global_slots():
    """Without a block table the s_q tokens of a sequence still share its
    top-k length."""
    gh = _gh()
    w = make_custom(B=3, H=32, topk=128, swa=16, seq_lens=[3000, 800, 300], seed=240, s_q=3,
                    valid_len_range=(40, 128))
    slots = np.where(w.topk_idx >= 0,
                     w.block_table[np.arange(w.B)[:, None] // 3, np.maximum(w.topk_idx, 0)
                                   // w.block_size] * w.block_size
                     + np.maximum(w.topk_idx, 0) % w.block_size, -1).astype(np.int32)
    dw = gh.DeviceWorkload(w)
    print("multi-token global slots", flush=True)
    out, lse = gh.gpu_decode(dw, num_splits=2, use_bt=False, topk_idx=torch.from_numpy(slots).cuda())
    ro, rl, _ = oracle.decode_workload(w, topk_idx=slots, use_block_table=False, num_splits=2)
    gh.assert_decode_close(out, lse, ro, rl, "multi-token global slots")
    ro2, rl2, _ = oracle.decode_workload(w, num_splits=2)
    gh.assert_decode_close(out, lse, ro2, rl2, "multi-token global slots vs block table")


def _merge_fp64(part_out, part_lse, sink):
    """The split merge as the C ABI defines it (log-sum-exp with the sink),
    in fp64 over the bf16 partials as given; empty splits (lse = -inf) drop
    out whatever their partial rows hold."""
    B, H, S, _ = part_out.shape
    out = np.zeros((B, H, 512))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            ls = part_lse[b, h]
            live = ~np.isneginf(ls)
            sk = -np.inf if sink is None else float(sink[h])
            M = max(ls[live].max() if live.any() else -np.inf, sk)
            if M == -np.inf:
                continue
            wts = np.exp(ls[live] - M)
            D = wts.sum() + (np.exp(sk - M) if sk != -np.inf else 0.0)
            out[b, h] = (wts[:, None] * part_out[b, h][live]).sum(0) / D
            lse[b, h] = M + np.log(D)
    return out, lse


# One (token, head) count per combine launch shape: 4 dim slices (<= 128
# rows), 2 slices (< 2048 rows), one workgroup per row (>= 2048 rows).
@pytest.mark.parametrize("B,H", [(1, 64), (3, 64), (32, 64)])
@pytest.mark.parametrize("S", [1, 2, 3, 5, 32, 64, 100])
@pytest.mark.parametrize("with_sink", [True, False])
def test_combine_launch_shapes_and_empty_split_contents(B, H, S, with_sink):
    print(f"combine B={B} H={H} S={S} sink={with_sink}", flush=True)
    rng = np.random.default_rng(500 + B + S)
    po = rng.standard_normal((B, H, S, 512)).astype(np.float32)
    pl = (3.0 * rng.standard_normal((B, H, S))).astype(np.float32)
    pl[rng.random((B, H, S)) < 0.2] = -np.inf          # empty splits
    pl[0, 1, :] = -np.inf                              # a row with every split empty
    sink = rng.standard_normal(H).astype(np.float32) if with_sink else None
    po_bf = torch.from_numpy(po).to(torch.bfloat16)
    exact = po_bf.double().numpy()
    ref_out, ref_lse = _merge_fp64(exact, pl.astype(np.float64), sink)
    sk = None if sink is None else torch.from_numpy(sink).cuda()
    runs = []
    for poison in (False, True):
        p = po_bf.clone()
        if poison:                                     # empty splits' rows hold NaN
            p[torch.from_numpy(np.isneginf(pl))] = float("nan")
        out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        dsv4.dsv4_combine_splits(B, H, S, p.cuda(), torch.from_numpy(pl).cuda(), sk, out, lse,
                                 None)
        torch.cuda.synchronize()
        runs.append((out.cpu(), lse.cpu()))
    gh = _gh()
    gh.assert_decode_close(runs[0][0].double().numpy(), runs[0][1].double().numpy(),
                           ref_out, ref_lse, f"combine B={B} H={H} S={S}")
    assert torch.equal(runs[0][0].view(torch.int16), runs[1][0].view(torch.int16))
    assert torch.equal(runs[0][1], runs[1][1])
    assert np.all(runs[0][0][0, 1].float().numpy() == 0.0)
    assert runs[0][1][0, 1].item() == (float(sink[1]) if with_sink else -np.inf)
