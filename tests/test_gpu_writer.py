"""Cache writer on the GPU against the oracle: every byte of the pool after
a quantise-and-store must equal the oracle's (integer and byte work:
bit-exact), with and without sanitising, over rows whose groups span ~60
scale codes and include zeros, infinities, NaNs, subnormals, the bf16
maximum, exact E4M3FN ties and signed zeros."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, make_writer_rows

pytestmark = pytest.mark.gpu


def _gpu_store(kv, rows, slots, *, block_size, sanitize, row_stride=512):
    n = rows.shape[0]
    r = np.zeros((n, row_stride), dtype=np.uint16)
    r[:, :512] = rows
    rows_d = torch.from_numpy(r.view(np.int16)).cuda()
    slots_d = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    kv_d = torch.from_numpy(np.ascontiguousarray(kv)).cuda()
    dsv4.dsv4_quantize_store(rows_d, row_stride, slots_d, n, kv_d, block_size, kv.shape[0],
                             kv.shape[1], dsv4.DSV4_STORE_SANITIZE if sanitize else 0)
    torch.cuda.synchronize()
    return kv_d.cpu().numpy()


def _pool(bs, nb, pad, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(nb, bs * 584 + pad), dtype=np.uint8)


@pytest.mark.parametrize("sanitize", [True, False])
@pytest.mark.parametrize("bs,nb,pad,n", [(64, 24, 0, 1000), (16, 70, 8, 999), (1, 300, 16, 257)])
def test_pool_matches_the_oracle_bytewise(sanitize, bs, nb, pad, n):
    print(f"writer bs={bs} nb={nb} pad={pad} n={n} sanitize={sanitize}", flush=True)
    rng = np.random.default_rng(bs * 1000 + n)
    kv = _pool(bs, nb, pad, seed=n)
    rows = make_writer_rows(n, seed=n + bs)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[rng.random(n) < 0.05] = -1 - rng.integers(0, 1000, size=1)
    slots[rng.random(n) < 0.03] = nb * bs + rng.integers(0, 5000, size=1)
    got = _gpu_store(kv, rows, slots, block_size=bs, sanitize=sanitize)
    want = oracle.store_rows(kv, rows, slots, block_size=bs, sanitize=sanitize)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:5].tolist()}"


@pytest.mark.parametrize("sanitize", [True, False])
def test_every_bf16_value_in_every_position(sanitize):
    """All 65536 bf16 patterns, 63 to a group next to a 448, again next to a
    2^20 and again next to a 2^-20 (the group's code follows whichever
    magnitude is largest), and as RoPE values."""
    b = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    rows = []
    for lead in (0x43E0, 0x4980, 0x3580):
        k = 0
        while k < len(b):
            r = np.zeros(512, dtype=np.uint16)
            for g in range(7):
                r[64 * g] = lead
                chunk = b[k:k + 63]
                r[64 * g + 1:64 * g + 1 + len(chunk)] = chunk
                k += 63
            r[448:] = b[(k + np.arange(64)) % len(b)]
            rows.append(r)
    rows = np.stack(rows)
    n = rows.shape[0]
    bs = 64
    nb = -(-n // bs)
    kv = _pool(bs, nb, 0, seed=3)
    slots = np.arange(n, dtype=np.int64)
    print(f"writer exhaustive n={n} sanitize={sanitize}", flush=True)
    got = _gpu_store(kv, rows, slots, block_size=bs, sanitize=sanitize)
    want = oracle.store_rows(kv, rows, slots, block_size=bs, sanitize=sanitize)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:5].tolist()}"


def test_row_stride_and_empty_call():
    bs, nb = 64, 8
    kv = _pool(bs, nb, 0, seed=9)
    rows = make_writer_rows(100, seed=10)
    slots = np.random.default_rng(11).permutation(nb * bs)[:100].astype(np.int64)
    got = _gpu_store(kv, rows, slots, block_size=bs, sanitize=True, row_stride=520)
    want = oracle.store_rows(kv, rows, slots, block_size=bs, sanitize=True)
    assert np.array_equal(got, want)
    kv_d = torch.from_numpy(kv).cuda()
    dsv4.dsv4_quantize_store(None, 512, None, 0, kv_d, bs, nb, kv.shape[1])
    torch.cuda.synchronize()
    assert np.array_equal(kv_d.cpu().numpy(), kv)


def test_full_size_bulk_write_sampled():
    """65536 rows into a 1024-page pool in one launch (the size the
    benchmark times); 2048 sampled rows checked against the oracle row by
    row, every other slot's bytes unchanged."""
    bs, nb, n = 64, 1100, 65536
    rng = np.random.default_rng(12)
    kv = _pool(bs, nb, 0, seed=13)
    rows = make_writer_rows(n, seed=14)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    print("writer full size", flush=True)
    got = _gpu_store(kv, rows, slots, block_size=bs, sanitize=True)
    for i in rng.choice(n, 2048, replace=False):
        p, o = divmod(int(slots[i]), bs)
        data, scales = oracle.quantize_row(rows[i], sanitize=True)
        assert np.array_equal(got[p, o * 576:o * 576 + 576], data), i
        assert np.array_equal(got[p, bs * 576 + o * 8:bs * 576 + o * 8 + 8], scales), i
    written = np.zeros(nb * bs, dtype=bool)
    written[slots] = True
    free = np.flatnonzero(~written)
    for s in free[:: max(1, len(free) // 256)]:
        p, o = divmod(int(s), bs)
        assert np.array_equal(got[p, o * 576:o * 576 + 576], kv[p, o * 576:o * 576 + 576])


def test_written_cache_decodes_like_the_oracle():
    """Rows written by the GPU writer at a workload's taking-part slots are
    then decoded on the GPU; the result matches the oracle's decode of the
    same pool (the writer and the decode agree on the layout)."""
    from tests import gpu_helpers as gh
    w = make_custom(B=2, H=64, topk=256, swa=32, seq_lens=[3000, 900], seed=15)
    bs = w.block_size
    slots = []
    for b in range(w.B):
        for s in np.unique(w.topk_idx[b][w.topk_idx[b] >= 0]):
            slots.append(int(w.block_table[b, s // bs]) * bs + int(s) % bs)
    slots = np.array(slots, dtype=np.int64)
    rows = make_writer_rows(len(slots), seed=16, specials=False, spread=2)
    w.kv = _gpu_store(w.kv, rows, slots, block_size=bs, sanitize=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=3)
    ro, rl, _ = oracle.decode_workload(w, num_splits=3)
    gh.assert_decode_close(out, lse, ro, rl, "decode of a GPU-written cache")


def test_writer_and_two_kernel_path_replay_in_one_graph():
    """A step that writes new rows into the cache, then gathers and attends
    over them (two-kernel path), captured once and replayed over three
    batches of new rows; each replay matches the eager bytes of the writer
    and the oracle's decode of the resulting pool."""
    from tests import gpu_helpers as gh
    w = make_custom(B=2, H=32, topk=128, swa=16, seq_lens=[1500, 600], seed=290,
                    valid_len_range=(60, 128))
    bs = w.block_size
    slots = []
    for b in range(w.B):
        for s in np.unique(w.topk_idx[b][w.topk_idx[b] >= 0])[:40]:
            slots.append(int(w.block_table[b, s // bs]) * bs + int(s) % bs)
    slots = np.array(slots, dtype=np.int64)
    n = len(slots)
    dw = gh.DeviceWorkload(w)
    rows_d = torch.zeros((n, 512), dtype=torch.int16, device="cuda")
    slots_d = torch.from_numpy(slots).cuda()
    Kt = w.topk + w.swa
    dense = torch.empty((w.B, Kt, 512), dtype=torch.bfloat16, device="cuda")
    mask = torch.empty((w.B, Kt), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w)
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")

    def step():
        dsv4.dsv4_quantize_store(rows_d, 512, slots_d, n, dw.kv, bs, w.num_blocks, w.page_stride,
                                 dsv4.DSV4_STORE_SANITIZE)
        dsv4.dsv4_gather_dequant(desc, dw.kv, dw.bt, dw.idx, dw.vl, dense, mask)
        dsv4.dsv4_dense_decode(desc, dw.q, dense, mask, dw.sink, out, lse, 1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    pool = w.kv.copy()
    for rep in range(3):
        rows = make_writer_rows(n, seed=291 + rep, specials=False, spread=2)
        rows_d.copy_(torch.from_numpy(rows.view(np.int16)).cuda())
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        pool = oracle.store_rows(pool, rows, slots, block_size=bs, sanitize=True)
        assert np.array_equal(dw.kv.cpu().numpy(), pool)
        w.kv = pool
        ro, rl, _ = oracle.decode_workload(w)
        gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(),
                               ro, rl, f"replay {rep}")
