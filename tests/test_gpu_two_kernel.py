"""The two-kernel decode path on the GPU: gather + dequantise into dense
bf16 rows with a mask, then attention over them.

Stage 1 is byte work and is compared bit for bit: every taking-part row
must hold the oracle's dequantised row (exact in bf16 for the cache's
codes), every other row zeros, and the mask must mark exactly the entries
the oracle's resolution rejects.  Stage 2 and the whole path are compared
with the oracle's decode to the decode tolerance (|d out| <= 2e-2 +
1e-2 |out_ref|, |d lse| <= 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, make_workload, poison_rows

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _gather(dw, flags=0, kv=None):
    gh = _gh()
    w = dw.w
    Kt = w.topk + w.swa
    desc = gh.make_desc(w, flags=flags)
    kv_out = torch.full((w.B, Kt, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    mask = torch.full((w.B, Kt), 7, dtype=torch.uint8, device="cuda")
    dsv4.dsv4_gather_dequant(desc, dw.kv if kv is None else kv, dw.bt, dw.idx, dw.vl, kv_out, mask)
    torch.cuda.synchronize()
    return kv_out, mask


def _dense(dw, kv_out, mask, S):
    gh = _gh()
    w = dw.w
    desc = gh.make_desc(w)
    n = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws)
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    dsv4.dsv4_dense_decode(desc, dw.q, kv_out, mask, dw.sink, out, lse, S)
    torch.cuda.synchronize()
    return out.float().double().cpu().numpy(), lse.double().cpu().numpy()


def _expected_rows(w, kv=None):
    """Oracle rows and mask for every (token, column)."""
    kv = w.kv if kv is None else kv
    Kt = w.topk + w.swa
    desc = oracle.make_desc(B=w.B, H=w.H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                            num_blocks=w.num_blocks, page_stride=w.page_stride,
                            sm_scale=w.sm_scale, block_table=w.block_table,
                            max_blocks_per_seq=w.max_blocks_per_seq, s_q=w.s_q)
    rows = np.zeros((w.B, Kt, 512), dtype=np.uint16)
    mask = np.ones((w.B, Kt), dtype=np.uint8)
    for b in range(w.B):
        r = b // w.s_q
        vl = w.topk if w.valid_len is None else int(np.clip(w.valid_len[r], 0, w.topk))
        for k in range(Kt):
            if k < w.topk and k >= vl:
                continue
            hit = oracle.resolve(desc, w.block_table, r, int(w.topk_idx[b, k]))
            if hit is None:
                continue
            mask[b, k] = 0
            rows[b, k] = _bf16_bits(oracle.dequant_row(desc, kv, *hit))
    return rows, mask


@pytest.mark.parametrize("s_q", [1, 2])
def test_gather_dequant_is_bit_exact(s_q):
    gh = _gh()
    w = make_custom(B=3, H=16, topk=200, swa=40, seq_lens=[3000, 500, 150], seed=170 + s_q,
                    invalid_frac=0.05, valid_len_range=(80, 200), s_q=s_q)
    # an index past the table and one whose page entry is negative take no part
    w.topk_idx[0, 3] = w.max_blocks_per_seq * w.block_size + 5
    print(f"gather s_q={s_q}", flush=True)
    dw = gh.DeviceWorkload(w)
    kv_out, mask = _gather(dw)
    rows, want_mask = _expected_rows(w)
    got = kv_out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(mask.cpu().numpy(), want_mask)
    assert np.array_equal(got, rows)


def test_gather_with_scrub_zeroes_poison():
    gh = _gh()
    w = make_custom(B=2, H=16, topk=128, swa=16, seq_lens=[900, 400], seed=180)
    used = [int(x) for x in w.topk_idx[0, :128] if x >= 0][:5]
    kv_p, kv_c = poison_rows(w, 0, used, seed=181)
    dw = gh.DeviceWorkload(w)
    a, ma = _gather(dw, flags=dsv4.DSV4_DECODE_SCRUB, kv=torch.from_numpy(kv_p).cuda())
    w.kv = kv_c
    dw2 = gh.DeviceWorkload(w)
    b_, mb = _gather(dw2)
    assert torch.equal(ma, mb) and torch.equal(a.view(torch.int16), b_.view(torch.int16))


@pytest.mark.parametrize("S", [1, 3, 0])
def test_two_kernel_path_matches_the_oracle(S):
    gh = _gh()
    w = make_custom(B=4, H=64, topk=512, swa=64, seq_lens=[9000, 3000, 700, 200], seed=190,
                    invalid_frac=0.03, valid_len_range=(200, 512))
    print(f"two-kernel S={S}", flush=True)
    dw = gh.DeviceWorkload(w)
    kv_out, mask = _gather(dw)
    out, lse = _dense(dw, kv_out, mask, S)
    ro, rl, _ = oracle.decode_workload(w, num_splits=S)
    gh.assert_decode_close(out, lse, ro, rl, f"two-kernel S={S}")


def test_masked_dense_rows_are_never_read():
    """Rows whose mask byte is 1 may hold anything (here NaN): the output is
    bit-identical to the run over the gathered zeros."""
    gh = _gh()
    w = make_custom(B=2, H=32, topk=256, swa=32, seq_lens=[5000, 2000], seed=200,
                    invalid_frac=0.1, valid_len_range=(100, 256))
    dw = gh.DeviceWorkload(w)
    kv_out, mask = _gather(dw)
    clean = _dense(dw, kv_out, mask, 2)
    dirty_rows = kv_out.clone()
    dirty_rows[mask.bool()] = float("nan")
    dirty = _dense(dw, dirty_rows, mask, 2)
    assert np.array_equal(clean[0], dirty[0]) and np.array_equal(clean[1], dirty[1])


@pytest.mark.parametrize("ci", [3, 4])
def test_two_kernel_path_at_full_size(ci):
    gh = _gh()
    w = make_workload(ci)
    print(f"two-kernel full size workload {ci} {w.name}", flush=True)
    dw = gh.DeviceWorkload(w)
    kv_out, mask = _gather(dw)
    out, lse = _dense(dw, kv_out, mask, 0)
    del kv_out, mask
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, f"two-kernel workload {ci}")
