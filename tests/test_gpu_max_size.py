"""The longest index list the plan accepts (topk + swa = 2^24), against
closed forms.

Every entry of the 2^24-entry list names the same cache row r, so every score
of head h is s_h = sm_scale * q_h . k_r and the softmax weights are equal
(the attention definition the oracle's attend_one writes out).  With
N = 2^24 entries and a sink logit c_h:

    out_h = V_r * N e^{s_h} / (N e^{s_h} + e^{c_h}),   lse_h = ln(N e^{s_h} + e^{c_h}),

and without a sink out_h = V_r, lse_h = s_h + ln N.  V_r (the row's 512
dequantised values) is exact in bf16.  With 64 splits each split holds 2^18
entries: its probabilities are all 1, its running sum 2^18 and its normalised
partial V_r, all exact, and the merge of 64 equal partials is V_r again, so
without a sink the output must equal V_r bit for bit.  A sink of
s_h + ln N takes half of the mass (out = V_r / 2).  The plan's limit on
topk + swa is in include/dsv4.h.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom

pytestmark = pytest.mark.gpu

N = 1 << 24
SWA = 64


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _max_workload(H, seed):
    """A small cache and one query token whose 2^24 entries all name one row."""
    w = make_custom(B=1, H=H, topk=64, swa=0, seq_lens=[256], seed=seed)
    r = int(w.topk_idx[0, 0])
    assert r >= 0
    desc = oracle.make_desc(B=1, H=H, topk=64, swa=0, block_size=w.block_size,
                            num_blocks=w.num_blocks, page_stride=w.page_stride,
                            sm_scale=w.sm_scale, block_table=w.block_table,
                            max_blocks_per_seq=w.max_blocks_per_seq)
    page, off = oracle.resolve(desc, w.block_table, 0, r)
    v = oracle.dequant_row(desc, w.kv, page, off)                       # [512] fp64
    q = w.q[0].astype(np.uint32) << 16
    q = q.view(np.float32).astype(np.float64)                            # [H, 512]
    s = (q @ v) * float(w.sm_scale)                                      # [H]
    w.topk, w.swa = N - SWA, SWA
    w.topk_idx = np.full((1, N), r, dtype=np.int32)
    w.valid_len = None
    w.sink = None
    return w, v, s


def _expected(v, s, sink):
    if sink is None:
        return np.broadcast_to(v, (s.shape[0], 512)), s + math.log(N)
    c = sink.astype(np.float64)
    m = np.maximum(s, c)
    den = N * np.exp(s - m) + np.exp(c - m)
    frac = N * np.exp(s - m) / den
    return v[None, :] * frac[:, None], m + np.log(den)


def _run(w, sink, S, with_slots=False):
    gh = _gh()
    dw = gh.DeviceWorkload(w)
    sk = None if sink is None else torch.from_numpy(sink).cuda()
    if not with_slots:
        out, lse = gh.gpu_decode(dw, num_splits=S, sink=sk, valid_len=None)
        return out, lse, None
    desc = gh.make_desc(w)
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws)
    out = torch.full((1, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, w.H), float("nan"), dtype=torch.float32, device="cuda")
    slots = torch.full((1, N), -7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_sparse_decode_with_slots(desc, dw.q, dw.kv, dw.bt, dw.idx, None, sk, out, lse,
                                       S, slots)
    torch.cuda.synchronize()
    return (out.float().double().cpu().numpy(), lse.double().cpu().numpy(),
            slots.cpu().numpy())


def test_max_list_without_sink_is_the_row_bit_for_bit():
    w, v, s = _max_workload(16, seed=3101)
    print(f"max list: H=16 S=64 topk+swa={N}", flush=True)
    out, lse, _ = _run(w, None, 64)
    want_out, want_lse = _expected(v, s, None)
    assert np.array_equal(out[0], want_out), float(np.max(np.abs(out[0] - want_out)))
    assert np.max(np.abs(lse[0] - want_lse)) <= 1e-3


@pytest.mark.parametrize("with_slots", [False, True])
def test_max_list_with_half_mass_sink_128_heads(with_slots):
    w, v, s = _max_workload(128, seed=3102 + with_slots)
    sink = (s + math.log(N)).astype(np.float32)
    sink[::4] = -np.inf                       # a quarter of the heads without a sink
    print(f"max list: H=128 selector plan sink=half slots={with_slots}", flush=True)
    out, lse, slots = _run(w, sink, 0, with_slots)
    want_out, want_lse = _expected(v, s, np.where(np.isinf(sink), -np.inf, sink))
    err = np.abs(out[0] - want_out)
    # bf16 output: two units in the last place of the expected value.
    assert np.all(err <= 2.0 ** -7 * np.abs(want_out) + 1e-6), float(np.max(err))
    assert np.max(np.abs(lse[0] - want_lse)) <= 1e-3
    if with_slots:
        r = int(w.topk_idx[0, 0])
        page = int(w.block_table[0, r // w.block_size])
        assert np.all(slots == page * w.block_size + r % w.block_size)
