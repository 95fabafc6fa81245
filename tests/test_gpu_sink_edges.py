"""Sink logits at their edges on the GPU, against the fp64 oracle.

Per-head sinks mix -inf (the sink takes no part: plain softmax), +25 (the
sink holds almost all the mass), -25 and N(0,1).  The batch holds a token
with no taking-part entry at all, one with only its sliding-window entries,
one whose main list valid_len masks to nothing, and an ordinary one.  A
(token, head) with no taking-part entry must give out = 0 and lse = sink
(-inf for a -inf sink), never NaN (vLLM PR #52212 page, implementation item
1: the sink semantics; the contract in include/dsv4.h).  Both the fused
decode and the two-kernel path (gather + dense decode) run with one split
(the sink folded into the kernel's own epilogue) and with four (the sink
folded in by the combine).
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _edge_workload(H, seed):
    w = make_custom(B=4, H=H, topk=96, swa=16, seq_lens=[700, 700, 700, 700], seed=seed,
                    invalid_frac=0.05, valid_len_range=(40, 96))
    w.topk_idx[0, :] = -1                          # nothing takes part
    w.topk_idx[1, :w.topk] = -1                    # sliding window only
    w.valid_len[2] = 0                             # main list masked by valid_len
    sink = np.random.default_rng(seed + 1).standard_normal(H).astype(np.float32)
    sink[0::4] = -np.inf
    sink[1::4] = 25.0
    sink[2::8] = -25.0
    w.sink = sink
    return w


def _dense_decode(dw, S):
    gh = _gh()
    w = dw.w
    Kt = w.topk + w.swa
    desc = gh.make_desc(w)
    rows = torch.empty((w.B, Kt, 512), dtype=torch.bfloat16, device="cuda")
    mask = torch.empty((w.B, Kt), dtype=torch.uint8, device="cuda")
    dsv4.dsv4_gather_dequant(desc, dw.kv, dw.bt, dw.idx, dw.vl, rows, mask)
    n = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws)
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    dsv4.dsv4_dense_decode(desc, dw.q, rows, mask, dw.sink, out, lse, S)
    torch.cuda.synchronize()
    return out.float().double().cpu().numpy(), lse.double().cpu().numpy()


def _check_empty_rows(w, out, lse):
    # Token 0 has no taking-part entry at all.
    assert np.all(out[0] == 0.0)
    assert np.array_equal(np.isneginf(lse[0]), np.isneginf(w.sink))
    fin = np.isfinite(w.sink)
    assert np.allclose(lse[0][fin], w.sink[fin], atol=1e-6, rtol=0)


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("H", [16, 64])
def test_sink_edges_fused(H, S):
    gh = _gh()
    w = _edge_workload(H, seed=300 + H)
    print(f"sink edges fused H={H} S={S}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=S)
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, f"sink edges fused H={H} S={S}")
    _check_empty_rows(w, out, lse)


@pytest.mark.parametrize("S", [1, 4])
def test_sink_edges_two_kernel(S):
    gh = _gh()
    w = _edge_workload(32, seed=340)
    print(f"sink edges two-kernel S={S}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = _dense_decode(dw, S)
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, f"sink edges two-kernel S={S}")
    _check_empty_rows(w, out, lse)


def test_all_sinks_minus_inf_equal_no_sink():
    """A sink of -inf for every head is the same softmax as no sink at all:
    the outputs and lse agree bit for bit at S = 1 and S = 4."""
    gh = _gh()
    w = _edge_workload(16, seed=350)
    w.sink = np.full(w.H, -np.inf, dtype=np.float32)
    dw = gh.DeviceWorkload(w)
    for S in (1, 4):
        a = gh.gpu_decode(dw, num_splits=S)
        b = gh.gpu_decode(dw, num_splits=S, sink=None)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), S
