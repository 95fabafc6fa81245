"""Multi-token decode (s_q query tokens per sequence) and graph-stable
launches on the GPU, against the fp64 oracle to the decode tolerance
(|d out| <= 2e-2 + 1e-2 |out_ref|, |d lse| <= 1e-3).

A decode's launch configuration depends only on the descriptor's shapes,
never on index, length or cache contents, so one captured HIP graph serves
every later batch of the same shape: each row picks its active splits from
its own valid length on the device (vLLM PR #52212 page, implementation
item 2: fixed grid under graph capture, per-row active splits, no host
synchronisation).  Padding rows (all indices -1, length 0) of a graph
captured at the maximum batch produce out = 0 and lse = sink.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_custom

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


@pytest.mark.parametrize("s_q,S", [(2, 1), (2, 4), (3, 1), (3, 7), (4, 2)])
def test_multi_token_decode(s_q, S):
    gh = _gh()
    w = make_custom(B=3, H=64, topk=256, swa=64, seq_lens=[4000, 700, 300], seed=140 + s_q,
                    invalid_frac=0.03, valid_len_range=(100, 256), s_q=s_q)
    print(f"multi-token s_q={s_q} S={S} tokens={w.B}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=S)
    ro, rl, _ = oracle.decode_workload(w, num_splits=S)
    gh.assert_decode_close(out, lse, ro, rl, f"s_q={s_q} S={S}")


def test_multi_token_at_full_size():
    """An MTP step of the large-batch shape: 128 sequences x 2 tokens, H=64,
    top-k 512 + SWA 128 over 8192-slot sequences, the selector's launch."""
    gh = _gh()
    w = make_custom(B=128, H=64, topk=512, swa=128, seq_lens=[8192] * 128, seed=150, s_q=2)
    print(f"multi-token full size tokens={w.B}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=0)
    ro, rl, _ = oracle.decode_workload(w)
    gh.assert_decode_close(out, lse, ro, rl, "MTP full size")


def _copy_into(dst, src):
    dst.copy_(src)


def test_one_graph_serves_new_batches_and_padding():
    """Capture the decode (split path with combine) once; then, three times,
    write a new batch of the same shape into the captured input buffers,
    with the last tokens padded (indices -1, length 0), replay, and compare
    with the oracle and with an eager call (bitwise).  Eager work runs
    between the replays."""
    import sparse_mla_attention_block_amd as dsv4
    gh = _gh()
    kw = dict(B=6, H=64, topk=512, swa=64, seq_lens=[9000, 3000, 800, 5000, 600, 2000],
              invalid_frac=0.02, valid_len_range=(200, 512), s_q=2)
    w0 = make_custom(seed=160, **kw)
    dw = gh.DeviceWorkload(w0)
    S = 4
    desc = gh.make_desc(w0)
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w0, workspace=ws)
    out = torch.zeros((w0.B, w0.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((w0.B, w0.H), dtype=torch.float32, device="cuda")

    def call(o, l):
        dsv4.dsv4_sparse_decode(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, o, l, S)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)

    for rep, seed in enumerate((161, 162, 163)):
        w = make_custom(seed=seed, **kw)
        pad_seq = 2 - rep % 2                     # last 1 or 2 sequences are padding
        n_real = (6 - pad_seq) * 2
        w.topk_idx[n_real:] = -1
        w.valid_len[6 - pad_seq:] = 0
        assert w.kv.shape == w0.kv.shape and w.block_table.shape == w0.block_table.shape
        for dst, src in ((dw.q, w.q.view(np.int16)), (dw.kv, w.kv), (dw.bt, w.block_table),
                         (dw.idx, w.topk_idx), (dw.vl, w.valid_len), (dw.sink, w.sink)):
            t = torch.from_numpy(np.ascontiguousarray(src))
            _copy_into(dst, t.view(dst.dtype).cuda())
        torch.cuda.synchronize()
        print(f"graph replay {rep} seed={seed} padding sequences={pad_seq}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        o_g = out.float().double().cpu().numpy()
        l_g = lse.double().cpu().numpy()
        # eager work between replays, then an eager call into fresh buffers
        e_out = torch.full_like(out, float("nan"))
        e_lse = torch.full_like(lse, float("nan"))
        call(e_out, e_lse)
        torch.cuda.synchronize()
        assert torch.equal(e_out, out) and torch.equal(e_lse, lse)
        ro, rl, _ = oracle.decode_workload(w, num_splits=S)
        gh.assert_decode_close(o_g, l_g, ro, rl, f"replay {rep}")
        assert np.all(o_g[n_real:] == 0)
        assert np.allclose(l_g[n_real:], np.broadcast_to(w.sink, l_g[n_real:].shape), atol=0)
