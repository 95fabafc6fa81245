"""Device-side plumbing shared by the GPU tests: move a synth workload to the
GPU, call the library through its C ABI, and compare with the oracle to the
stated tolerance (|d out| <= 2e-2 + 1e-2 |out_ref| elementwise on the bf16
output, |d lse| <= 1e-3, infinities equal)."""

from __future__ import annotations

import numpy as np
import torch

import sparse_mla_attention_block_amd as dsv4

OUT_ATOL = 2e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def _t(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


class DeviceWorkload:
    def __init__(self, w):
        self.w = w
        self.q = _t(w.q.view(np.int16), torch.bfloat16)
        self.kv = _t(w.kv)
        self.bt = _t(w.block_table)
        self.idx = _t(w.topk_idx)
        self.vl = _t(w.valid_len)
        self.sink = _t(w.sink)


_KEEP = object()


def make_desc(w, *, use_bt=True, workspace=None, flags=0):
    return dsv4.make_desc(batch=w.B, num_heads=w.H, topk=w.topk, swa=w.swa,
                          block_size=w.block_size, num_blocks=w.num_blocks,
                          page_stride=w.page_stride, sm_scale=w.sm_scale,
                          max_blocks_per_seq=w.max_blocks_per_seq if use_bt else 0,
                          block_table_stride=w.block_table.shape[1] if use_bt else 0,
                          workspace=workspace, flags=flags, tokens_per_seq=w.s_q)


def gpu_decode(dw: DeviceWorkload, *, num_splits=None, use_bt=True, topk_idx=None,
               valid_len=_KEEP, sink=_KEEP, partial_then_combine=False, stream=None,
               want_lse=True, kv=None, flags=0):
    """Runs the decode; returns (out, lse) as float64 numpy arrays."""
    w = dw.w
    S = w.num_splits if num_splits is None else num_splits
    desc = make_desc(w, use_bt=use_bt, flags=flags)
    nbytes = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None
    desc = make_desc(w, use_bt=use_bt, workspace=ws, flags=flags)
    kv = dw.kv if kv is None else kv
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = dw.idx if topk_idx is None else topk_idx
    vl = dw.vl if valid_len is _KEEP else valid_len
    sk = dw.sink if sink is _KEEP else sink
    bt = dw.bt if use_bt else None
    if partial_then_combine:
        plan = dsv4.dsv4_sparse_decode_plan(desc, S)
        dsv4.dsv4_sparse_decode_partial(desc, dw.q, kv, bt, idx, vl, sk, out,
                                        lse if want_lse else None, S, stream)
        if plan.num_splits > 1:
            po, pl = dsv4.workspace_split_views(ws, w.B, w.H, plan.num_splits)
            dsv4.dsv4_combine_splits(w.B, w.H, plan.num_splits, po, pl, sk, out,
                                     lse if want_lse else None, stream)
    else:
        dsv4.dsv4_sparse_decode(desc, dw.q, kv, bt, idx, vl, sk, out,
                                lse if want_lse else None, S, stream)
    torch.cuda.synchronize()
    return out.float().double().cpu().numpy(), lse.double().cpu().numpy()


def assert_decode_close(out, lse, ref_out, ref_lse, what=""):
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    assert not np.isnan(out).any(), f"{what}: NaN in output (unwritten or poisoned)"
    err = np.abs(out - ref_out)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs off; worst |d|={err.max():.3e} at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)}")
    inf_ref = np.isinf(ref_lse)
    assert np.array_equal(np.isinf(lse), inf_ref), f"{what}: lse infinities differ"
    assert np.array_equal(lse[inf_ref], ref_lse[inf_ref])
    if (~inf_ref).any():
        dl = np.abs(lse[~inf_ref] - ref_lse[~inf_ref])
        assert dl.max() <= LSE_ATOL, f"{what}: |d lse| max {dl.max():.3e}"


def gpu_convert(*, token_indices, block_table, max_blocks_per_req, block_size, width=None,
                req_id=None, num_reqs=None, cu_seqlens=None, invalid_fill=0, stream=None):
    ti = _t(token_indices.astype(np.int32))
    bt = _t(block_table.astype(np.int32))
    T = token_indices.shape[0]
    width = token_indices.shape[1] if width is None else width
    rq = _t(req_id)
    cu = _t(cu_seqlens)
    nreq = block_table.shape[0] if num_reqs is None else num_reqs
    n_out = int(cu_seqlens[-1]) if cu_seqlens is not None else T * width
    out = torch.full((max(n_out, 1),), np.iinfo(np.int32).min, dtype=torch.int32, device="cuda")
    dsv4.dsv4_convert_req_index_to_global(rq, nreq, bt, block_table.shape[1], max_blocks_per_req,
                                          ti, token_indices.shape[1], T, width, block_size, cu,
                                          invalid_fill, out, stream)
    torch.cuda.synchronize()
    o = out.cpu().numpy()[:n_out]
    return o if cu_seqlens is not None else o.reshape(T, width)
