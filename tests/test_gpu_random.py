"""Seeded random decode cases on the GPU, mixing features the targeted tests
cover one at a time: head counts 16-128 (every head-group variant), forced
and selected split counts, block sizes, masked tails, invalid entries,
several query tokens per sequence, a separate SWA pool, the pipelined
kernel forced, balanced splits (DSV4_DECODE_BALANCE) and the scrub
variants (DSV4_DECODE_SCRUB, on caches with no non-finite element).  Each case is
compared with the oracle to the decode tolerance (|d out| <= 2e-2 +
1e-2 |out_ref|, |d lse| <= 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_custom, split_swa_pool

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(seed)
    H = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    B = int(rng.integers(1, 6))
    s_q = int(rng.integers(1, 3))
    topk = int(rng.integers(1, 700))
    swa = int(rng.choice([0, 0, 16, 64, 128]))
    bs = int(rng.choice([1, 16, 64, 128]))
    lens = [int(x) for x in rng.integers(s_q + 1, 20000, size=B)]
    S = int(rng.choice([0, 0, 1, 2, 3, 8, 64]))
    w = make_custom(B=B, H=H, topk=topk, swa=swa, seq_lens=lens, seed=seed, block_size=bs,
                    invalid_frac=float(rng.choice([0.0, 0.05, 0.3])),
                    valid_len_range=(0, topk) if rng.random() < 0.5 else None,
                    with_sink=bool(rng.random() < 0.8), s_q=s_q,
                    page_pad=int(rng.choice([0, 8, 64])))
    dual = swa > 0 and rng.random() < 0.4
    if dual:
        w = split_swa_pool(w, block_size=int(rng.choice([1, 16, 64])), seed=seed + 1)
    flags = ((dsv4.DSV4_DECODE_BALANCE if rng.random() < 0.4 else 0)
             | (dsv4.DSV4_DECODE_PIPELINED if rng.random() < 0.3 else 0))
    # The scrub variants on finite caches give the plain decode's result.
    flags |= dsv4.DSV4_DECODE_SCRUB if rng.random() < 0.25 else 0
    return w, S, dual, flags


@pytest.mark.parametrize("seed", range(300, 348))
def test_random_case(seed):
    from tests import gpu_helpers as gh
    w, S, dual, flags = _case(seed)
    print(f"random seed={seed} B={w.B} H={w.H} topk={w.topk} swa={w.swa} bs={w.block_size} "
          f"s_q={w.s_q} S={S} dual={dual} flags={flags}", flush=True)
    desc = gh.make_desc(w, flags=flags)
    n = dsv4.dsv4_sparse_decode_workspace_bytes(desc, S)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    desc = gh.make_desc(w, workspace=ws, flags=flags)
    dw = gh.DeviceWorkload(w)
    out = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    if dual:
        sp = w.swa_pool
        main = dsv4.make_pool(dw.kv, dw.bt, block_size=w.block_size,
                              max_blocks_per_seq=w.max_blocks_per_seq)
        kv2 = torch.from_numpy(sp["kv"]).cuda()
        bt2 = torch.from_numpy(sp["block_table"]).cuda()
        swa = dsv4.make_pool(kv2, bt2, block_size=sp["block_size"],
                             max_blocks_per_seq=sp["max_blocks_per_seq"])
        dsv4.dsv4_sparse_decode_dual(desc, dw.q, main, swa, dw.idx, dw.vl, dw.sink, out, lse, S)
    else:
        dsv4.dsv4_sparse_decode(desc, dw.q, dw.kv, dw.bt, dw.idx, dw.vl, dw.sink, out, lse, S)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.decode_workload(w, num_splits=S)
    gh.assert_decode_close(out.float().double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl,
                           f"seed {seed}")
