"""Every FP8 byte under every UE8M0 scale code, on the GPU.

The sanitising cache writer clamps scale codes to [0, 254] (vLLM PR #52212
page, implementation item 3), so a cache can hold any of them; code 255 (a
NaN scale) appears only in a cache written without sanitising, which the
decode reads with its scrub flag.  The pools come from
``synth.make_code_sweep``: every row's seven codes are equal and its 448
NoPE bytes hold all 256 byte values.

* Gather (dsv4_gather_dequant): bit for bit against the bf16 rounding
  (nearest, ties to even) of the oracle's exact fp64 row, NaN where the
  oracle has NaN (FP8 bytes 0x7F / 0xFF), +-inf where the exact product lies
  past the bf16 range.
* Gather with the scrub flag, codes 255, 254, 250, 247 and a few ordinary
  ones: non-finite elements read as 0; a product past the bf16 range is
  also read as 0 (the kernel tests finiteness after its bf16 convert, a
  reading the oracle's fp64 scrub does not share, so the expected row
  applies it to the bf16 rounding).
* Decode (dsv4_sparse_decode): codes 0..254 with rows fit for attention
  (no NaN byte, values within +-4 in units of the scale, no product within
  a factor 8 of the bf16 range) against the oracle to the decode tolerance,
  then again with each token's NoPE output scaled back by 2^(127-code), so
  that every code is held to the bar of code 127 (the tolerance's absolute
  term is sized for values of order one).
* A cache written by dsv4_quantize_store from rows whose 64-dim groups span
  2^-30 .. 2^30 plus special groups (zeros, infinities, NaN, subnormals,
  2^100, ...) is decoded with the scrub flag against the oracle's scrub mode.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_block_amd as dsv4
from synth import make_code_sweep, make_custom, make_writer_rows

pytestmark = pytest.mark.gpu


def _gh():
    from tests import gpu_helpers
    return gpu_helpers


def _bf16_bits(x):
    """bf16 bit patterns of fp64 values, rounded to nearest even (exact
    products of an FP8 value and a power of two fit fp32, so the cast through
    fp32 rounds once)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _odesc(w, scrub=False):
    return oracle.make_desc(B=w.B, H=w.H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                            num_blocks=w.num_blocks, page_stride=w.page_stride,
                            sm_scale=w.sm_scale, scrub=scrub)


def _gather(w, flags=0):
    gh = _gh()
    dw = gh.DeviceWorkload(w)
    Kt = w.topk + w.swa
    desc = gh.make_desc(w, use_bt=False, flags=flags)
    kv_out = torch.full((w.B, Kt, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    mask = torch.full((w.B, Kt), 7, dtype=torch.uint8, device="cuda")
    dsv4.dsv4_gather_dequant(desc, dw.kv, None, dw.idx, None, kv_out, mask)
    torch.cuda.synchronize()
    return kv_out.view(torch.int16).cpu().numpy().view(np.uint16), mask.cpu().numpy()


def _expected(w, scrub=False):
    d = _odesc(w, scrub)
    vals = np.zeros((w.B, w.topk, 512), dtype=np.float64)
    for b in range(w.B):
        for k in range(w.topk):
            s = int(w.topk_idx[b, k])
            vals[b, k] = oracle.dequant_row(d, w.kv, s // w.block_size, s % w.block_size)
    return vals


def _assert_bits(got, want_vals, what):
    nan = np.isnan(want_vals)
    got_nan = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(got_nan, nan), f"{what}: NaN positions differ"
    want = _bf16_bits(np.where(nan, 0.0, want_vals))
    bad = (got != want) & ~nan
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements differ, first at {tuple(i)}: "
                             f"got 0x{got[tuple(i)]:04x}, want 0x{want[tuple(i)]:04x} "
                             f"({want_vals[tuple(i)]!r})")


def test_gather_every_byte_under_every_code():
    w = make_code_sweep(seed=400)                       # codes 0..254
    print(f"code sweep gather: {w.B} codes x {w.topk} rows", flush=True)
    got, mask = _gather(w)
    assert np.all(mask == 0)
    vals = _expected(w)
    assert np.isinf(vals).sum() == 0                    # fp64 never overflows here
    _assert_bits(got, vals, "gather")
    # The sweep does reach past the bf16 range (large bytes under codes >= 247).
    assert (np.abs(vals[np.isfinite(vals)]) >= 2.0 ** 128).any()


def test_gather_nan_scale_and_overflow_under_scrub():
    codes = [255, 254, 250, 247, 200, 127, 40, 1, 0]
    w = make_code_sweep(seed=401, codes=codes, rows_per_code=3)
    print("code sweep gather with scrub", flush=True)
    got, mask = _gather(w, flags=dsv4.DSV4_DECODE_SCRUB)
    assert np.all(mask == 0)
    vals = _expected(w, scrub=True)                     # NaN elements (bytes, code 255) -> 0
    assert not np.isnan(vals).any()
    want = _bf16_bits(vals)
    over = (want & 0x7FFF) == 0x7F80                    # past the bf16 range: read as 0
    want = np.where(over, 0, want)
    assert over.any()
    assert np.array_equal(got, want)
    assert np.all(got[0][:, :448] == 0)                 # code 255: every NoPE element is NaN-scaled


@pytest.mark.parametrize("S", [1, 2])
def test_decode_every_code(S):
    gh = _gh()
    w = make_code_sweep(seed=402, decode_safe=True)
    print(f"code sweep decode S={S}", flush=True)
    dw = gh.DeviceWorkload(w)
    out, lse = gh.gpu_decode(dw, num_splits=S, use_bt=False)
    ro, rl, n = oracle.decode_workload(w, use_block_table=False)
    assert n == w.B * w.topk
    codes = np.arange(255)
    # The tolerance's absolute term is sized for values of order one.  In
    # natural units it is held where the scale is at most 1 (codes <= 127);
    # then, for every code from 8 on, in units of each token's scale (a power
    # of two, so the rescaling is exact) on the NoPE dims, RoPE dims as they
    # are.  Below code 8 the bf16 output itself is subnormal and its step
    # nears the absolute bound in those units.
    lo = codes <= 127
    gh.assert_decode_close(out[lo], lse[lo], ro[lo], rl[lo], f"code sweep S={S}, codes <= 127")
    keep = codes >= 8
    f = np.exp2(127.0 - codes[keep])[:, None, None]
    o, r = out[keep].copy(), ro[keep].copy()
    o[:, :, :448] *= f
    r[:, :, :448] *= f
    gh.assert_decode_close(o, lse[keep], r, rl[keep], f"code sweep S={S}, in units of the scale")


def test_writer_cache_with_spread_codes():
    """A cache written by the GPU writer with sanitising (codes clamped to
    [0, 254], RoPE non-finite -> 0; a NaN NoPE element still stores the FP8
    NaN byte) from rows whose 64-dim groups are N(0,1) times 2^e, e drawn
    per (token, group) from [-30, 30], plus the writer's special groups
    (zeros, infinities, NaN, subnormals, the bf16 maximum, 2^100, ...).
    * Gather: every taking-part row bit for bit against the bf16 rounding of
      the oracle's row (NaN where it has NaN).
    * Decode with the scrub flag against the oracle's scrub mode, NoPE output
      dims compared in units of 2^e of their (token, group), RoPE dims as
      they are.  q's NoPE dims are 0, so the scores come from the RoPE dims
      and stay of order one whatever the groups hold; every group still
      enters the output through PV.  Left out of the decode (not of the
      gather): entries whose row holds a value past the bf16 range (a
      bf16-maximum or infinite input stores 2^128 or more), which bf16
      cannot hold, and rows with a special group far outside their token's
      scale (the 2^100 and E4M3 tie groups, > 2^24 in those units): two of
      them in one group can cancel to far below their own size, where the
      bound's absolute term, sized for values of order one, no longer
      covers the bf16 rounding of the weights."""
    gh = _gh()
    w = make_custom(B=2, H=64, topk=256, swa=32, seq_lens=[3000, 900], seed=410)
    bs = w.block_size
    ex = np.random.default_rng(412).integers(-30, 31, size=(w.B, 7))
    slots, owner = [], []
    for b in range(w.B):
        for s in np.unique(w.topk_idx[b][w.topk_idx[b] >= 0]):
            slots.append(int(w.block_table[b, s // bs]) * bs + int(s) % bs)
            owner.append(b)
    slots = np.array(slots, dtype=np.int64)
    rows = make_writer_rows(len(slots), seed=411, specials=True, group_exponents=ex[owner])
    dw = gh.DeviceWorkload(w)
    rows_d = torch.from_numpy(rows.view(np.int16)).cuda()
    slots_d = torch.from_numpy(slots).cuda()
    print("writer cache with spread codes", flush=True)
    dsv4.dsv4_quantize_store(rows_d, 512, slots_d, len(slots), dw.kv, bs, w.num_blocks,
                             w.page_stride, dsv4.DSV4_STORE_SANITIZE)
    torch.cuda.synchronize()
    pool = dw.kv.cpu().numpy()
    assert np.array_equal(pool, oracle.store_rows(w.kv, rows, slots, block_size=bs,
                                                  sanitize=True))
    w.kv = pool
    codes = pool[(slots // bs)[:, None], bs * 576 + (slots % bs)[:, None] * 8 + np.arange(7)]
    assert codes.min() < 100 and codes.max() > 150

    # Gather, bit for bit.
    dw = gh.DeviceWorkload(w)
    desc = gh.make_desc(w)
    kv_out = torch.full((w.B, w.Kt, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    mask = torch.full((w.B, w.Kt), 7, dtype=torch.uint8, device="cuda")
    dsv4.dsv4_gather_dequant(desc, dw.kv, dw.bt, dw.idx, dw.vl, kv_out, mask)
    torch.cuda.synchronize()
    got = kv_out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(mask.cpu().numpy() == (w.topk_idx < 0))
    d = _odesc(w)
    vals = np.zeros((w.B, w.Kt, 512), dtype=np.float64)
    for b in range(w.B):
        for k in range(w.Kt):
            s = int(w.topk_idx[b, k])
            if s >= 0:
                vals[b, k] = oracle.dequant_row(d, pool, int(w.block_table[b, s // bs]), s % bs)
    _assert_bits(got, vals, "writer cache gather")

    # Decode with scrub.
    f = np.ones((w.B, 1, 512))
    f[:, 0, :448] = np.repeat(np.exp2(-ex.astype(np.float64)), 64, axis=1)
    mag = np.abs(np.nan_to_num(vals))
    over = (mag >= 2.0 ** 128).any(axis=2)
    outlier = (mag * f > 2.0 ** 24).any(axis=2)
    assert over.any() and outlier.any()
    w.topk_idx[over | outlier] = -1
    assert (w.topk_idx >= 0).sum() > 400
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).float()
    qf[:, :, :448] = 0.0
    w.q = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dw = gh.DeviceWorkload(w)
    for S in (1, 3):
        out, lse = gh.gpu_decode(dw, num_splits=S, flags=dsv4.DSV4_DECODE_SCRUB)
        ro, rl, _ = oracle.decode_workload(w, num_splits=S, scrub=True)
        gh.assert_decode_close(out * f, lse, ro * f, rl, f"writer cache decode S={S}")
