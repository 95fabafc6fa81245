"""Pins of the oracle's byte decoders and row reader against library routines
and the generator's own (pre-rounding) values."""

import numpy as np
import pytest
import torch

import oracle
from synth import make_custom, ROW_BYTES


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    return bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def test_e4m3fn_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3fn(c) for c in range(256)])
    assert _same(got, ref)
    # Two NaN codes, finite maximum 448, smallest subnormal 2^-9.
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_ue8m0_all_codes_match_torch_and_power_of_two():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.ue8m0(c) for c in range(256)])
    assert _same(got, ref)
    for c in range(255):
        assert got[c] == np.ldexp(1.0, c - 127)
    assert np.isnan(got[255])


def test_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32)
    ref = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    ref = ref.to(torch.float64).numpy()
    got = np.array([oracle.bf16(int(c)) for c in codes])
    assert _same(got, ref)


def _desc(block_size, num_blocks, page_stride, bt=None):
    return oracle.make_desc(B=1, H=1, topk=1, swa=0, block_size=block_size, num_blocks=num_blocks,
                            page_stride=page_stride, sm_scale=1.0, block_table=bt)


def test_dequant_row_hand_built_page():
    """A row placed by hand: bs=3, a padded page stride, page 2, slot 1.
    Data at page*stride + off*576, scales in their own region at
    page*stride + bs*576 + off*8 (SGLang PR #26208 page, gather+dequant
    snippet)."""
    bs, stride, npages, page, off = 3, 3 * ROW_BYTES + 40, 4, 2, 1
    kv = np.full(npages * stride, 0xFF, dtype=np.uint8)
    rng = np.random.default_rng(7)
    nope = rng.integers(0, 256, size=448).astype(np.uint8)
    nope[(nope & 0x7F) == 0x7F] = 0x38            # keep the row finite
    codes = np.array([120, 127, 130, 1, 200, 127, 126], dtype=np.uint8)
    rope = torch.randn(64, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    d0 = page * stride + off * 576
    s0 = page * stride + bs * 576 + off * 8
    kv[d0:d0 + 448] = nope
    kv[d0 + 448:d0 + 576] = rope.view(np.uint8)
    kv[s0:s0 + 7] = codes
    kv[s0 + 7] = 0x00
    got = oracle.dequant_row(_desc(bs, npages, stride), kv.reshape(npages, stride), page, off)
    fp8 = torch.from_numpy(nope).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    want = np.concatenate([fp8 * np.repeat(sc, 64),
                           torch.from_numpy(rope).view(torch.bfloat16).to(torch.float64).numpy()])
    assert np.array_equal(got, want)
    # The neighbouring poisoned slots decode to NaN: the reader does not
    # stray outside its row.
    assert np.isnan(oracle.dequant_row(_desc(bs, npages, stride), kv.reshape(npages, stride),
                                       page, 0)).all()


@pytest.mark.parametrize("bs,pad", [(64, 0), (1, 0), (16, 24)])
def test_dequant_rows_recover_generator_values(bs, pad):
    """Every referenced row read back through the block table equals the
    generator's pre-rounding values within FP8/bf16 rounding (independent of
    the byte layout code on either side)."""
    w = make_custom(B=2, H=1, topk=40, swa=8, seq_lens=[300, 77], seed=3, block_size=bs,
                    page_pad=pad, keep_floats=True)
    ref_b, ref_slot, codes, nope_x, rope_f = w.source_rows
    desc = oracle.make_desc(B=w.B, H=w.H, topk=w.topk, swa=w.swa, block_size=w.block_size,
                            num_blocks=w.num_blocks, page_stride=w.page_stride, sm_scale=1.0,
                            block_table=w.block_table)
    for i in range(len(ref_b)):
        r = oracle.resolve(desc, w.block_table, int(ref_b[i]), int(ref_slot[i]))
        assert r is not None
        row = oracle.dequant_row(desc, w.kv, *r)
        scale = np.repeat(np.exp2(codes[i].astype(np.float64) - 127), 64)
        x = nope_x[i].astype(np.float64)
        # E4M3 RNE: |err| <= 2^-4 |x| for normals, <= 2^-10 absolute in subnormals.
        tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) * scale
        assert np.all(np.abs(row[:448] - x * scale) <= tol + 1e-300)
        assert np.all(np.abs(row[448:] - rope_f[i]) <= np.abs(rope_f[i]) * 2.0 ** -8)


def test_resolve_rules():
    bt = np.array([[5, -1, 2, 7]], dtype=np.int32)
    d = oracle.make_desc(B=1, H=1, topk=1, swa=0, block_size=4, num_blocks=7, page_stride=4 * 584,
                         sm_scale=1.0, block_table=bt, max_blocks_per_seq=3)
    assert oracle.resolve(d, bt, 0, 1) == (5, 1)       # block 0 -> page 5
    assert oracle.resolve(d, bt, 0, 4) is None         # page entry -1
    assert oracle.resolve(d, bt, 0, 10) == (2, 2)      # block 2 -> page 2, offset 2
    assert oracle.resolve(d, bt, 0, 12) is None        # block 3 past max_blocks_per_seq
    assert oracle.resolve(d, bt, 0, -1) is None
    assert oracle.resolve(d, bt, 0, -9) is None
    bt2 = np.array([[7]], dtype=np.int32)
    d2 = oracle.make_desc(B=1, H=1, topk=1, swa=0, block_size=4, num_blocks=7, page_stride=4 * 584,
                          sm_scale=1.0, block_table=bt2)
    assert oracle.resolve(d2, bt2, 0, 0) is None       # page 7 outside the pool of 7
    # Without a table the index is a pool slot.
    d3 = oracle.make_desc(B=1, H=1, topk=1, swa=0, block_size=4, num_blocks=7, page_stride=4 * 584,
                          sm_scale=1.0)
    assert oracle.resolve(d3, None, 0, 27) == (6, 3)
    assert oracle.resolve(d3, None, 0, 28) is None
