"""Pins of the oracle's cache writer (quantise-and-store into fp8_ds_mla).

The writer follows the sanitising writer snippet of the vLLM PR #52212 page:
UE8M0 codes clamped to [0, 254] (255 without sanitising) and non-finite RoPE
values stored as 0.  The amax -> code step is not printed on the pages; the
reading is the smallest code whose scale brings the group's largest
magnitude into the E4M3FN range (|v| <= 448).

Pins, none of which re-types the oracle's own formulas:
  * hand-worked rows (bytes derived on paper from the E4M3FN and UE8M0
    encodings, listed in each case);
  * the rounding of every in-range bf16 value against torch's float32 ->
    float8_e4m3fn cast (a library routine);
  * the round trip through the independently pinned decoders (within half
    an FP8 step of the scaled value);
  * placement: stored rows read back through the decode oracle's row
    reader at the slots given, other bytes untouched, bad slots skipped;
  * the pages' equivalence: decoding a sanitised cache without the scrub
    equals decoding the unsanitised cache with it.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_custom


def _bits(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def _set(x, j, value):
    x[j] = _bits([value])[0]


@pytest.mark.parametrize("sanitize", [False, True])
def test_hand_worked_rows(sanitize):
    x = np.zeros(512, dtype=np.uint16)
    # group 0: max 448 -> code 127 (scale 1).  448 = 1.75*2^8 -> 0 1111 110;
    # -1 -> 1 0111 000; 0.5 -> 0 0110 000; -0 -> 0x80; 1.0625 is the tie
    # between 1 and 1.125 -> even mantissa 1.0 (0x38); 1.1875 is the tie
    # between 1.125 and 1.25 -> 1.25 (0x3A); 2^-9 is the smallest subnormal
    # (0x01); 2^-10 ties 0 and 2^-9 -> 0; 3*2^-10 ties 2^-9 and 2^-8 -> 0x02.
    for j, v in enumerate([448.0, -1.0, 0.5, -0.0, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -10,
                           3 * 2.0 ** -10]):
        _set(x, j, v)
    # group 1: max 450 -> code 128 (448*2 >= 450 > 448); 450/2 = 225 -> 224
    # (1.75*2^7 -> 0 1110 110 = 0x76); -3/2 = -1.5 -> 1 0111 100 = 0xBC.
    _set(x, 64, 450.0)
    _set(x, 65, -3.0)
    # group 2: max 1 -> code 119 (448*2^-8 = 1.75 >= 1 > 448*2^-9); 1*2^8 ->
    # 0 1111 000 = 0x78.
    _set(x, 128, 1.0)
    # group 3: all zero -> code 0, bytes 0.
    # group 4: bf16 max 0x7F7F (~3.39e38 = 1.9921875*2^127) -> code 247
    # (448*2^120 = 1.75*2^128 >= it > 1.75*2^127); it scales to
    # 1.9921875*2^7 = 255, between 240 (0x77) and 256 (0x78), nearer 256.
    x[256] = 0x7F7F
    # group 5: the smallest bf16 subnormal 2^-133 -> code 0 (448*2^-127
    # covers it); scaled by 2^127 it is 2^-6 = 0 0001 000 = 0x08.
    x[320] = 0x0001
    # group 6: a NaN element does not set the scale: max 2 -> code 120
    # (1.75*2^1 >= 2 > 1.75); 2*2^7 = 256 -> 0x78; the NaN byte is 0x7F.
    x[384] = 0x7FC0
    _set(x, 385, 2.0)
    # RoPE: finite values are kept bit for bit; NaN and +inf are zeroed only
    # with sanitize.
    x[448] = _bits([1.5])[0]
    x[449] = 0x7FC0
    x[450] = 0x7F80
    x[451] = 0xFF80
    data, scales = oracle.quantize_row(x, sanitize=sanitize)
    assert list(scales) == [127, 128, 119, 0, 247, 0, 120, 0]
    assert list(data[:9]) == [0x7E, 0xB8, 0x30, 0x80, 0x38, 0x3A, 0x01, 0x00, 0x02]
    assert data[9:64].tolist() == [0] * 55
    assert (data[64], data[65], data[128], data[256], data[320]) == (0x76, 0xBC, 0x78, 0x78, 0x08)
    assert (data[384], data[385]) == (0x7F, 0x78)
    rope = data[448:].view("<u2")
    want = [_bits([1.5])[0], 0x7FC0, 0x7F80, 0xFF80]
    if sanitize:
        want[1:] = [0, 0, 0]
    assert rope[:4].tolist() == [int(v) for v in want]
    assert rope[4:].tolist() == [0] * 60


@pytest.mark.parametrize("sanitize,code", [(False, 255), (True, 254)])
def test_infinite_nope_caps_the_code(sanitize, code):
    """An infinity makes no code sufficient: the cap is stored.  Finite
    neighbours scale by 2^(127-cap) and vanish; +-inf clamps to +-448."""
    x = np.zeros(512, dtype=np.uint16)
    x[70] = 0x7F80
    x[71] = 0xFF80
    _set(x, 72, 1000.0)
    data, scales = oracle.quantize_row(x, sanitize=sanitize)
    assert scales[1] == code and scales[0] == 0
    assert (data[70], data[71], data[72]) == (0x7E, 0xFE, 0x00)


def _all_bf16_in_range():
    b = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    return b[keep], v[keep]


def test_rounding_matches_the_library_cast_for_every_in_range_bf16():
    """With a 448 in each group the code is 127 (scale 1), so the stored byte
    of every other element is the plain float -> E4M3FN rounding."""
    b, v = _all_bf16_in_range()
    per = 63
    n = -(-len(b) // (7 * per))
    rows = np.zeros((n, 512), dtype=np.uint16)
    pos = []
    k = 0
    for r in range(n):
        for g in range(7):
            rows[r, 64 * g] = _bits([448.0])[0]
            for j in range(1, 64):
                if k < len(b):
                    rows[r, 64 * g + j] = b[k]
                    pos.append((r, 64 * g + j))
                    k += 1
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.empty(len(b), dtype=np.uint8)
    for r in range(n):
        data, scales = oracle.quantize_row(rows[r], sanitize=True)
        assert (scales[:7] == 127).all()
        sel = [i for i, (rr, _) in enumerate(pos) if rr == r]
        got[sel] = data[[pos[i][1] for i in sel]]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_is_within_half_an_fp8_step(seed):
    """Random groups of very different magnitudes: each stored element
    decodes (through the pinned E4M3FN/UE8M0 decoders) to within half an
    FP8 step of its input, the largest magnitude of a group lands in
    (224, 448] after scaling unless the code hit 0, and RoPE is exact."""
    rng = np.random.default_rng(seed)
    x = np.zeros(512, dtype=np.float32)
    for g in range(7):
        x[64 * g:64 * g + 64] = rng.standard_normal(64) * 2.0 ** rng.integers(-140, 120)
    x[448:] = rng.standard_normal(64)
    xb = _bits(x)
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    data, scales = oracle.quantize_row(xb, sanitize=True)
    for g in range(7):
        c = int(scales[g])
        sc = oracle.ue8m0(c)
        grp = slice(64 * g, 64 * g + 64)
        y = xv[grp] / sc
        amax = np.abs(y).max()
        assert amax <= 448.0 and (c == 0 or amax > 224.0)
        dec = np.array([oracle.e4m3fn(int(d)) for d in data[grp]])
        # E4M3FN steps: 2^(e-3) for |y| in [2^e, 2^(e+1)), 2^-9 below 2^-6.
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        step = 2.0 ** (e - 3)
        assert np.all(np.abs(dec - y) <= step / 2 + 1e-300)
    assert np.array_equal(data[448:].view("<u2"), xb[448:])


def _pool(bs, nb, pad=0, fill=0xA5):
    return np.full((nb, bs * 584 + pad), fill, dtype=np.uint8)


def test_rows_land_at_their_slots_and_nothing_else_changes():
    bs, nb = 16, 6
    kv = _pool(bs, nb, pad=8)
    rng = np.random.default_rng(5)
    rows = _bits(rng.standard_normal((5, 512)))
    slots = np.array([0, 17, 95, -1, 6 * 16], dtype=np.int64)   # last one is past the pool
    out = oracle.store_rows(kv, rows, slots, block_size=bs, sanitize=True)
    desc = oracle.make_desc(B=1, H=16, topk=1, swa=0, block_size=bs, num_blocks=nb,
                            page_stride=kv.shape[1], sm_scale=1.0)
    touched = np.zeros_like(kv, dtype=bool)
    for i, s in enumerate(slots[:3]):
        p, o = divmod(int(s), bs)
        data, scales = oracle.quantize_row(rows[i], sanitize=True)
        assert np.array_equal(out[p, o * 576:o * 576 + 576], data)
        sc0 = bs * 576 + o * 8
        assert np.array_equal(out[p, sc0:sc0 + 8], scales)
        touched[p, o * 576:o * 576 + 576] = True
        touched[p, sc0:sc0 + 8] = True
        got = oracle.dequant_row(desc, out, p, o)
        xv = torch.from_numpy(rows[i].view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.allclose(got, xv, rtol=2 ** -4, atol=0)
    assert np.array_equal(out[~touched], kv[~touched])


def test_sanitised_cache_without_scrub_equals_raw_cache_with_scrub():
    """The pages' reason for the sanitising writer: a decode that skips the
    scrub over a sanitised cache gives what a scrubbing decode gives over
    the legacy cache.  Rows with non-finite RoPE values and finite NoPE."""
    w = make_custom(B=2, H=16, topk=64, swa=16, seq_lens=[400, 300], seed=21)
    rng = np.random.default_rng(22)
    bs = w.block_size
    slots, rows = [], []
    for b in range(w.B):
        for k in range(0, w.topk + w.swa, 3):
            s = int(w.topk_idx[b, k])
            if s < 0:
                continue
            x = rng.standard_normal(512).astype(np.float32)
            xb = _bits(x)
            if k % 2 == 0:
                xb[448 + int(rng.integers(0, 64))] = [0x7FC0, 0x7F80, 0xFF80][k % 3]
            slots.append(int(w.block_table[b, s // bs]) * bs + s % bs)
            rows.append(xb)
    rows = np.stack(rows)
    slots = np.array(slots, dtype=np.int64)
    clean = oracle.store_rows(w.kv, rows, slots, block_size=bs, sanitize=True)
    raw = oracle.store_rows(w.kv, rows, slots, block_size=bs, sanitize=False)
    o1, l1, _ = oracle.decode_workload(w, kv=clean)
    o2, l2, _ = oracle.decode_workload(w, kv=raw, scrub=True)
    assert np.all(np.isfinite(o1))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, _, _ = oracle.decode_workload(w, kv=raw)
    assert np.isnan(o3).any()
