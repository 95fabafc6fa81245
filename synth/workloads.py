"""Seeded workloads for sparse FP8 MLA decode over an ``fp8_ds_mla`` cache.

Cache format (vLLM PR #52212 and SGLang PR #26208 pages; SGLang page,
"key source snippets", the DSV4 constants and the gather+dequant kernel):

* a row is 576 data bytes: 448 FP8-E4M3 NoPE bytes then 64 bf16 RoPE values
  (128 bytes, little endian), plus 8 scale bytes: 7 UE8M0 codes, one per 64
  NoPE dims, and one pad byte;
* a page of ``block_size`` rows keeps the data rows first and the scale
  words in a separate region after them:
  ``page*page_stride + off*576`` (data), ``page*page_stride + bs*576 + off*8``
  (scales).

Value recipe (one reading of the spec description, the same for all
configurations): NoPE = E4M3FN(round-to-nearest-even(clamp(N(0,1) / 2^(c-127),
+-448))) with codes c uniform in [120, 130]; RoPE = bf16(N(0,1)); q =
bf16(N(0,1)); sink logits fp32 N(0,1); softmax scale fp32(512^-0.5).

Only cache rows that some index list references get data.  Every other byte
of the pool (unreferenced slots, slots past a sequence's length, slack pages)
holds 0xFF, which decodes to NaN in every field, so a kernel that reads a row
it should not read cannot go unnoticed.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import numpy as np
import torch

D_QK = 512
D_NOPE = 448
D_ROPE = 64
ROW_DATA_BYTES = 576
ROW_SCALE_BYTES = 8
ROW_BYTES = ROW_DATA_BYTES + ROW_SCALE_BYTES
FP8_E4M3_MAX = 448.0
POISON = 0xFF

# The five decode workloads.  ``seq_len`` is ("fixed", L) or
# ("loguniform", lo, hi); ``invalid_frac`` is the share of main top-k
# positions set to -1; ``valid_len`` is None or an inclusive (lo, hi) range
# for the per-row length of the main list; ``per_row_splits``: the split
# count is chosen per row from the lengths (the ragged batch's configuration).
CONFIGS = [
    dict(name="tiny", B=1, H=16, topk=128, swa=0, seq_len=("fixed", 2048),
         invalid_frac=0.05, valid_len=None, num_splits=1),
    dict(name="short_batch", B=4, H=64, topk=512, swa=128, seq_len=("fixed", 8192),
         invalid_frac=0.02, valid_len=None, num_splits=0),
    dict(name="long_lowbatch", B=1, H=64, topk=2048, swa=0, seq_len=("fixed", 131072),
         invalid_frac=0.01, valid_len=None, num_splits=0),
    dict(name="large_batch", B=256, H=64, topk=512, swa=128, seq_len=("fixed", 8192),
         invalid_frac=0.0, valid_len=None, num_splits=0),
    dict(name="ragged", B=32, H=128, topk=2048, swa=128, seq_len=("loguniform", 1024, 65536),
         invalid_frac=0.05, valid_len=(1024, 2048), num_splits=0, per_row_splits=True),
]


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    H: int
    topk: int
    swa: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    page_stride: int
    seq_lens: np.ndarray          # int64 [B / s_q]
    q: np.ndarray                 # uint16 [B, H, 512], bf16 bit patterns
    kv: np.ndarray                # uint8 [num_blocks, page_stride]
    block_table: np.ndarray       # int32 [B / s_q, max_blocks_per_seq], -1 = unused
    topk_idx: np.ndarray          # int32 [B, topk + swa], req-local slots, -1 = invalid
    valid_len: Optional[np.ndarray]  # int32 [B / s_q] or None
    sink: Optional[np.ndarray]    # float32 [H] or None
    sm_scale: float               # an exact fp32 value
    num_splits: int               # 0 = let the library choose
    # With keep_floats: (seq, slot, codes [n,7], NoPE values before FP8
    # rounding [n,448] as float32, RoPE values before bf16 rounding [n,64]).
    source_rows: Optional[tuple] = None
    s_q: int = 1                  # query tokens per sequence: B = sequences * s_q
    # A second pool for the SWA entries (dict: kv, block_table, block_size,
    # num_blocks, page_stride, max_blocks_per_seq), or None: one pool.
    swa_pool: Optional[dict] = None
    # The workload's configuration asks for a split count chosen per row.
    per_row_splits: bool = False

    @property
    def Kt(self) -> int:
        return self.topk + self.swa


def _fp8_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """Round float32 values (already clamped to +-448) to E4M3FN bytes, RNE."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _round_half_up(v: float) -> int:
    return int(math.floor(v + 0.5))


def make_custom(*, B: int, H: int, topk: int, swa: int, seq_lens: Sequence[int],
                seed: int, block_size: int = 64, invalid_frac: float = 0.0,
                valid_len_range: Optional[tuple] = None, with_sink: bool = True,
                page_pad: int = 0, slack_frac: float = 0.02, num_splits: int = 0,
                poison_masked_rows: bool = False, name: str = "custom",
                keep_floats: bool = False, s_q: int = 1,
                rng: Optional[np.random.Generator] = None) -> Workload:
    """Build one seeded workload of B sequences and B * s_q query tokens.

    ``seq_lens`` gives the slot count of every sequence.  Query token j of a
    sequence of length L (multi-token decode: the sequence's last s_q
    positions) sits at position P = L - s_q + j and sees slots [0, P].  Its
    main indices are drawn uniformly without replacement from those slots
    (all of them when fewer than ``topk``, the rest -1); exactly
    round(invalid_frac*topk) main positions are then set to -1; the SWA part
    is the last ``swa`` visible slots, ascending.  With s_q = 1 this is the
    whole sequence.  With ``poison_masked_rows`` the
    rows that only masked-tail entries (past ``valid_len``) name keep their
    0xFF poison instead of data.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    assert seq_lens.shape == (B,)
    bs = int(block_size)
    Kt = topk + swa

    # Pages: one shuffled pool, ceil(L/bs) pages per sequence, slack left poisoned.
    pages_per_seq = (seq_lens + bs - 1) // bs
    needed = int(pages_per_seq.sum())
    pool = needed + int(math.ceil(slack_frac * needed))
    perm = rng.permutation(pool).astype(np.int64)
    max_blocks = max(int(pages_per_seq.max()), 1)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        block_table[b, :n] = perm[cursor:cursor + n]
        cursor += n

    # Index lists: [main top-k | SWA], req-local slots, one per query token.
    T = B * s_q
    topk_idx = np.full((T, Kt), -1, dtype=np.int32)
    n_invalid = _round_half_up(invalid_frac * topk)
    for t in range(T):
        L = int(seq_lens[t // s_q]) - s_q + t % s_q + 1      # visible slots
        n = min(topk, max(L, 0))
        topk_idx[t, :n] = rng.choice(L, size=n, replace=False) if n else []
        if n_invalid:
            pos = rng.choice(topk, size=n_invalid, replace=False)
            topk_idx[t, pos] = -1
        for j in range(swa):
            p = L - swa + j
            topk_idx[t, topk + j] = p if p >= 0 else -1

    valid_len = None
    if valid_len_range is not None:
        lo, hi = valid_len_range
        valid_len = rng.integers(lo, hi + 1, size=B).astype(np.int32)

    q = _bf16_bits(rng.standard_normal((T, H, D_QK), dtype=np.float32))
    sink = rng.standard_normal(H).astype(np.float32) if with_sink else None
    sm_scale = float(np.float32(D_QK ** -0.5))

    # Rows for every referenced (sequence, slot) pair, in a fixed order.
    ref_b, ref_slot = [], []
    for b in range(B):
        rows_b = topk_idx[b * s_q:(b + 1) * s_q]
        keep = rows_b >= 0
        if poison_masked_rows and valid_len is not None:
            vl = int(np.clip(valid_len[b], 0, topk))
            keep = keep & ((np.arange(Kt) < vl) | (np.arange(Kt) >= topk))[None, :]
        u = np.unique(rows_b[keep].astype(np.int64))
        ref_b.append(np.full(u.shape, b, dtype=np.int64))
        ref_slot.append(u)
    ref_b = np.concatenate(ref_b) if ref_b else np.zeros(0, np.int64)
    ref_slot = np.concatenate(ref_slot) if ref_slot else np.zeros(0, np.int64)
    n_rows = ref_b.shape[0]

    codes = rng.integers(120, 131, size=(n_rows, 7)).astype(np.uint8)
    nope_n = rng.standard_normal((n_rows, D_NOPE), dtype=np.float32)
    rope_n = rng.standard_normal((n_rows, D_ROPE), dtype=np.float32)
    scale = np.exp2(codes.astype(np.float32) - 127.0)
    nope_x = np.clip(nope_n / np.repeat(scale, 64, axis=1), -FP8_E4M3_MAX, FP8_E4M3_MAX)
    nope_b = _fp8_e4m3_bytes(nope_x)
    rope_b = _bf16_bits(rope_n).view(np.uint8).reshape(n_rows, 2 * D_ROPE)
    data = np.concatenate([nope_b, rope_b], axis=1)  # [n, 576]
    sc = np.concatenate([codes, np.zeros((n_rows, 1), np.uint8)], axis=1)  # [n, 8]

    page_stride = bs * ROW_BYTES + int(page_pad)
    kv = np.full((pool, page_stride), POISON, dtype=np.uint8)
    if n_rows:
        page = block_table[ref_b, ref_slot // bs].astype(np.int64)
        off = ref_slot % bs
        flat = kv.reshape(-1)
        d0 = page * page_stride + off * ROW_DATA_BYTES
        s0 = page * page_stride + bs * ROW_DATA_BYTES + off * ROW_SCALE_BYTES
        flat[d0[:, None] + np.arange(ROW_DATA_BYTES)[None, :]] = data
        flat[s0[:, None] + np.arange(ROW_SCALE_BYTES)[None, :]] = sc

    return Workload(name=name, seed=seed, B=T, H=H, topk=topk, swa=swa, block_size=bs,
                    num_blocks=pool, max_blocks_per_seq=max_blocks, page_stride=page_stride,
                    seq_lens=seq_lens, q=q, kv=kv, block_table=block_table, topk_idx=topk_idx,
                    valid_len=valid_len, sink=sink, sm_scale=sm_scale, num_splits=num_splits,
                    source_rows=((ref_b, ref_slot, codes, nope_x.astype(np.float32), rope_n)
                                 if keep_floats else None), s_q=s_q)


def make_workload(config: int, *, seed: Optional[int] = None, block_size: int = 64,
                  **overrides) -> Workload:
    """One of the five decode workloads; seed defaults to 1000 + config."""
    c = CONFIGS[config]
    seed = 1000 + config if seed is None else seed
    rng = np.random.default_rng(seed)
    kind = c["seq_len"][0]
    if kind == "fixed":
        seq_lens = np.full(c["B"], c["seq_len"][1], dtype=np.int64)
    else:
        lo, hi = c["seq_len"][1], c["seq_len"][2]
        u = rng.uniform(math.log(lo), math.log(hi), size=c["B"])
        seq_lens = np.floor(np.exp(u)).astype(np.int64)
    kw = dict(B=c["B"], H=c["H"], topk=c["topk"], swa=c["swa"], seq_lens=seq_lens, seed=seed,
              block_size=block_size, invalid_frac=c["invalid_frac"],
              valid_len_range=c["valid_len"], num_splits=c["num_splits"], name=c["name"], rng=rng)
    kw.update(overrides)
    w = make_custom(**kw)
    w.per_row_splits = bool(c.get("per_row_splits", False))
    return w


def workload_digest(w: Workload) -> str:
    h = hashlib.sha256()
    for a in (w.seq_lens, w.q, w.kv, w.block_table, w.topk_idx, w.valid_len, w.sink):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    h.update(repr((w.B, w.H, w.topk, w.swa, w.block_size, w.num_blocks, w.page_stride,
                   w.sm_scale)).encode())
    return h.hexdigest()


@dataclasses.dataclass
class ConvertCase:
    req_id: np.ndarray        # int32 [num_tokens]
    block_table: np.ndarray   # int32 [num_reqs, bt_cols]
    max_blocks: int           # columns that may be used (<= bt_cols)
    token_indices: np.ndarray  # int32 [num_tokens, ti_cols]
    width: int                # columns per token (<= ti_cols)
    block_size: int
    cu_seqlens: Optional[np.ndarray]  # int32 [num_tokens + 1] or None


def make_convert_case(*, seed: int, num_tokens: int, width: int, block_size: int,
                      num_reqs: int, max_blocks: int, ragged: bool,
                      bt_extra_cols: int = 3, ti_extra_cols: int = 5,
                      bad_frac: float = 0.1) -> ConvertCase:
    """Inputs for the req-local -> global index conversion with every kind of
    bad entry mixed in: -1 and other negatives, block numbers past the table,
    negative page entries, requests outside the table."""
    rng = np.random.default_rng(seed)
    bt = rng.integers(0, 1 << 16, size=(num_reqs, max_blocks + bt_extra_cols)).astype(np.int32)
    holes = rng.random(bt.shape) < bad_frac
    bt[holes] = -1
    req = rng.integers(0, num_reqs, size=num_tokens).astype(np.int32)
    if num_tokens > 2:
        req[rng.integers(0, num_tokens)] = num_reqs  # one request past the table
    span = max_blocks * block_size
    ti = rng.integers(0, span, size=(num_tokens, width + ti_extra_cols)).astype(np.int32)
    r = rng.random(ti.shape)
    ti[r < bad_frac] = -1
    ti[(r >= bad_frac) & (r < 1.5 * bad_frac)] = -7
    hi = (r >= 1.5 * bad_frac) & (r < 2 * bad_frac)
    ti[hi] = rng.integers(span, span + 4 * block_size, size=int(hi.sum()))
    cu = None
    if ragged:
        n = rng.integers(0, width + 1, size=num_tokens)
        cu = np.zeros(num_tokens + 1, dtype=np.int32)
        cu[1:] = np.cumsum(n)
    return ConvertCase(req_id=req, block_table=bt, max_blocks=max_blocks, token_indices=ti,
                       width=width, block_size=block_size, cu_seqlens=cu)


def poison_rows(w: Workload, b: int, slots: Sequence[int], seed: int, base=None):
    """Plants non-finite encodings in the cache rows of token ``b``'s
    request-local ``slots``: five FP8 NaN bytes (0x7F or 0xFF) in the NoPE
    part of each row, a NaN scale code (255) on group 3 of the first row, and
    a bf16 NaN then a bf16 -inf at a random RoPE position of each row.
    Returns (poisoned pool, cleaned pool): the cleaned pool holds, at each
    planted element, the encoding of a finite zero (byte 0; for the NaN scale
    group all 64 bytes 0 and code 127).  ``base`` = an earlier (poisoned,
    cleaned) pair to add to instead of ``w.kv``."""
    rng = np.random.default_rng(seed)
    kv_p, kv_c = (w.kv.copy(), w.kv.copy()) if base is None else (base[0].copy(), base[1].copy())
    bs = w.block_size
    for i, slot in enumerate(slots):
        pg, off = int(w.block_table[b, slot // bs]), slot % bs
        data = off * ROW_DATA_BYTES
        scale = bs * ROW_DATA_BYTES + off * ROW_SCALE_BYTES
        nan_bytes = rng.choice(D_NOPE, size=5, replace=False)
        kv_p[pg, data + nan_bytes] = np.where(rng.random(5) < 0.5, 0x7F, 0xFF)
        kv_c[pg, data + nan_bytes] = 0
        if i == 0:
            kv_p[pg, scale + 3] = 255
            kv_c[pg, scale + 3] = 127
            kv_c[pg, data + 192:data + 256] = 0
        r = D_NOPE + 2 * int(rng.integers(0, D_ROPE - 1))
        kv_p[pg, data + r:data + r + 4] = [0xC0, 0x7F, 0x80, 0xFF]   # bf16 NaN, bf16 -inf
        kv_c[pg, data + r:data + r + 4] = 0
    return kv_p, kv_c


def make_writer_rows(n: int, seed: int, *, specials: bool = True, spread: int = 30,
                     group_exponents: Optional[np.ndarray] = None) -> np.ndarray:
    """Seeded bf16 rows (uint16 bits [n, 512]) for the cache writer: each
    64-dim NoPE group is N(0,1) times its own power of two drawn from
    [2^-spread, 2^spread] (at 30 the UE8M0 codes spread over ~60 values), or
    2^group_exponents[row, group] when those are given; RoPE is N(0,1).  With ``specials``, one row in 8 also gets a special group:
    all zeros, a lone +-inf, NaN elements, bf16 subnormals, the bf16 maximum,
    exact E4M3FN ties, +-0 mixtures or values near 2^100, and one row in 16
    a NaN or infinite RoPE value."""
    rng = np.random.default_rng(seed)
    x = np.empty((n, 512), dtype=np.float32)
    ex = rng.integers(-spread, spread + 1, size=(n, 7))
    if group_exponents is not None:
        ex = np.asarray(group_exponents).reshape(n, 7)
    scale = 2.0 ** ex.astype(np.float32)
    x[:, :448] = (rng.standard_normal((n, 7, 64)).astype(np.float32) * scale[:, :, None]).reshape(n, 448)
    x[:, 448:] = rng.standard_normal((n, 64)).astype(np.float32)
    bits = _bf16_bits(x)
    if specials:
        for i in range(0, n, 8):
            g = int(rng.integers(0, 7))
            grp = slice(64 * g, 64 * g + 64)
            kind = int(rng.integers(0, 8))
            if kind == 0:
                bits[i, grp] = 0
            elif kind == 1:
                bits[i, 64 * g + int(rng.integers(0, 64))] = 0x7F80 if rng.random() < 0.5 else 0xFF80
            elif kind == 2:
                bits[i, 64 * g + rng.choice(64, 3, replace=False)] = [0x7FC0, 0xFFC1, 0x7F81]
            elif kind == 3:
                bits[i, grp] = rng.integers(0, 0x80, size=64).astype(np.uint16) | \
                    (rng.integers(0, 2, size=64).astype(np.uint16) << 15)
            elif kind == 4:
                bits[i, 64 * g] = 0x7F7F
            elif kind == 5:
                # 448 fixes the scale at 1; the rest are midpoints of E4M3FN steps
                bits[i, 64 * g] = 0x43E0
                m = rng.integers(0, 8, size=63)
                e = rng.integers(-6, 8, size=63)
                v = (1.0 + (2 * m + 1) / 16.0) * 2.0 ** e
                bits[i, 64 * g + 1:64 * g + 64] = _bf16_bits(v.astype(np.float32))
            elif kind == 6:
                bits[i, grp] = np.where(rng.random(64) < 0.5, 0x0000, 0x8000)
            else:
                bits[i, grp] = _bf16_bits((rng.standard_normal(64) * 2.0 ** 100).astype(np.float32))
            if i % 16 == 0:
                bits[i, 448 + int(rng.integers(0, 64))] = [0x7FC0, 0x7F80, 0xFF80][int(rng.integers(0, 3))]
    return bits



def split_swa_pool(w: Workload, *, block_size: int, seed: int, page_pad: int = 0,
                   slack_frac: float = 0.02) -> Workload:
    """Moves the rows that SWA entries (index columns >= topk) name into a
    second fp8_ds_mla pool with its own shuffled pages, block table and block
    size; rows that only SWA entries name become 0xFF poison in the first
    pool, so reading an SWA row from the wrong pool cannot go unnoticed.
    Index lists, q and lengths are unchanged (SWA indices stay req-local
    slots, now resolved through the second block table)."""
    rng = np.random.default_rng(seed)
    bs2 = int(block_size)
    B = w.block_table.shape[0]
    seq_lens = np.asarray(w.seq_lens, dtype=np.int64)
    pages_per_seq = (seq_lens + bs2 - 1) // bs2
    needed = int(pages_per_seq.sum())
    pool = needed + int(math.ceil(slack_frac * needed))
    perm = rng.permutation(pool).astype(np.int64)
    max_blocks = max(int(pages_per_seq.max()), 1)
    bt2 = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        bt2[b, :n] = perm[cursor:cursor + n]
        cursor += n
    stride2 = bs2 * ROW_BYTES + int(page_pad)
    kv2 = np.full((pool, stride2), POISON, dtype=np.uint8)
    kv1 = w.kv.copy()
    bs1 = w.block_size

    def addr(kv_stride, pg, off, bs):
        return pg * kv_stride + off * ROW_DATA_BYTES, pg * kv_stride + bs * ROW_DATA_BYTES + off * ROW_SCALE_BYTES

    main_used, swa_used = set(), set()
    for t in range(w.B):
        r = t // w.s_q
        for k, idx in enumerate(w.topk_idx[t]):
            if idx < 0:
                continue
            (swa_used if k >= w.topk else main_used).add((r, int(idx)))
    f1, f2 = w.kv.reshape(-1), kv2.reshape(-1)
    k1 = kv1.reshape(-1)
    for r, slot in sorted(swa_used):
        p1 = int(w.block_table[r, slot // bs1])
        d1, s1 = addr(w.page_stride, p1, slot % bs1, bs1)
        p2 = int(bt2[r, slot // bs2])
        d2, s2 = addr(stride2, p2, slot % bs2, bs2)
        f2[d2:d2 + ROW_DATA_BYTES] = f1[d1:d1 + ROW_DATA_BYTES]
        f2[s2:s2 + ROW_SCALE_BYTES] = f1[s1:s1 + ROW_SCALE_BYTES]
        if (r, slot) not in main_used:
            k1[d1:d1 + ROW_DATA_BYTES] = POISON
            k1[s1:s1 + ROW_SCALE_BYTES] = POISON
    return dataclasses.replace(w, kv=kv1, swa_pool=dict(
        kv=kv2, block_table=bt2, block_size=bs2, num_blocks=pool, page_stride=stride2,
        max_blocks_per_seq=max_blocks))


def make_code_sweep(*, seed: int, codes: Sequence[int] = tuple(range(255)), rows_per_code: int = 4,
                    H: int = 16, block_size: int = 64, decode_safe: bool = False) -> Workload:
    """A pool that holds every FP8 byte under every given UE8M0 code.

    Token i reads ``rows_per_code`` rows whose seven scale codes all equal
    codes[i]; each row's 448 NoPE bytes are a seeded shuffle of the byte
    values 0..255 repeated (every byte appears at least once per row).  The
    indices are global pool slots (no block table).  RoPE values are
    bf16(N(0,1)).

    With ``decode_safe`` the rows are fit for attention at the decode
    tolerance, which is absolute for values of order one: the two FP8 NaN
    bytes (0x7F, 0xFF) become +-0; bytes of magnitude above 4 have their
    exponent field lowered by 8 (the same mantissa 256 times smaller), so
    values lie within +-4 in units of the scale; and under codes where a
    byte's value times 2^(code-127) would reach 2^125 (within a factor 8 of
    the end of the bf16 and fp32 ranges, so that no sum of a few such rows
    overflows) that byte becomes the largest byte that stays below it, with
    its sign.  q's NoPE dims are then N(0,1) * 2^(127-code), the exponent
    clipped to [-126, 124] (zero below -126), so that scores stay of order
    one at every code, and its RoPE dims N(0,1).  Without it q is
    bf16(N(0,1)).  Byte magnitudes are read with torch's float8_e4m3fn type
    (a library decode)."""
    rng = np.random.default_rng(seed)
    codes = [int(c) for c in codes]
    T = len(codes)
    n_rows = T * rows_per_code
    mag = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .double().abs().numpy()
    data = np.empty((n_rows, ROW_DATA_BYTES), dtype=np.uint8)
    sc = np.zeros((n_rows, ROW_SCALE_BYTES), dtype=np.uint8)
    base = (np.arange(D_NOPE) % 256).astype(np.uint8)
    for i, c in enumerate(codes):
        for k in range(rows_per_code):
            r = i * rows_per_code + k
            nope = rng.permutation(base)
            if decode_safe:
                nope = np.where((nope & 0x7F) == 0x7F, nope & 0x80, nope)
                nope = np.where(mag[nope] > 4.0, nope - 0x40, nope).astype(np.uint8)
                limit = 2.0 ** (252 - c)          # |v| * 2^(c-127) < 2^125
                ok = np.flatnonzero((mag < limit) & np.isfinite(mag))
                top = ok[np.argmax(mag[ok])] & 0x7F
                big = (mag[nope] >= limit) & np.isfinite(mag[nope])
                nope = np.where(big, (nope & 0x80) | top, nope)
            data[r, :D_NOPE] = nope
            data[r, D_NOPE:] = _bf16_bits(rng.standard_normal(D_ROPE, dtype=np.float32)) \
                .view(np.uint8)
            sc[r, :7] = c
    bs = int(block_size)
    pages = (n_rows + bs - 1) // bs + 1
    page_stride = bs * ROW_BYTES
    kv = np.full((pages, page_stride), POISON, dtype=np.uint8)
    slots = rng.permutation(pages * bs)[:n_rows].astype(np.int64)
    flat = kv.reshape(-1)
    page, off = slots // bs, slots % bs
    d0 = page * page_stride + off * ROW_DATA_BYTES
    s0 = page * page_stride + bs * ROW_DATA_BYTES + off * ROW_SCALE_BYTES
    flat[d0[:, None] + np.arange(ROW_DATA_BYTES)[None, :]] = data
    flat[s0[:, None] + np.arange(ROW_SCALE_BYTES)[None, :]] = sc
    topk_idx = slots.reshape(T, rows_per_code).astype(np.int32)
    qf = rng.standard_normal((T, H, D_QK), dtype=np.float32)
    if decode_safe:
        e = 127 - np.asarray(codes, dtype=np.float64)
        s = np.where(e >= -126, np.exp2(np.clip(e, -126, 124)), 0.0).astype(np.float32)
        qf[:, :, :D_NOPE] *= s[:, None, None]
    return Workload(name="code_sweep", seed=seed, B=T, H=H, topk=rows_per_code, swa=0,
                    block_size=bs, num_blocks=pages, max_blocks_per_seq=0,
                    page_stride=page_stride, seq_lens=np.full(T, pages * bs, dtype=np.int64),
                    q=_bf16_bits(qf), kv=kv, block_table=None, topk_idx=topk_idx,
                    valid_len=None, sink=rng.standard_normal(H).astype(np.float32),
                    sm_scale=float(np.float32(D_QK ** -0.5)), num_splits=0)
