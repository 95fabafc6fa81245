"""Pins of the oracle's attention against things other than itself:

* torch's fp64 scaled-dot-product attention (math backend, which also returns
  the softmax weights) on rows rebuilt from the generator's own values, with
  the sink as an extra key of zero value whose logit is the sink;
* closed forms (identical rows, a single entry, no valid entry);
* invariants (index order, split count, page placement, poison rows never
  read, weights plus sink mass equal to one).
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_custom, poison_rows, split_swa_pool

RTOL = 1e-10
ATOL = 1e-12


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _source_row_table(w):
    """(seq, slot) -> dequantised row rebuilt from the generator's values:
    torch rounds the NoPE values to E4M3FN and the RoPE values to bf16."""
    ref_b, ref_slot, codes, nope_x, rope_f = w.source_rows
    nope = torch.from_numpy(nope_x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    nope = nope * np.repeat(np.exp2(codes.astype(np.float64) - 127.0), 64, axis=1)
    rope = torch.from_numpy(rope_f).to(torch.bfloat16).to(torch.float64).numpy()
    rows = np.concatenate([nope, rope], axis=1)
    return {(int(b), int(s)): rows[i] for i, (b, s) in enumerate(zip(ref_b, ref_slot))}


def _entry_mask(w, b):
    """Taking-part columns of token b (its sequence's top-k length applies)."""
    Kt = w.topk + w.swa
    cols = np.arange(Kt)
    r = b // w.s_q
    vl = w.topk if w.valid_len is None else int(np.clip(w.valid_len[r], 0, w.topk))
    return (w.topk_idx[b] >= 0) & ((cols < vl) | (cols >= w.topk))


def sdpa_reference(w, sink_bias_when_none=0.0):
    """Returns (out, lse) from torch's math-backend SDPA in fp64."""
    table = _source_row_table(w)
    B, H, Kt = w.B, w.H, w.topk + w.swa
    out = np.zeros((B, H, 512))
    lse = np.zeros((B, H))
    for b in range(B):
        m = _entry_mask(w, b)
        K = np.zeros((Kt + 1, 512))
        for k in range(Kt):
            if m[k]:
                K[k] = table[(b // w.s_q, int(w.topk_idx[b, k]))]
        bias = np.full((H, Kt + 1), -np.inf)
        bias[:, :Kt][:, m] = 0.0
        c = w.sink.astype(np.float64) if w.sink is not None else np.full(H, sink_bias_when_none)
        bias[:, Kt] = c                          # extra key: zero vector, logit = sink
        q = torch.from_numpy(_bf16_to_f64(w.q[b]))[None, :, None, :]
        kk = torch.from_numpy(K)[None, None].expand(1, H, Kt + 1, 512)
        o, wts = torch.ops.aten._scaled_dot_product_attention_math(
            q, kk, kk, attn_mask=torch.from_numpy(bias)[None, :, None, :], scale=w.sm_scale)
        o = o[0, :, 0].numpy()
        ws = wts[0, :, 0, Kt].numpy()            # weight that went to the extra key
        if w.sink is not None:
            out[b] = o
            lse[b] = c - np.log(ws)
        else:
            out[b] = o / (1.0 - ws)[:, None]
            lse[b] = c + np.log((1.0 - ws) / ws)
    return out, lse


def _w(seed, **kw):
    base = dict(B=3, H=4, topk=40, swa=8, seq_lens=[500, 90, 41], seed=seed, invalid_frac=0.15,
                valid_len_range=(10, 40), keep_floats=True)
    base.update(kw)
    return make_custom(**base)


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("bs", [64, 16, 1])
def test_matches_sdpa_with_sink(seed, bs):
    w = _w(seed, block_size=bs)
    out, lse, _ = oracle.decode_workload(w)
    ro, rl = sdpa_reference(w)
    np.testing.assert_allclose(out, ro, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(lse, rl, rtol=RTOL, atol=ATOL)


@pytest.mark.parametrize("seed", [4, 5])
def test_matches_sdpa_without_sink(seed):
    w = _w(seed, with_sink=False, valid_len_range=None)
    out, lse, _ = oracle.decode_workload(w)
    ro, rl = sdpa_reference(w)
    np.testing.assert_allclose(out, ro, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(lse, rl, rtol=RTOL, atol=ATOL)


def _one_row_case(seed, K, with_sink=True):
    """B=1 workload whose list names one slot K times (and -1 elsewhere)."""
    w = make_custom(B=1, H=3, topk=16, swa=0, seq_lens=[64], seed=seed, keep_floats=True,
                    with_sink=with_sink)
    slot = int(w.topk_idx[0, 0])
    w.topk_idx[0, :] = -1
    w.topk_idx[0, :K] = slot
    v = _source_row_table(w)[(0, slot)]
    q = _bf16_to_f64(w.q[0])
    s = w.sm_scale * (q @ v)           # [H] logits
    return w, v, s


@pytest.mark.parametrize("K", [1, 2, 7])
def test_closed_form_identical_rows_with_sink(K):
    w, v, s = _one_row_case(11 + K, K)
    out, lse, n = oracle.decode_workload(w)
    assert n == K
    sink = w.sink.astype(np.float64)
    den = K * np.exp(s) + np.exp(sink)
    np.testing.assert_allclose(out[0], (K * np.exp(s) / den)[:, None] * v[None, :], rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(den), rtol=1e-12, atol=1e-14)
    if K == 1:  # one entry: weight = sigmoid(s - sink)
        sig = 1.0 / (1.0 + np.exp(-(s - sink)))
        np.testing.assert_allclose(out[0], sig[:, None] * v[None, :], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[0], np.logaddexp(s, sink), rtol=1e-12)


@pytest.mark.parametrize("K", [1, 5])
def test_closed_form_no_sink_returns_the_row(K):
    w, v, s = _one_row_case(21 + K, K, with_sink=False)
    out, lse, _ = oracle.decode_workload(w)
    np.testing.assert_allclose(out[0], np.broadcast_to(v, out[0].shape), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse[0], s + np.log(K), rtol=1e-13)


def test_weights_plus_sink_mass_is_one():
    w, v, s = _one_row_case(31, 6)
    out, lse, _ = oracle.decode_workload(w)
    j = int(np.argmax(np.abs(v)))
    total_w = out[0, :, j] / v[j]
    sink_mass = np.exp(w.sink.astype(np.float64) - lse[0])
    np.testing.assert_allclose(total_w + sink_mass, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("with_sink", [True, False])
def test_all_invalid_row_is_zero(with_sink):
    w = _w(41, with_sink=with_sink)
    w.topk_idx[1, :] = -1                 # whole row invalid
    w.topk_idx[2, : w.topk] = -1          # main invalid, SWA still there
    out, lse, _ = oracle.decode_workload(w)
    assert np.all(out[1] == 0.0)
    if with_sink:
        assert np.array_equal(lse[1], w.sink.astype(np.float64))
    else:
        assert np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(out[2])) and np.any(out[2] != 0)


def test_index_order_invariance():
    w = _w(51)
    out, lse, _ = oracle.decode_workload(w)
    rng = np.random.default_rng(0)
    ti = w.topk_idx.copy()
    for b in range(w.B):
        vl = int(np.clip(w.valid_len[b], 0, w.topk))
        ti[b, :vl] = ti[b, :vl][rng.permutation(vl)]
        ti[b, vl:w.topk] = ti[b, vl:w.topk][rng.permutation(w.topk - vl)]
        ti[b, w.topk:] = ti[b, w.topk:][rng.permutation(w.swa)]
    o2, l2, _ = oracle.decode_workload(w, topk_idx=ti)
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l2, lse, rtol=1e-13)
    # Without valid_len every position may move anywhere.
    w.valid_len = None
    out, lse, _ = oracle.decode_workload(w)
    ti = np.stack([r[rng.permutation(r.size)] for r in w.topk_idx])
    o3, l3, _ = oracle.decode_workload(w, topk_idx=ti)
    np.testing.assert_allclose(o3, out, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l3, lse, rtol=1e-13)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 32, 64])
def test_split_merge_identity(S):
    w = _w(61, B=2, topk=48, seq_lens=[700, 33])
    out, lse, _ = oracle.decode_workload(w)
    o, l, _ = oracle.decode_workload(w, num_splits=S)
    np.testing.assert_allclose(o, out, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l, lse, rtol=1e-12, atol=1e-15)


def test_valid_len_semantics():
    w = _w(71)
    base_vl = w.valid_len.copy()
    # valid_len = 0 masks the whole main list; the same as main entries set to -1.
    w.valid_len = np.zeros(w.B, np.int32)
    o0, l0, _ = oracle.decode_workload(w)
    ti = w.topk_idx.copy()
    ti[:, :w.topk] = -1
    o1, l1, _ = oracle.decode_workload(w, topk_idx=ti, valid_len=None)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # Negative clamps to 0, above topk clamps to topk (== no valid_len).
    w.valid_len = np.full(w.B, -5, np.int32)
    o2, l2, _ = oracle.decode_workload(w)
    assert np.array_equal(o2, o0) and np.array_equal(l2, l0)
    w.valid_len = np.full(w.B, w.topk + 9, np.int32)
    o3, l3, _ = oracle.decode_workload(w)
    o4, l4, _ = oracle.decode_workload(w, valid_len=None)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    # valid_len = v is the same as setting main[v:] to -1.
    w.valid_len = base_vl
    o5, l5, _ = oracle.decode_workload(w)
    ti = w.topk_idx.copy()
    for b in range(w.B):
        ti[b, base_vl[b]:w.topk] = -1
    o6, l6, _ = oracle.decode_workload(w, topk_idx=ti, valid_len=None)
    assert np.array_equal(o5, o6) and np.array_equal(l5, l6)


def test_duplicates_count_as_a_multiset():
    w = _w(81, valid_len_range=None)
    ti = w.topk_idx.copy()
    ti[:, 1] = ti[:, 0]                   # entry 0 listed twice
    w.topk_idx = ti
    out, lse, _ = oracle.decode_workload(w)
    ro, rl = sdpa_reference(w)
    np.testing.assert_allclose(out, ro, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(lse, rl, rtol=RTOL, atol=ATOL)


def test_page_placement_invariance():
    """Moving pages around the pool (and the table with them) changes
    nothing; an identity table equals a table-free call on pool slots."""
    w = _w(91, B=1, seq_lens=[700])
    out, lse, _ = oracle.decode_workload(w)
    n = int((w.seq_lens[0] + w.block_size - 1) // w.block_size)
    kv2 = w.kv.copy()
    kv2[:n] = w.kv[w.block_table[0, :n]]
    ident = np.arange(w.max_blocks_per_seq, dtype=np.int32)[None, :]
    o1, l1, _ = oracle.decode_workload(w, kv=kv2, block_table=ident)
    assert np.array_equal(o1, out) and np.array_equal(l1, lse)
    o2, l2, _ = oracle.decode_workload(w, kv=kv2, use_block_table=False)
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)


def test_poison_rows_are_never_read():
    """Masked-tail entries re-pointed at poisoned (0xFF) slots, and entries
    whose block lies past the table, leave the output bit-identical."""
    w = _w(101, B=1, seq_lens=[900], topk=40)
    out, lse, _ = oracle.decode_workload(w)
    used = set(int(x) for x in w.topk_idx[0] if x >= 0)
    free = [s for s in range(int(w.seq_lens[0])) if s not in used]
    ti = w.topk_idx.copy()
    vl = int(w.valid_len[0])
    for k in range(vl, w.topk):
        if ti[0, k] >= 0:
            ti[0, k] = free.pop()
    ti[0, vl:w.topk][::3] = w.max_blocks_per_seq * w.block_size + 5
    o2, l2, _ = oracle.decode_workload(w, topk_idx=ti)
    assert np.all(np.isfinite(o2))
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)



def _poisoned_and_cleaned(w, seed):
    """Poison four taking-part rows of token 0 (see synth.poison_rows)."""
    m = _entry_mask(w, 0)
    slots = [int(w.topk_idx[0, k]) for k in np.flatnonzero(m)][:4]
    return poison_rows(w, 0, slots, seed)

def test_scrub_is_the_identity_on_a_finite_cache():
    w = _w(111)
    out, lse, _ = oracle.decode_workload(w)
    o2, l2, _ = oracle.decode_workload(w, scrub=True)
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)


@pytest.mark.parametrize("S", [0, 3])
def test_scrub_reads_non_finite_elements_as_zero(S):
    """Scrubbing a poisoned pool gives exactly what the same pool with those
    elements set to a finite 0 gives without scrubbing; unscrubbed, the poison
    reaches token 0's output."""
    w = _w(112, B=2, seq_lens=[700, 300])
    kv_p, kv_c = _poisoned_and_cleaned(w, 5)
    o_s, l_s, _ = oracle.decode_workload(w, kv=kv_p, scrub=True, num_splits=S)
    o_c, l_c, _ = oracle.decode_workload(w, kv=kv_c, num_splits=S)
    assert np.all(np.isfinite(o_s)) and np.array_equal(o_s, o_c) and np.array_equal(l_s, l_c)
    o_u, _, _ = oracle.decode_workload(w, kv=kv_p, num_splits=S)
    assert np.isnan(o_u[0]).any() and np.array_equal(o_u[1], o_c[1])


@pytest.mark.parametrize("s_q", [2, 3])
def test_multi_token_decode_matches_sdpa(s_q):
    """s_q query tokens per sequence, each with its own causal top-k list,
    sharing the sequence's block table and top-k length."""
    w = _w(120 + s_q, s_q=s_q)
    assert w.B == 3 * s_q and w.block_table.shape[0] == 3
    out, lse, _ = oracle.decode_workload(w)
    ro, rl = sdpa_reference(w)
    np.testing.assert_allclose(out, ro, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(lse, rl, rtol=RTOL, atol=ATOL)


def test_multi_token_equals_single_token_with_expanded_tables():
    """Repeating each sequence's block-table row and top-k length once per
    token and calling with s_q = 1 gives the identical result."""
    w = _w(125, s_q=4, block_size=16)
    out, lse, n = oracle.decode_workload(w)
    bt = np.repeat(w.block_table, 4, axis=0)
    vl = np.repeat(w.valid_len, 4)
    o1, l1, n1 = oracle.decode_workload(w, block_table=bt, valid_len=vl, s_q=1)
    assert n == n1 and np.array_equal(out, o1) and np.array_equal(lse, l1)


@pytest.mark.parametrize("bs2", [16, 1, 64])
def test_dual_pool_decode_matches_sdpa(bs2):
    """SWA entries resolved through a second pool (own pages, block table and
    block size; the first pool holds poison where only SWA rows were)."""
    w = split_swa_pool(_w(130 + bs2), block_size=bs2, seed=131)
    out, lse, _ = oracle.decode_workload(w)
    ro, rl = sdpa_reference(w)
    np.testing.assert_allclose(out, ro, rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(lse, rl, rtol=RTOL, atol=ATOL)


def test_dual_pool_equals_the_single_pool_it_was_split_from():
    w = _w(140, s_q=2)
    w2 = split_swa_pool(w, block_size=16, seed=141, page_pad=24)
    a = oracle.decode_workload(w, num_splits=3)
    b = oracle.decode_workload(w2, num_splits=3)
    assert a[2] == b[2] and np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


from hypothesis import given, settings, strategies as st, HealthCheck


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 10 ** 6), B=st.integers(1, 3), H=st.sampled_from([1, 2, 16]),
       topk=st.integers(1, 48), swa=st.integers(0, 12), bs=st.sampled_from([1, 3, 16, 64]),
       invalid=st.sampled_from([0.0, 0.2]), masked=st.booleans(), s_q=st.integers(1, 3),
       split_pool=st.booleans(), splits=st.sampled_from([0, 1, 2, 5]))
def test_random_workloads_match_sdpa(seed, B, H, topk, swa, bs, invalid, masked, s_q, split_pool,
                                     splits):
    """Random small shapes: the oracle's decode (plain, or split and merged)
    equals torch's fp64 SDPA over the rows rebuilt from the generator's own
    values, with the sink as an extra key."""
    rng = np.random.default_rng(seed)
    seq_lens = [int(x) for x in rng.integers(s_q + 1, 300, size=B)]
    w = make_custom(B=B, H=H, topk=topk, swa=swa, seq_lens=seq_lens, seed=seed, block_size=bs,
                    invalid_frac=invalid, valid_len_range=(0, topk) if masked else None,
                    keep_floats=True, s_q=s_q)
    if split_pool:
        w = split_swa_pool(w, block_size=max(1, bs // 2), seed=seed + 1)
    out, lse, _ = oracle.decode_workload(w, num_splits=splits)
    ro, rl = sdpa_reference(w)
    tol = 1e-9 if splits else RTOL
    np.testing.assert_allclose(out, ro, rtol=tol, atol=1e-11)
    np.testing.assert_allclose(lse, rl, rtol=tol, atol=1e-11)
