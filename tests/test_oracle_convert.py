"""Pins of the oracle's req-local -> global conversion: values worked out by
hand from the conversion rule on the vLLM PR #41217 page (key source
snippets: block = idx / BLOCK_SIZE, offset = idx % BLOCK_SIZE, invalid ->
fill, ragged store from the token's sequence start), an identity table, and
the edge rules."""

import numpy as np

import oracle

BT = np.array([[3, 9, -1, 5],
               [0, 1, 2, 3]], dtype=np.int32)
TI = np.array([[0, 5, 9, 16, -1],
               [6, 8, 13, 3, 100]], dtype=np.int32)
REQ = np.array([1, 0], dtype=np.int32)


def test_hand_worked_dense():
    # token 0 uses request 1 (identity pages); token 1 uses request 0.
    #   0 -> blk 0 page 0 -> 0;  5 -> blk 1 page 1 -> 5;  9 -> blk 2 page 2 -> 9
    #  16 -> blk 4 >= 4 -> fill; -1 -> fill
    #   6 -> blk 1 page 9 -> 38; 8 -> blk 2 page -1 -> fill; 13 -> blk 3 page 5 -> 21
    #   3 -> blk 0 page 3 -> 15; 100 -> blk 25 -> fill
    for fill in (0, -1):
        f = fill
        want = np.array([[0, 5, 9, f, f], [38, f, 21, 15, f]], dtype=np.int32)
        got = oracle.convert_req_index_to_global(token_indices=TI, block_table=BT,
                                                 max_blocks_per_req=4, block_size=4, req_id=REQ,
                                                 invalid_fill=fill)
        assert np.array_equal(got, want)


def test_hand_worked_ragged():
    cu = np.array([0, 3, 5], dtype=np.int32)   # token 0 keeps 3 entries, token 1 keeps 2
    got = oracle.convert_req_index_to_global(token_indices=TI, block_table=BT,
                                             max_blocks_per_req=4, block_size=4, req_id=REQ,
                                             cu_seqlens=cu, invalid_fill=-1)
    assert np.array_equal(got, np.array([0, 5, 9, 38, -1], dtype=np.int32))


def test_ragged_longer_than_width_stops_at_width():
    cu = np.array([0, 9, 10], dtype=np.int32)  # token 0 claims 9 > width 5
    got = oracle.convert_req_index_to_global(token_indices=TI, block_table=BT,
                                             max_blocks_per_req=4, block_size=4, req_id=REQ,
                                             cu_seqlens=cu, invalid_fill=-1)
    sentinel = np.iinfo(np.int32).min
    assert np.array_equal(got[:5], [0, 5, 9, -1, -1])
    assert np.all(got[5:9] == sentinel)         # never written
    assert got[9] == 38


def test_identity_table_is_identity():
    rng = np.random.default_rng(0)
    bs, nb = 64, 50
    bt = np.tile(np.arange(nb, dtype=np.int32), (3, 1))
    ti = rng.integers(-3, nb * bs, size=(3, 200)).astype(np.int32)
    got = oracle.convert_req_index_to_global(token_indices=ti, block_table=bt,
                                             max_blocks_per_req=nb, block_size=bs,
                                             invalid_fill=-1)
    assert np.array_equal(got, np.where(ti >= 0, ti, -1))


def test_block_size_one_maps_through_the_table():
    bt = np.array([[7, 3, 11]], dtype=np.int32)
    ti = np.array([[2, 0, 1, 3]], dtype=np.int32)
    got = oracle.convert_req_index_to_global(token_indices=ti, block_table=bt,
                                             max_blocks_per_req=3, block_size=1, invalid_fill=-2)
    assert np.array_equal(got, [[11, 7, 3, -2]])


def test_overflow_and_bad_request_give_fill():
    bt = np.array([[1 << 30, 5]], dtype=np.int32)
    ti = np.array([[1, 4], [1, 4]], dtype=np.int32)
    got = oracle.convert_req_index_to_global(token_indices=ti, block_table=bt,
                                             max_blocks_per_req=2, block_size=4,
                                             req_id=np.array([0, 3], np.int32), num_reqs=1,
                                             invalid_fill=-1)
    # 2^30*4 + 1 does not fit in int32; request 3 is outside the table.
    assert np.array_equal(got, [[-1, 20], [-1, -1]])
