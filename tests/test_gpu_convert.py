"""Index conversion on the GPU: bit-exact against the oracle."""

import numpy as np
import pytest

import oracle
from synth import make_workload
from synth.workloads import make_convert_case

pytestmark = pytest.mark.gpu


def _both(**kw):
    from tests.gpu_helpers import gpu_convert
    want = oracle.convert_req_index_to_global(**kw)
    got = gpu_convert(**kw)
    return got, want


@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("fill", [0, -1])
@pytest.mark.parametrize("bs,T,width", [(64, 7, 300), (1, 5, 700), (16, 33, 2048), (64, 1, 1)])
def test_random_cases_bit_exact(ragged, fill, bs, T, width):
    c = make_convert_case(seed=T * 131 + width + bs, num_tokens=T, width=width, block_size=bs,
                          num_reqs=9, max_blocks=max(1, 4096 // bs), ragged=ragged)
    kw = dict(token_indices=c.token_indices, block_table=c.block_table,
              max_blocks_per_req=c.max_blocks, block_size=bs, width=c.width, req_id=c.req_id,
              num_reqs=c.block_table.shape[0], cu_seqlens=c.cu_seqlens, invalid_fill=fill)
    got, want = _both(**kw)
    print(f"convert bs={bs} T={T} width={width} ragged={ragged} fill={fill}", flush=True)
    assert np.array_equal(got, want)


def test_overflow_negative_pages_and_missing_req_ids():
    bt = np.array([[1 << 30, 5, -4]], dtype=np.int32)
    ti = np.array([[1, 4, 9, -1, 12, 2_000_000_000]], dtype=np.int32)
    got, want = _both(token_indices=ti, block_table=bt, max_blocks_per_req=3, block_size=4,
                      invalid_fill=-1)
    assert np.array_equal(got, want)
    assert np.array_equal(got, [[-1, 20, -1, -1, -1, -1]])


@pytest.mark.parametrize("ci", range(5))
def test_workload_index_lists_bit_exact(ci):
    """The req-local lists of every decode workload, converted with fill -1."""
    w = make_workload(ci)
    kw = dict(token_indices=w.topk_idx, block_table=w.block_table,
              max_blocks_per_req=w.max_blocks_per_seq, block_size=w.block_size,
              invalid_fill=-1)
    print(f"convert workload {ci} {w.name}", flush=True)
    got, want = _both(**kw)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ragged", [False, True])
def test_rows_wider_than_one_grid_of_column_tiles(ragged):
    """Rows of 65535 x 256 + 1000 columns: more 256-column tiles than one grid
    dimension holds, so the kernel walks the columns in grid strides."""
    width = 65535 * 256 + 1000
    rng = np.random.default_rng(4242 + ragged)
    bs, mb, T = 64, 512, 2
    bt = rng.integers(-1, 1 << 20, size=(3, mb)).astype(np.int32)
    ti = rng.integers(-2, bs * mb + 100, size=(T, width)).astype(np.int32)
    kw = dict(token_indices=ti, block_table=bt, max_blocks_per_req=mb, block_size=bs,
              invalid_fill=-1, req_id=np.array([2, 0], dtype=np.int32), num_reqs=3)
    if ragged:
        kw["cu_seqlens"] = np.array([0, width - 7, 2 * width - 300], dtype=np.int32)
        kw["width"] = width
    print(f"convert width={width} ragged={ragged}", flush=True)
    got, want = _both(**kw)
    assert np.array_equal(got, want)
