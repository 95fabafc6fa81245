"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/dsv4.h declares, plans every workload the way the selector rule
says, and rejects bad arguments with the documented status codes."""

import ctypes
import os
import re
import subprocess

import pytest

import sparse_mla_attention_block_amd as dsv4
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dsv4_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_symbols()
    for want in ("dsv4_sparse_decode", "dsv4_sparse_decode_partial", "dsv4_combine_splits",
                 "dsv4_convert_req_index_to_global", "dsv4_sparse_decode_plan",
                 "dsv4_sparse_decode_workspace_bytes", "dsv4_status_string", "dsv4_last_error",
                 "dsv4_gather_floor", "dsv4_quantize_store", "dsv4_gather_dequant",
                 "dsv4_dense_decode", "dsv4_decode_flags_for_cache", "dsv4_sparse_decode_dual",
                 "dsv4_sparse_decode_with_slots"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dsv4.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_library_is_built_for_gfx950_only():
    data = open(dsv4.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in data


@pytest.mark.parametrize("struct", ["dsv4_decode_desc", "dsv4_plan", "dsv4_cache_pool"])
def test_binding_structs_match_the_c_layout(struct, tmp_path):
    """Every field of the Python mirror sits at the offset a C compiler gives
    it in include/dsv4.h, and the sizes agree."""
    cls = getattr(dsv4, struct)
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"dsv4.h\"\n"
                   "int main(void) {\n"
                   + "".join(f'    printf("%zu\\n", offsetof({struct}, {f}));\n' for f in fields)
                   + f'    printf("%zu\\n", sizeof({struct}));\n    return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [getattr(cls, f).offset for f in fields] + [ctypes.sizeof(cls)]
    assert got == want


def test_tokens_per_seq_must_divide_the_batch():
    dsv4.dsv4_sparse_decode_plan(_desc(6, 64, 10, 0, tokens_per_seq=3))
    dsv4.dsv4_sparse_decode_plan(_desc(6, 64, 10, 0, tokens_per_seq=0))
    assert _status(_desc(6, 64, 10, 0, tokens_per_seq=4)) == dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert "tokens_per_seq" in dsv4.dsv4_last_error()
    assert _status(_desc(6, 64, 10, 0, tokens_per_seq=-1)) == dsv4.DSV4_ERR_INVALID_ARGUMENT


def test_unknown_decode_flags_are_rejected():
    dsv4.dsv4_sparse_decode_plan(_desc(1, 64, 10, 0, flags=dsv4.DSV4_DECODE_SCRUB))
    dsv4.dsv4_sparse_decode_plan(_desc(1, 64, 10, 0, flags=dsv4.DSV4_DECODE_PIPELINED))
    dsv4.dsv4_sparse_decode_plan(_desc(1, 64, 10, 0, flags=dsv4.DSV4_DECODE_BALANCE))
    for bad in (0x8, 0x80000000):
        assert _status(_desc(1, 64, 10, 0, flags=bad)) == dsv4.DSV4_ERR_INVALID_ARGUMENT
        assert "flags" in dsv4.dsv4_last_error()


@pytest.mark.parametrize("ci,kernel", [(0, 1), (1, 1), (2, 1), (3, 0), (4, 0)])
def test_partial_kernel_of_each_workload(ci, kernel):
    """Splits of at most 128 entries (4 tiles) with 16, 32 or 64 heads per
    workgroup run the short-split kernel, longer ones the pipelined kernel;
    the pipelined flag forces the latter."""
    c = CONFIGS[ci]
    d = _desc(c["B"], c["H"], c["topk"], c["swa"])
    plan = dsv4.dsv4_sparse_decode_plan(d, c["num_splits"])
    assert plan.partial_kernel == kernel
    Kt = c["topk"] + c["swa"]
    chunk = -(-(-(-Kt // plan.num_splits)) // 32) * 32
    assert (chunk <= 128) == (kernel == dsv4.DSV4_KERNEL_SHORT)
    d = _desc(c["B"], c["H"], c["topk"], c["swa"], flags=dsv4.DSV4_DECODE_PIPELINED)
    assert dsv4.dsv4_sparse_decode_plan(d, c["num_splits"]).partial_kernel == 0


def _desc(B, H, topk, swa, bs=64, num_blocks=1000, **kw):
    d = dict(batch=B, num_heads=H, topk=topk, swa=swa, block_size=bs, num_blocks=num_blocks,
             page_stride=bs * 584, sm_scale=512 ** -0.5, max_blocks_per_seq=16,
             block_table_stride=16)
    d.update(kw)
    return dsv4.make_desc(**d)


def _want(B, groups, Kt):
    """Splits that still give every workgroup its own CU, at most 32 and at
    most one per 32-entry tile."""
    if B >= 256:
        return 1
    return max(1, min(256 // (B * groups), 32, -(-Kt // 32)))


def _whole_tiles(want, Kt):
    tiles = -(-Kt // 32)
    return -(-tiles // -(-tiles // want))


def _expected_splits(B, groups, Kt, forced):
    return forced if forced else _whole_tiles(_want(B, groups, Kt), Kt)


def _expected_plan(B, H, Kt, forced=0):
    """(heads_per_group, splits).  Selector splits: the smallest of
    16/32/48/64 dividing H whose splits (>= 2) fill the chip (one more would
    pass 256 workgroups) with at most 8 tiles of 32 entries each.  Otherwise
    the largest group that fills the chip (forced S: B * S * groups >= 256),
    else 16."""
    if not forced:
        for hg in (16, 32, 48, 64):
            if H % hg:
                continue
            g = H // hg
            want = _want(B, g, Kt)
            S = _whole_tiles(want, Kt)
            if S >= 2 and -(-(-(-Kt // S)) // 32) <= 8 and B * g * (want + 1) > 256:
                return hg, S
    for hg in (64, 48, 32, 16):
        if H % hg:
            continue
        g = H // hg
        if forced:
            S = forced
            if B * S * g >= 256:
                break
        else:
            want = _want(B, g, Kt)
            S = _whole_tiles(want, Kt)
            if B * g * (want + 1) > 256:
                break
    return hg, S


@pytest.mark.parametrize("ci", range(5))
def test_plan_of_each_workload(ci):
    c = CONFIGS[ci]
    Kt = c["topk"] + c["swa"]
    p = dsv4.dsv4_sparse_decode_plan(_desc(c["B"], c["H"], c["topk"], c["swa"]), c["num_splits"])
    hg, S = _expected_plan(c["B"], c["H"], Kt, c["num_splits"])
    assert (p.heads_per_group, p.num_splits) == (hg, S)
    assert p.heads_per_group * p.head_groups == c["H"]
    assert p.heads_per_group <= 64 and p.heads_per_group % 16 == 0
    units = c["B"] * S
    assert p.grid_partial == -(-units // 8) * 8 * p.head_groups
    assert p.block_partial == 512
    if S > 1:
        assert p.workspace_bytes == c["B"] * c["H"] * S * (512 * 2 + 4)
        rows = c["B"] * c["H"]
        # Few rows: 4 (<= 128 rows) or 2 dim slices per row, as many waves
        # per workgroup; else one 128-thread workgroup per row.
        q = 4 if rows <= 128 else 2 if rows < 2048 else 1
        assert p.grid_combine == rows * q
        assert p.block_combine == (64 * q if q > 1 else 128)
    else:
        assert p.workspace_bytes == 0 and p.grid_combine == 0
    assert p.lds_bytes <= 160 * 1024


def test_selector_values_for_the_five_workloads():
    got = [dsv4.dsv4_sparse_decode_plan(_desc(c["B"], c["H"], c["topk"], c["swa"]),
                                        c["num_splits"]).num_splits for c in CONFIGS]
    assert got == [1, 10, 32, 1, 4]


def test_head_grouping_of_the_five_workloads():
    got = [dsv4.dsv4_sparse_decode_plan(_desc(c["B"], c["H"], c["topk"], c["swa"]),
                                        c["num_splits"]).heads_per_group for c in CONFIGS]
    assert got == [16, 16, 16, 64, 64]


@pytest.mark.parametrize("H,hg,groups", [(16, 16, 1), (32, 32, 1), (48, 48, 1), (64, 64, 1),
                                          (80, 16, 5), (96, 48, 2), (112, 16, 7), (128, 64, 2)])
def test_head_grouping_when_the_batch_fills_the_chip(H, hg, groups):
    p = dsv4.dsv4_sparse_decode_plan(_desc(256, H, 100, 0), 1)
    assert (p.heads_per_group, p.head_groups) == (hg, groups)


@pytest.mark.parametrize("H,B,S,hg", [(64, 256, 1, 64), (64, 64, 1, 16), (64, 64, 2, 32),
                                       (64, 32, 2, 16), (128, 16, 8, 64), (128, 2, 8, 16),
                                       (96, 2, 4, 16), (96, 64, 2, 48)])
def test_head_grouping_shrinks_while_cus_would_idle(H, B, S, hg):
    p = dsv4.dsv4_sparse_decode_plan(_desc(B, H, 1000, 0), S)
    assert p.heads_per_group == hg == _expected_plan(B, H, 1000, S)[0]
    assert p.head_groups * p.heads_per_group == H


def _status(desc, splits=0):
    with pytest.raises(dsv4.Dsv4Error) as e:
        dsv4.dsv4_sparse_decode_plan(desc, splits)
    return e.value.status


def test_validation_errors():
    E = dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert _status(_desc(0, 64, 10, 0)) == E
    assert _status(_desc(1, 24, 10, 0)) == E            # not a multiple of 16
    assert _status(_desc(1, 144, 10, 0)) == E           # more than 128
    assert _status(_desc(1, 64, 0, 0)) == E             # nothing to attend
    assert _status(_desc(1, 64, -1, 5)) == E
    assert _status(_desc(1, 64, 10, 0, bs=0)) == E
    assert _status(_desc(1, 64, 10, 0, num_blocks=0)) == E
    assert _status(_desc(1, 64, 10, 0, page_stride=64 * 584 - 8)) == E
    assert _status(_desc(1, 64, 10, 0, page_stride=64 * 584 + 4)) == E
    assert _status(_desc(1, 64, 10, 2, topk_idx_stride=11)) == E
    assert _status(_desc(1, 64, 10, 0), 65) == E
    assert _status(_desc(1, 64, 10, 0), -1) == E
    assert _status(_desc(1, 136, 10, 0)) == E
    assert "num_heads" in dsv4.dsv4_last_error()


def test_workspace_bytes():
    d = _desc(4, 64, 512, 128)
    assert dsv4.dsv4_sparse_decode_workspace_bytes(d, 1) == 0
    assert dsv4.dsv4_sparse_decode_workspace_bytes(d, 4) == 4 * 64 * 4 * (512 * 2 + 4)
    assert dsv4.dsv4_sparse_decode_workspace_bytes(_desc(0, 64, 1, 0), 4) == 0   # invalid


def test_decode_rejects_null_and_missing_workspace_without_touching_the_gpu():
    d = _desc(1, 64, 100, 0)
    fake = ctypes.c_void_p(4096)
    st = dsv4._lib.dsv4_sparse_decode(ctypes.byref(d), None, fake, None, fake, None, None, fake,
                                      None, 1, None)
    assert st == dsv4.DSV4_ERR_INVALID_ARGUMENT
    st = dsv4._lib.dsv4_sparse_decode(ctypes.byref(d), fake, fake, None, fake, None, None, fake,
                                      None, 4, None)
    assert st == dsv4.DSV4_ERR_WORKSPACE_TOO_SMALL
    st = dsv4._lib.dsv4_sparse_decode(ctypes.byref(d), ctypes.c_void_p(4100), fake, None, fake,
                                      None, None, fake, None, 1, None)
    assert st == dsv4.DSV4_ERR_INVALID_ARGUMENT          # q misaligned
    st = dsv4._lib.dsv4_convert_req_index_to_global(None, 1, None, 4, 4, fake, 4, 1, 4, 64, None,
                                                    -1, fake, None)
    assert st == dsv4.DSV4_ERR_INVALID_ARGUMENT          # no block table
    assert dsv4._lib.dsv4_convert_req_index_to_global(None, 1, fake, 4, 4, fake, 4, 0, 4, 64,
                                                      None, -1, fake, None) == dsv4.DSV4_OK
    assert dsv4._lib.dsv4_combine_splits(1, 64, 0, fake, fake, None, fake, None, None) == \
        dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert dsv4.dsv4_status_string(3) == "DSV4_ERR_WORKSPACE_TOO_SMALL"


def test_decode_with_slots_validation_without_touching_the_gpu():
    d = _desc(1, 64, 100, 0)
    d.max_blocks_per_seq, d.block_table_stride = 2, 2
    fake = ctypes.c_void_p(4096)
    f = dsv4._lib.dsv4_sparse_decode_with_slots
    # no block table, no slots buffer, a misaligned slots buffer
    assert f(ctypes.byref(d), fake, fake, None, fake, None, None, fake, None, 1, fake,
             None) == dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, None, 1, None,
             None) == dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, None, 1,
             ctypes.c_void_p(4098), None) == dsv4.DSV4_ERR_INVALID_ARGUMENT
    assert "global_slots" in dsv4.dsv4_last_error()
    # the decode's own checks still apply (split partials need a workspace)
    assert f(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, None, 4, fake,
             None) == dsv4.DSV4_ERR_WORKSPACE_TOO_SMALL


def test_writer_validation_without_touching_the_gpu():
    lib = dsv4._lib
    fake = ctypes.c_void_p(4096)
    E = dsv4.DSV4_ERR_INVALID_ARGUMENT
    S = dsv4.DSV4_STORE_SANITIZE
    assert lib.dsv4_quantize_store(fake, 512, fake, 0, fake, 64, 10, 64 * 584, S, None) == 0
    assert lib.dsv4_quantize_store(None, 512, fake, 4, fake, 64, 10, 64 * 584, S, None) == E
    assert lib.dsv4_quantize_store(fake, 512, fake, 4, fake, 64, 10, 64 * 584, 0x2, None) == E
    assert "flags" in dsv4.dsv4_last_error()
    assert lib.dsv4_quantize_store(fake, 500, fake, 4, fake, 64, 10, 64 * 584, S, None) == E
    assert lib.dsv4_quantize_store(fake, 516, fake, 4, fake, 64, 10, 64 * 584, S, None) == E
    assert lib.dsv4_quantize_store(fake, 512, fake, 4, fake, 64, 10, 64 * 584 - 8, S, None) == E
    assert lib.dsv4_quantize_store(fake, 512, fake, 4, fake, 0, 10, 64 * 584, S, None) == E
    assert lib.dsv4_quantize_store(fake, 512, fake, 4, fake, 64, 0, 64 * 584, S, None) == E
    assert lib.dsv4_quantize_store(ctypes.c_void_p(4104), 512, fake, 4, fake, 64, 10, 64 * 584,
                                   S, None) == E          # rows misaligned
    assert lib.dsv4_quantize_store(fake, 512, fake, -1, fake, 64, 10, 64 * 584, S, None) == E


def test_two_kernel_path_validation_without_touching_the_gpu():
    lib = dsv4._lib
    fake = ctypes.c_void_p(4096)
    E = dsv4.DSV4_ERR_INVALID_ARGUMENT
    d = _desc(2, 64, 100, 20)
    assert lib.dsv4_gather_dequant(ctypes.byref(d), fake, None, fake, None, None, fake, None) == E
    assert lib.dsv4_gather_dequant(ctypes.byref(d), fake, None, fake, None, ctypes.c_void_p(4104),
                                   fake, None) == E                       # kv_out misaligned
    assert lib.dsv4_dense_decode(ctypes.byref(d), fake, fake, None, None, fake, None, 1, None) == E
    assert lib.dsv4_dense_decode(ctypes.byref(d), fake, fake, fake, None, fake, None, 4,
                                 None) == dsv4.DSV4_ERR_WORKSPACE_TOO_SMALL
    ds = _desc(2, 64, 100, 20, flags=dsv4.DSV4_DECODE_SCRUB)
    assert lib.dsv4_dense_decode(ctypes.byref(ds), fake, fake, fake, None, fake, None, 1, None) == E


def test_provenance_gate_truth_table():
    """The scrub may be skipped for exactly one of the 16 provenances: an
    fp8_ds_mla cache with its extra cache, no KV transfer and a sanitising
    writer."""
    import itertools
    for fmt, xfer, extra, san in itertools.product((False, True), repeat=4):
        flags = dsv4.dsv4_decode_flags_for_cache(cache_is_fp8_ds_mla=fmt, has_kv_transfer=xfer,
                                                 has_extra_cache=extra, writer_sanitizes=san)
        trusted = fmt and not xfer and extra and san
        assert flags == (0 if trusted else dsv4.DSV4_DECODE_SCRUB), (fmt, xfer, extra, san)


def test_dual_cache_validation_without_touching_the_gpu():
    lib = dsv4._lib
    fake = ctypes.c_void_p(4096)
    E = dsv4.DSV4_ERR_INVALID_ARGUMENT
    d = _desc(2, 64, 100, 20)

    def pool(bt=fake, bs=64, nb=10, stride=64 * 584, kv=fake):
        pl = dsv4.dsv4_cache_pool()
        pl.kv_cache, pl.block_table = kv, bt
        pl.num_blocks, pl.page_stride, pl.block_table_stride = nb, stride, 16
        pl.block_size, pl.max_blocks_per_seq = bs, 16
        return pl

    def call(a, b, q=fake):
        return lib.dsv4_sparse_decode_dual(ctypes.byref(d), q, ctypes.byref(a), ctypes.byref(b),
                                           fake, None, None, fake, None, 1, None)
    assert call(pool(), pool(bt=None)) == E              # tables on one side only
    assert call(pool(), pool(bs=0)) == E
    assert call(pool(), pool(stride=16 * 584)) == E      # stride below block_size * 584
    assert call(pool(kv=None), pool()) == E
    assert call(pool(), pool(), q=None) == E
    assert "swa pool" in (call(pool(), pool(nb=0)) == E and dsv4.dsv4_last_error())


@pytest.mark.parametrize("B,hg,S", [(1, 16, 32), (2, 16, 32), (4, 16, 16), (8, 16, 8),
                                     (16, 32, 8), (32, 64, 8), (64, 64, 4), (256, 64, 1)])
def test_selector_on_the_headline_shape_across_batch_sizes(B, hg, S):
    """H=64, top-k 2048: the groupings a batch sweep on the GPU measured
    fastest (B = 4, 8, 16 gain 10-24 % over the largest filling group)."""
    p = dsv4.dsv4_sparse_decode_plan(_desc(B, 64, 2048, 0), 0)
    assert (p.heads_per_group, p.num_splits) == (hg, S) == _expected_plan(B, 64, 2048)


@pytest.mark.parametrize("H", [16, 64, 128])
def test_selector_never_asks_for_a_second_round_of_workgroups(H):
    """One partial workgroup fills a compute unit: an auto plan keeps
    B * S * head_groups within the 256 CUs unless B * head_groups alone
    exceeds them, and each split holds whole tiles with none left empty."""
    for B in (1, 2, 3, 4, 5, 7, 12, 33, 100, 255, 256, 300):
        for Kt in (17, 128, 640, 1000, 2048, 2176, 9000):
            p = dsv4.dsv4_sparse_decode_plan(_desc(B, H, Kt, 0), 0)
            assert (p.heads_per_group, p.num_splits) == _expected_plan(B, H, Kt)
            real = B * p.num_splits * p.head_groups
            assert real <= max(256, B * p.head_groups)
            tiles = -(-Kt // 32)
            per = -(-tiles // p.num_splits)
            assert -(-tiles // per) == p.num_splits          # no split without entries


def test_short_timeline_refuses_other_kernels_without_touching_the_gpu():
    """The phase timeline exists for the short-split kernel only: a plan that
    picks the pipelined kernel (the large batch) or the scrub flag is refused
    before any pointer is looked at."""
    import ctypes
    c = CONFIGS[3]
    d = _desc(c["B"], c["H"], c["topk"], c["swa"])
    assert dsv4.dsv4_sparse_decode_plan(d, 0).partial_kernel == dsv4.DSV4_KERNEL_PIPELINED
    st = dsv4._lib.dsv4_short_timeline(ctypes.byref(d), None, None, None, None, None, None, None,
                                      None, 0, None, None)
    assert st == dsv4.DSV4_ERR_NOT_SUPPORTED and "short-split" in dsv4.dsv4_last_error()
    d = _desc(1, 64, 2048, 0, flags=dsv4.DSV4_DECODE_SCRUB)
    st = dsv4._lib.dsv4_short_timeline(ctypes.byref(d), None, None, None, None, None, None, None,
                                      None, 0, None, None)
    assert st == dsv4.DSV4_ERR_NOT_SUPPORTED


def test_make_pool_keeps_its_tensors_alive():
    """The pool struct carries raw pointers; the binding keeps the tensors
    they point into referenced for as long as the pool lives."""
    import gc
    import weakref
    import torch
    kv = torch.zeros((4, 64 * 584), dtype=torch.uint8)
    bt = torch.zeros((2, 3), dtype=torch.int32)
    refs = weakref.ref(kv), weakref.ref(bt)
    pl = dsv4.make_pool(kv, bt, block_size=64, max_blocks_per_seq=3)
    del kv, bt
    gc.collect()
    assert refs[0]() is not None and refs[1]() is not None
    assert pl.kv_cache == refs[0]().data_ptr() and pl.num_blocks == 4
    del pl
    gc.collect()
    assert refs[0]() is None and refs[1]() is None
