"""Python binding of libdsv4.so, the MI355X sparse FP8 MLA decode library.

Argument marshalling only: each dsv4_* function here has the name of a C
entry point in include/dsv4.h, turns torch tensors into device pointers and
calls it through ctypes; make_desc, make_pool and workspace_split_views only
fill the ABI's structs or view a workspace.  Every step of the path runs in the HIP kernels; there is
no CPU or PyTorch fallback.  If the library has not been built, importing
this package fails.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsv4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m sparse_mla_attention_block_amd.build` "
        "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

DSV4_OK = 0
DSV4_ERR_INVALID_ARGUMENT = 1
DSV4_ERR_NOT_SUPPORTED = 2
DSV4_ERR_WORKSPACE_TOO_SMALL = 3
DSV4_ERR_HIP = 4
MAX_SPLITS = 64
DSV4_DECODE_SCRUB = 0x1
DSV4_DECODE_PIPELINED = 0x2
DSV4_DECODE_BALANCE = 0x4
DSV4_KERNEL_PIPELINED = 0
DSV4_KERNEL_SHORT = 1
DSV4_STORE_SANITIZE = 0x1


class dsv4_decode_desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("swa", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("topk_idx_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("tokens_per_seq", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class dsv4_cache_pool(ctypes.Structure):
    _fields_ = [
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
    ]


def make_pool(kv_cache: torch.Tensor, block_table: Optional[torch.Tensor], *, block_size: int,
              max_blocks_per_seq: int = 0) -> dsv4_cache_pool:
    """A pool over a [num_blocks, page_stride] uint8 cache tensor.  The pool
    holds references to both tensors, so their memory stays allocated while
    the pool is in use."""
    pl = dsv4_cache_pool()
    pl._tensors = (kv_cache, block_table)
    pl.kv_cache = kv_cache.data_ptr()
    pl.block_table = block_table.data_ptr() if block_table is not None else None
    pl.num_blocks, pl.page_stride = kv_cache.shape[0], kv_cache.shape[1]
    pl.block_table_stride = block_table.shape[1] if block_table is not None else 0
    pl.block_size = block_size
    pl.max_blocks_per_seq = max_blocks_per_seq
    return pl


class dsv4_plan(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32),
        ("heads_per_group", ctypes.c_int32),
        ("head_groups", ctypes.c_int32),
        ("tile_entries", ctypes.c_int32),
        ("grid_partial", ctypes.c_int64),
        ("block_partial", ctypes.c_int32),
        ("grid_combine", ctypes.c_int64),
        ("block_combine", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("lds_bytes", ctypes.c_size_t),
        ("partial_kernel", ctypes.c_int32),
        ("balanced_splits", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_P = ctypes.c_void_p
_DESC = ctypes.POINTER(dsv4_decode_desc)
_lib.dsv4_status_string.argtypes = [ctypes.c_int]
_lib.dsv4_status_string.restype = ctypes.c_char_p
_lib.dsv4_last_error.argtypes = []
_lib.dsv4_last_error.restype = ctypes.c_char_p
_lib.dsv4_sparse_decode_plan.argtypes = [_DESC, ctypes.c_int32, ctypes.POINTER(dsv4_plan)]
_lib.dsv4_sparse_decode_plan.restype = ctypes.c_int
_lib.dsv4_sparse_decode_workspace_bytes.argtypes = [_DESC, ctypes.c_int32]
_lib.dsv4_sparse_decode_workspace_bytes.restype = ctypes.c_size_t
NOALLOC_SCRATCH_BYTES = 32 << 20
for _name in ("dsv4_sparse_decode", "dsv4_sparse_decode_partial", "dsv4_sparse_decode_noalloc"):
    _f = getattr(_lib, _name)
    _f.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P]
    _f.restype = ctypes.c_int
_lib.dsv4_combine_splits.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                     _P, _P, _P]
_lib.dsv4_combine_splits.restype = ctypes.c_int
_lib.dsv4_convert_req_index_to_global.argtypes = [
    _P, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int32,
    ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P]
_lib.dsv4_convert_req_index_to_global.restype = ctypes.c_int
_lib.dsv4_gather_floor.argtypes = [_DESC, _P, _P, _P, _P, ctypes.c_int32, _P, _P]
_lib.dsv4_gather_floor.restype = ctypes.c_int
_lib.dsv4_short_timeline.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P]
_lib.dsv4_sparse_decode_with_slots.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_int32, _P, _P]
_lib.dsv4_sparse_decode_with_slots.restype = ctypes.c_int
_lib.dsv4_sparse_decode_partial_with_slots.argtypes = _lib.dsv4_sparse_decode_with_slots.argtypes
_lib.dsv4_sparse_decode_partial_with_slots.restype = ctypes.c_int
_lib.dsv4_short_timeline.restype = ctypes.c_int
_lib.dsv4_decode_flags_for_cache.argtypes = [ctypes.c_int32] * 4
_lib.dsv4_decode_flags_for_cache.restype = ctypes.c_uint32
_lib.dsv4_sparse_decode_dual.argtypes = [_DESC, _P, ctypes.POINTER(dsv4_cache_pool),
                                         ctypes.POINTER(dsv4_cache_pool), _P, _P, _P, _P, _P,
                                         ctypes.c_int32, _P]
_lib.dsv4_sparse_decode_dual.restype = ctypes.c_int
_lib.dsv4_gather_dequant.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P]
_lib.dsv4_gather_dequant.restype = ctypes.c_int
_lib.dsv4_dense_decode.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P]
_lib.dsv4_dense_decode.restype = ctypes.c_int
_lib.dsv4_quantize_store.argtypes = [_P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32, _P]
_lib.dsv4_quantize_store.restype = ctypes.c_int


class Dsv4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{dsv4_status_string(status)}: {message}")
        self.status = status


def dsv4_status_string(status: int) -> str:
    return _lib.dsv4_status_string(status).decode()


def dsv4_last_error() -> str:
    return _lib.dsv4_last_error().decode()


def _check(status: int) -> None:
    if status != DSV4_OK:
        raise Dsv4Error(status, dsv4_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def make_desc(*, batch: int, num_heads: int, topk: int, swa: int, block_size: int,
              num_blocks: int, page_stride: int, sm_scale: float, max_blocks_per_seq: int = 0,
              block_table_stride: int = 0, topk_idx_stride: int = 0,
              workspace: Optional[torch.Tensor] = None, flags: int = 0,
              tokens_per_seq: int = 1) -> dsv4_decode_desc:
    d = dsv4_decode_desc()
    d.batch, d.num_heads, d.topk, d.swa = batch, num_heads, topk, swa
    d.block_size, d.max_blocks_per_seq = block_size, max_blocks_per_seq
    d.num_blocks, d.block_table_stride, d.page_stride = num_blocks, block_table_stride, page_stride
    d.topk_idx_stride = topk_idx_stride
    d.sm_scale = sm_scale
    d.flags = flags
    d.tokens_per_seq = tokens_per_seq
    if workspace is not None:
        d.workspace = workspace.data_ptr()
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    return d


def dsv4_sparse_decode_plan(desc: dsv4_decode_desc, num_splits: int = 0) -> dsv4_plan:
    plan = dsv4_plan()
    _check(_lib.dsv4_sparse_decode_plan(ctypes.byref(desc), num_splits, ctypes.byref(plan)))
    return plan


def dsv4_sparse_decode_workspace_bytes(desc: dsv4_decode_desc, num_splits: int = 0) -> int:
    return int(_lib.dsv4_sparse_decode_workspace_bytes(ctypes.byref(desc), num_splits))


def dsv4_sparse_decode(desc: dsv4_decode_desc, q: torch.Tensor, kv_cache: torch.Tensor,
                       block_table: Optional[torch.Tensor], topk_idx: torch.Tensor,
                       valid_len: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                       out: torch.Tensor, lse: Optional[torch.Tensor], num_splits: int = 0,
                       stream=None) -> None:
    _check(_lib.dsv4_sparse_decode(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   _ptr(topk_idx), _ptr(valid_len), _ptr(sink), _ptr(out),
                                   _ptr(lse), num_splits, _stream(stream)))


def dsv4_sparse_decode_noalloc(desc: dsv4_decode_desc, q: torch.Tensor, kv_cache: torch.Tensor,
                               block_table: Optional[torch.Tensor], topk_idx: torch.Tensor,
                               valid_len: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                               out: torch.Tensor, lse: Optional[torch.Tensor], num_splits: int = 0,
                               stream=None) -> None:
    _check(_lib.dsv4_sparse_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(kv_cache),
                                           _ptr(block_table), _ptr(topk_idx), _ptr(valid_len),
                                           _ptr(sink), _ptr(out), _ptr(lse), num_splits,
                                           _stream(stream)))


def dsv4_sparse_decode_with_slots(desc: dsv4_decode_desc, q: torch.Tensor,
                                  kv_cache: torch.Tensor, block_table: torch.Tensor,
                                  topk_idx: torch.Tensor, valid_len: Optional[torch.Tensor],
                                  sink: Optional[torch.Tensor], out: torch.Tensor,
                                  lse: Optional[torch.Tensor], num_splits: int,
                                  global_slots: torch.Tensor, stream=None) -> None:
    """dsv4_sparse_decode through the block table that also writes the global
    slots of topk_idx (int32 [B, topk + swa], fill -1) into `global_slots`."""
    _check(_lib.dsv4_sparse_decode_with_slots(ctypes.byref(desc), _ptr(q), _ptr(kv_cache),
                                              _ptr(block_table), _ptr(topk_idx), _ptr(valid_len),
                                              _ptr(sink), _ptr(out), _ptr(lse), num_splits,
                                              _ptr(global_slots), _stream(stream)))


def dsv4_sparse_decode_partial_with_slots(desc: dsv4_decode_desc, q: torch.Tensor,
                                          kv_cache: torch.Tensor, block_table: torch.Tensor,
                                          topk_idx: torch.Tensor,
                                          valid_len: Optional[torch.Tensor],
                                          sink: Optional[torch.Tensor], out: torch.Tensor,
                                          lse: Optional[torch.Tensor], num_splits: int,
                                          global_slots: torch.Tensor, stream=None) -> None:
    """First stage of dsv4_sparse_decode_with_slots alone."""
    _check(_lib.dsv4_sparse_decode_partial_with_slots(
        ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(topk_idx),
        _ptr(valid_len), _ptr(sink), _ptr(out), _ptr(lse), num_splits, _ptr(global_slots),
        _stream(stream)))


def dsv4_sparse_decode_partial(desc: dsv4_decode_desc, q: torch.Tensor, kv_cache: torch.Tensor,
                               block_table: Optional[torch.Tensor], topk_idx: torch.Tensor,
                               valid_len: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                               out: torch.Tensor, lse: Optional[torch.Tensor],
                               num_splits: int = 0, stream=None) -> None:
    _check(_lib.dsv4_sparse_decode_partial(ctypes.byref(desc), _ptr(q), _ptr(kv_cache),
                                           _ptr(block_table), _ptr(topk_idx), _ptr(valid_len),
                                           _ptr(sink), _ptr(out), _ptr(lse), num_splits,
                                           _stream(stream)))


def dsv4_combine_splits(batch: int, num_heads: int, num_splits: int, part_out: torch.Tensor,
                        part_lse: torch.Tensor, sink: Optional[torch.Tensor], out: torch.Tensor,
                        lse: Optional[torch.Tensor], stream=None) -> None:
    _check(_lib.dsv4_combine_splits(batch, num_heads, num_splits, _ptr(part_out), _ptr(part_lse),
                                    _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def dsv4_convert_req_index_to_global(req_id: Optional[torch.Tensor], num_reqs: int,
                                     block_table: torch.Tensor, bt_stride: int,
                                     max_blocks_per_req: int, token_indices: torch.Tensor,
                                     ti_stride: int, num_tokens: int, width: int, block_size: int,
                                     cu_seqlens: Optional[torch.Tensor], invalid_fill: int,
                                     out: torch.Tensor, stream=None) -> None:
    _check(_lib.dsv4_convert_req_index_to_global(
        _ptr(req_id), num_reqs, _ptr(block_table), bt_stride, max_blocks_per_req,
        _ptr(token_indices), ti_stride, num_tokens, width, block_size, _ptr(cu_seqlens),
        invalid_fill, _ptr(out), _stream(stream)))


def dsv4_decode_flags_for_cache(*, cache_is_fp8_ds_mla: bool, has_kv_transfer: bool,
                                has_extra_cache: bool, writer_sanitizes: bool) -> int:
    return int(_lib.dsv4_decode_flags_for_cache(int(cache_is_fp8_ds_mla), int(has_kv_transfer),
                                                int(has_extra_cache), int(writer_sanitizes)))


def dsv4_sparse_decode_dual(desc, q: torch.Tensor, main_pool: dsv4_cache_pool,
                            swa_pool: dsv4_cache_pool, topk_idx: torch.Tensor,
                            valid_len: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                            out: torch.Tensor, lse: Optional[torch.Tensor], num_splits: int = 0,
                            stream=None) -> None:
    _check(_lib.dsv4_sparse_decode_dual(ctypes.byref(desc), _ptr(q), ctypes.byref(main_pool),
                                        ctypes.byref(swa_pool), _ptr(topk_idx), _ptr(valid_len),
                                        _ptr(sink), _ptr(out), _ptr(lse), num_splits,
                                        _stream(stream)))


def dsv4_gather_dequant(desc, kv_cache: torch.Tensor, block_table: Optional[torch.Tensor],
                        topk_idx: torch.Tensor, valid_len: Optional[torch.Tensor],
                        kv_out: torch.Tensor, mask_out: torch.Tensor, stream=None) -> None:
    _check(_lib.dsv4_gather_dequant(ctypes.byref(desc), _ptr(kv_cache), _ptr(block_table),
                                    _ptr(topk_idx), _ptr(valid_len), _ptr(kv_out), _ptr(mask_out),
                                    _stream(stream)))


def dsv4_dense_decode(desc, q: torch.Tensor, kv_dense: torch.Tensor, mask: torch.Tensor,
                      sink: Optional[torch.Tensor], out: torch.Tensor, lse: Optional[torch.Tensor],
                      num_splits: int = 0, stream=None) -> None:
    _check(_lib.dsv4_dense_decode(ctypes.byref(desc), _ptr(q), _ptr(kv_dense), _ptr(mask),
                                  _ptr(sink), _ptr(out), _ptr(lse), num_splits, _stream(stream)))


def dsv4_quantize_store(rows: torch.Tensor, row_stride: int, slot_mapping: torch.Tensor,
                        num_rows: int, kv_cache: torch.Tensor, block_size: int, num_blocks: int,
                        page_stride: int, flags: int = DSV4_STORE_SANITIZE, stream=None) -> None:
    _check(_lib.dsv4_quantize_store(_ptr(rows), row_stride, _ptr(slot_mapping), num_rows,
                                    _ptr(kv_cache), block_size, num_blocks, page_stride, flags,
                                    _stream(stream)))


def dsv4_gather_floor(desc, kv_cache: torch.Tensor, block_table: Optional[torch.Tensor],
                      topk_idx: torch.Tensor, valid_len: Optional[torch.Tensor], num_splits: int,
                      words: torch.Tensor, stream=None) -> None:
    """Gather floor of the partial kernel (include/dsv4_diag.h): same grid, same
    row loads, no arithmetic; `words` is int32/uint32 [grid_partial * 512]."""
    _check(_lib.dsv4_gather_floor(ctypes.byref(desc), _ptr(kv_cache), _ptr(block_table),
                                  _ptr(topk_idx), _ptr(valid_len), num_splits, _ptr(words),
                                  _stream(stream)))


def dsv4_short_timeline(desc, q: torch.Tensor, kv_cache: torch.Tensor,
                        block_table: Optional[torch.Tensor], topk_idx: torch.Tensor,
                        valid_len: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                        out: torch.Tensor, lse: Optional[torch.Tensor], num_splits: int,
                        stamps: torch.Tensor, stream=None) -> None:
    """Phase timeline of the short-split kernel (include/dsv4_diag.h): the
    first decode stage with 10 stamps per workgroup written to `stamps`
    (int64 [plan.grid_partial * 10])."""
    _check(_lib.dsv4_short_timeline(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                    _ptr(topk_idx), _ptr(valid_len), _ptr(sink), _ptr(out),
                                    _ptr(lse), num_splits, _ptr(stamps), _stream(stream)))


def workspace_split_views(workspace: torch.Tensor, batch: int, num_heads: int,
                          num_splits: int):
    """(part_out bf16 [B,H,S,512], part_lse float32 [B,H,S]) views of a decode
    workspace (a flat uint8 tensor), as laid out by dsv4_sparse_decode_partial."""
    n = batch * num_heads * num_splits
    w = workspace.view(torch.uint8)
    part_out = w[: n * 1024].view(torch.bfloat16).view(batch, num_heads, num_splits, 512)
    part_lse = w[n * 1024: n * 1028].view(torch.float32).view(batch, num_heads, num_splits)
    return part_out, part_lse
