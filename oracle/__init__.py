"""ctypes front end of the plain fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library under ``sparse_mla_attention_block_amd``) never loads
it, and the two share no code: the oracle decodes bytes and computes
attention with its own C.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
# A prebuilt oracle library to load instead (e.g. a sanitizer build made by
# the tests); it is used as is, never rebuilt.
_LIB_OVERRIDE = os.environ.get("DSV4_ORACLE_LIB")

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", tmp,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class OrcDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("swa", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_double),
        ("scrub", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
    ]


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or LIB_PATH
        if not _LIB_OVERRIDE and (not os.path.exists(LIB_PATH)
                                  or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC)):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.orc_e4m3fn.argtypes = [ctypes.c_uint8]
        L.orc_e4m3fn.restype = ctypes.c_double
        L.orc_ue8m0.argtypes = [ctypes.c_uint8]
        L.orc_ue8m0.restype = ctypes.c_double
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_bf16.restype = ctypes.c_double
        L.orc_resolve.argtypes = [ctypes.POINTER(OrcDesc), P, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
        L.orc_resolve.restype = ctypes.c_int
        L.orc_dequant_row.argtypes = [ctypes.POINTER(OrcDesc), P, ctypes.c_int64, ctypes.c_int32, P]
        L.orc_dequant_row.restype = None
        L.orc_sparse_decode.argtypes = [ctypes.POINTER(OrcDesc), P, P, P, P, P, P, ctypes.c_int32,
                                        P, P, ctypes.c_int32]
        L.orc_sparse_decode.restype = ctypes.c_int64
        L.orc_sparse_decode_dual.argtypes = [ctypes.POINTER(OrcDesc), ctypes.POINTER(OrcDesc),
                                             P, P, P, P, P, P, P, P, ctypes.c_int32, P, P,
                                             ctypes.c_int32]
        L.orc_sparse_decode_dual.restype = ctypes.c_int64
        L.orc_convert_req_index_to_global.argtypes = [
            P, ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P]
        L.orc_convert_req_index_to_global.restype = None
        L.orc_quantize_row.argtypes = [P, ctypes.c_int32, P, P]
        L.orc_quantize_row.restype = None
        L.orc_store_rows.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64, P, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        L.orc_store_rows.restype = None
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def e4m3fn(code: int) -> float:
    return lib().orc_e4m3fn(code)


def ue8m0(code: int) -> float:
    return lib().orc_ue8m0(code)


def bf16(bits: int) -> float:
    return lib().orc_bf16(bits)


def make_desc(*, B, H, topk, swa, block_size, num_blocks, page_stride, sm_scale,
              block_table=None, max_blocks_per_seq=None, scrub=False, s_q=1) -> OrcDesc:
    if block_table is not None:
        bt_stride = block_table.shape[1]
        mb = bt_stride if max_blocks_per_seq is None else max_blocks_per_seq
    else:
        bt_stride, mb = 0, 0
    return OrcDesc(B, H, topk, swa, block_size, mb, num_blocks, bt_stride, page_stride,
                   float(sm_scale), 1 if scrub else 0, int(s_q))


def resolve(desc: OrcDesc, block_table, b: int, idx: int):
    bt = _c(block_table, np.int32)
    page = ctypes.c_int64(0)
    off = ctypes.c_int32(0)
    ok = lib().orc_resolve(ctypes.byref(desc), _ptr(bt), b, idx, ctypes.byref(page),
                           ctypes.byref(off))
    return (page.value, off.value) if ok else None


def dequant_row(desc: OrcDesc, kv: np.ndarray, page: int, off: int) -> np.ndarray:
    kv = _c(kv, np.uint8)
    out = np.zeros(512, dtype=np.float64)
    lib().orc_dequant_row(ctypes.byref(desc), _ptr(kv), page, off, _ptr(out))
    return out


def sparse_decode(*, q, kv, topk_idx, topk, swa, block_size, num_blocks, page_stride,
                  sm_scale, block_table=None, max_blocks_per_seq=None, valid_len=None,
                  sink=None, num_splits=0, nthreads=None, scrub=False, s_q=1, swa_pool=None):
    """Returns (out [B,H,512] f64, lse [B,H] f64, number of valid entries).
    scrub: read every non-finite dequantised cache element as 0.  s_q: query
    tokens per sequence (block_table and valid_len have B / s_q rows).
    swa_pool: dict(kv, block_table, block_size, num_blocks, page_stride,
    max_blocks_per_seq) of a second pool the SWA entries resolve in."""
    q = _c(q, np.uint16)
    B, H, D = q.shape
    assert D == 512
    kv = _c(kv, np.uint8)
    ti = _c(topk_idx, np.int32)
    assert ti.shape == (B, topk + swa)
    bt = _c(block_table, np.int32)
    vl = _c(valid_len, np.int32)
    sk = _c(sink, np.float32)
    desc = make_desc(B=B, H=H, topk=topk, swa=swa, block_size=block_size,
                     num_blocks=num_blocks, page_stride=page_stride, sm_scale=sm_scale,
                     block_table=bt, max_blocks_per_seq=max_blocks_per_seq, scrub=scrub,
                     s_q=s_q)
    out = np.zeros((B, H, 512), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    if swa_pool is None:
        n = lib().orc_sparse_decode(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(bt), _ptr(ti),
                                    _ptr(vl), _ptr(sk), int(num_splits), _ptr(out), _ptr(lse),
                                    int(nthreads or default_threads()))
    else:
        kv2 = _c(swa_pool["kv"], np.uint8)
        bt2 = _c(swa_pool["block_table"], np.int32)
        d2 = make_desc(B=B, H=H, topk=topk, swa=swa, block_size=swa_pool["block_size"],
                       num_blocks=swa_pool["num_blocks"], page_stride=swa_pool["page_stride"],
                       sm_scale=sm_scale, block_table=bt2,
                       max_blocks_per_seq=swa_pool.get("max_blocks_per_seq"), scrub=scrub,
                       s_q=s_q)
        n = lib().orc_sparse_decode_dual(ctypes.byref(desc), ctypes.byref(d2), _ptr(q), _ptr(kv),
                                         _ptr(bt), _ptr(kv2), _ptr(bt2), _ptr(ti), _ptr(vl),
                                         _ptr(sk), int(num_splits), _ptr(out), _ptr(lse),
                                         int(nthreads or default_threads()))
    return out, lse, int(n)


def decode_workload(w, *, topk_idx=None, use_block_table=True, num_splits=0, nthreads=None,
                    **overrides):
    """Oracle decode of a ``synth.Workload`` (fields may be overridden)."""
    kw = dict(q=w.q, kv=w.kv, topk_idx=w.topk_idx if topk_idx is None else topk_idx,
              topk=w.topk, swa=w.swa, block_size=w.block_size, num_blocks=w.num_blocks,
              page_stride=w.page_stride, sm_scale=w.sm_scale,
              block_table=w.block_table if use_block_table else None,
              max_blocks_per_seq=w.max_blocks_per_seq if use_block_table else None,
              valid_len=w.valid_len, sink=w.sink, s_q=getattr(w, "s_q", 1),
              swa_pool=getattr(w, "swa_pool", None))
    kw.update(overrides)
    return sparse_decode(num_splits=num_splits, nthreads=nthreads, **kw)


def convert_req_index_to_global(*, token_indices, block_table, max_blocks_per_req, block_size,
                                width=None, req_id=None, num_reqs=None, cu_seqlens=None,
                                invalid_fill=0):
    ti = _c(token_indices, np.int32)
    bt = _c(block_table, np.int32)
    T = ti.shape[0]
    width = ti.shape[1] if width is None else width
    rq = _c(req_id, np.int32)
    nreq = bt.shape[0] if num_reqs is None else num_reqs
    cu = _c(cu_seqlens, np.int32)
    n_out = int(cu[-1]) if cu is not None else T * width
    out = np.full(max(n_out, 1), np.iinfo(np.int32).min, dtype=np.int32)
    lib().orc_convert_req_index_to_global(_ptr(rq), nreq, _ptr(bt), bt.shape[1],
                                          max_blocks_per_req, _ptr(ti), ti.shape[1], T, width,
                                          block_size, _ptr(cu), invalid_fill, _ptr(out))
    return out[:n_out] if cu is not None else out[:n_out].reshape(T, width)


def quantize_row(x_bits: np.ndarray, *, sanitize: bool):
    """One bf16 row (uint16 bits [512]) -> (576 data bytes, 8 scale bytes)."""
    x = _c(x_bits, np.uint16)
    assert x.shape == (512,)
    data = np.zeros(576, dtype=np.uint8)
    scales = np.zeros(8, dtype=np.uint8)
    lib().orc_quantize_row(_ptr(x), 1 if sanitize else 0, _ptr(data), _ptr(scales))
    return data, scales


def store_rows(kv: np.ndarray, rows_bits: np.ndarray, slots: np.ndarray, *, block_size: int,
               sanitize: bool) -> np.ndarray:
    """Returns a copy of the pool kv [num_blocks, page_stride] with the bf16
    rows (uint16 bits [n, 512]) quantised and stored at the global slots."""
    out = np.array(kv, dtype=np.uint8, copy=True, order="C")
    rows = _c(rows_bits, np.uint16)
    sl = _c(slots, np.int64)
    n = sl.shape[0]
    assert rows.shape == (n, 512)
    lib().orc_store_rows(_ptr(rows), 512, _ptr(sl), n, _ptr(out), block_size, out.shape[0],
                         out.shape[1], 1 if sanitize else 0)
    return out
