"""CPU oracle for paged MLA decode -- test infrastructure only.

``mla_oracle.c`` is the plain fp64 reference of the decode path (see its
header for the passages it follows).  This module builds it with gcc and calls
it through ctypes.  Only the tests, the smoke check and the benchmark's CPU
baseline use it; the product library neither links nor calls it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle (gcc, -O2, OpenMP).  No fast-math: summation order
    and IEEE semantics stay as written."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib):
    """Argument and result types of the oracle's C functions on a loaded
    library (the built oracle, or a test's compiled copy of it)."""
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_mla_decode.argtypes = [I, I, I, I, I, I, I, I, I, I, ctypes.c_float,
                                      P, P, P, P, P, I, P, P, P]
    lib.oracle_mla_decode.restype = I
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_decode_row.argtypes = [P, I, P]
    lib.oracle_decode_row.restype = None
    lib.oracle_num_threads.restype = I
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_quantize_row_fp8.argtypes = [P, P]
    lib.oracle_quantize_row_fp8.restype = None
    lib.oracle_kv_append_fp8.argtypes = [I, I, I, I, I, P, P, P, P]
    lib.oracle_kv_append_fp8.restype = None
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(code))


def bf16_round(x: float) -> int:
    return int(_load().oracle_bf16_round(x))


def e4m3_encode(v: float) -> int:
    """Nearest e4m3fn code (ties to even), saturated to +-448."""
    return int(_load().oracle_e4m3_encode(v))


def quantize_row_fp8(row_bf16: np.ndarray) -> np.ndarray:
    """bf16 bit row [576] -> the 656-byte FP8 row."""
    x = np.ascontiguousarray(row_bf16, dtype=np.uint16)
    assert x.shape == (576,)
    out = np.zeros(656, dtype=np.uint8)
    _load().oracle_quantize_row_fp8(_ptr(x), _ptr(out))
    return out


def kv_append_fp8(kv_new: np.ndarray, start_pos: np.ndarray, block_table: np.ndarray,
                  kv_pool: np.ndarray, page_size: int = 64) -> np.ndarray:
    """Quantise kv_new (bf16 bits [B, n_new, 576]) into a copy of kv_pool
    ([num_pages, page_size, 656] bytes) at positions start_pos[b] + j
    through block_table [B, max_pages]; returns the new pool."""
    kv_new = np.ascontiguousarray(kv_new, dtype=np.uint16)
    B, n_new, d = kv_new.shape
    assert d == 576
    sp = np.ascontiguousarray(start_pos, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    pool = np.array(kv_pool, dtype=np.uint8, copy=True, order="C")
    _load().oracle_kv_append_fp8(B, n_new, page_size, pool.shape[0], bt.shape[1], _ptr(kv_new),
                                 _ptr(sp), _ptr(bt), _ptr(pool))
    return pool


def decode_row(row: np.ndarray, kv_format: int) -> np.ndarray:
    """One cached latent row (uint8 bytes) -> float32[576] dequantised values."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    out = np.empty(576, dtype=np.float32)
    _load().oracle_decode_row(_ptr(row), int(kv_format), _ptr(out))
    return out


def mla_decode(w, *, n_splits: int = 1, natural: bool = False,
               unit_mask: Optional[np.ndarray] = None, is_causal: Optional[int] = None,
               softmax_scale: Optional[float] = None, block_table: Optional[np.ndarray] = None,
               kv: Optional[np.ndarray] = None, cache_seqlens: Optional[np.ndarray] = None,
               indices: Optional[np.ndarray] = None, topk: Optional[int] = None,
               q: Optional[np.ndarray] = None):
    """Run the oracle on a :class:`synth.Workload` (fields may be overridden).

    Returns ``(out fp64 [B, s_q, h_q, 512], lse fp64 [B, s_q, h_q])``.  Rows of
    units excluded by ``unit_mask`` are NaN.
    """
    q = np.ascontiguousarray(w.q if q is None else q, dtype=np.uint16)
    kv = np.ascontiguousarray(w.kv if kv is None else kv, dtype=np.uint8)
    bt = np.ascontiguousarray(w.block_table if block_table is None else block_table, dtype=np.int32)
    sl = np.ascontiguousarray(w.cache_seqlens if cache_seqlens is None else cache_seqlens, dtype=np.int32)
    tk = w.topk if topk is None else topk
    idx = w.indices if indices is None else indices
    idx = None if tk == 0 else np.ascontiguousarray(idx, dtype=np.int32)
    B, s_q, h_q = q.shape[0], q.shape[1], q.shape[2]
    out = np.full((B, s_q, h_q, 512), np.nan, dtype=np.float64)
    lse = np.full((B, s_q, h_q), np.nan, dtype=np.float64)
    mask = None if unit_mask is None else np.ascontiguousarray(unit_mask, dtype=np.uint8)
    rc = _load().oracle_mla_decode(
        B, s_q, h_q, w.page_size, kv.shape[0], bt.shape[1], w.kv_format, tk,
        w.is_causal if is_causal is None else is_causal, int(natural),
        float(np.float32(w.softmax_scale if softmax_scale is None else softmax_scale)),
        _ptr(q), _ptr(kv), _ptr(bt), _ptr(sl), _ptr(idx), int(n_splits), _ptr(mask),
        _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle rejected the workload (code {rc})")
    return out, lse


def timed_mla_decode(w, **kw):
    """(out, lse, seconds) with wall time around the oracle call only."""
    t0 = time.perf_counter()
    out, lse = mla_decode(w, **kw)
    return out, lse, time.perf_counter() - t0
