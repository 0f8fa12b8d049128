"""CPU oracle for MoE dispatch / combine -- TEST INFRASTRUCTURE ONLY.

A ctypes front end over ``oracle/oracle.c`` (plain C, built with
``gcc -O2 -ffp-contract=off -fopenmp``; one thread unless ``set_threads``
asks for more).  Only the test suite, the smoke entry point
and the benchmark's CPU-baseline leg may import this package; the HIP
library never does, and this package never imports the HIP library.

Functions take and return numpy arrays on the host.  The definitions, and the
passages of the pages each one follows, are documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CONTIGUOUS = 0
MASKED = 1
QUANT_NONE = 0
QUANT_FP8_F32 = 1
QUANT_FP8_UE8M0 = 2
QUANT_MXFP8 = 3

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fopenmp",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_dispatch_layout.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64,
                                           P, P, P, P, P, P, P, P]
    lib.oracle_dispatch_layout.restype = ctypes.c_int
    lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_dispatch.restype = None
    lib.oracle_combine.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_get_threads.argtypes = []
    lib.oracle_get_threads.restype = i32
    lib.oracle_set_threads(1)  # one thread unless a caller asks for more
    lib.oracle_rank_layout.argtypes = [i32, i32, i32, i32, i64, P, P, P, P, P]
    lib.oracle_rank_layout.restype = ctypes.c_int
    lib.oracle_dispatch_dedup.argtypes = [i32, i32, i32, i32, P, P, P, P]
    lib.oracle_dispatch_dedup.restype = None
    lib.oracle_expand.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_expand.restype = None
    lib.oracle_combine_partial.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_combine_partial.restype = None
    lib.oracle_combine_reduce.argtypes = [i32, i32, i32, P, P, P]
    lib.oracle_combine_reduce.restype = None
    lib.oracle_row_expert.argtypes = [i32, P, P, i64, P]
    lib.oracle_row_expert.restype = None
    lib.oracle_repack_masked_to_contiguous.argtypes = [i32, i32, i32, i32, i32, P, P, P, i64, P, P, P, P]
    lib.oracle_repack_masked_to_contiguous.restype = ctypes.c_int
    lib.oracle_repack_contiguous_to_masked.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_repack_contiguous_to_masked.restype = None
    lib.oracle_scales_mn_major.argtypes = [i64, i32, P, P]
    lib.oracle_scales_mn_major.restype = None
    for name in ("oracle_bf16_rne_array", "oracle_e4m3_encode_array",
                 "oracle_ue8m0_exponent_array", "oracle_mx_exponent_array"):
        getattr(lib, name).argtypes = [P, P, i64]
        getattr(lib, name).restype = None
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def rows_capacity(T: int, K: int, E: int, layout: int, align: int = 1,
                  capacity: int = 1) -> int:
    """Rows a dispatched buffer needs: T*K + E*(align-1) contiguous, E*C masked."""
    return T * K + E * (align - 1) if layout == CONTIGUOUS else E * capacity


def dispatch_layout(topk_idx: np.ndarray, E: int, R: int, layout: int,
                    align: int = 1, capacity: int = 1,
                    rows_cap: Optional[int] = None) -> dict:
    """Counts, offsets, stable slots and both maps for int32 ids [T, K]."""
    lib = _load()
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    if rows_cap is None:
        rows_cap = rows_capacity(T, K, E, layout, align, capacity)
    h = dict(expert_count=np.zeros(E, np.int32), recv_count=np.zeros(E, np.int32),
             expert_offset=np.zeros(E + 1, np.int32), rank_offset=np.zeros(R + 1, np.int32),
             pair_to_row=np.zeros(T * K, np.int32), row_to_pair=np.zeros(rows_cap, np.int32),
             status=np.zeros(2, np.int32))
    rc = lib.oracle_dispatch_layout(T, K, E, R, layout, align, capacity, rows_cap, _ptr(idx),
                                    _ptr(h["expert_count"]), _ptr(h["recv_count"]),
                                    _ptr(h["expert_offset"]), _ptr(h["rank_offset"]),
                                    _ptr(h["pair_to_row"]), _ptr(h["row_to_pair"]),
                                    _ptr(h["status"]))
    if rc != 0:
        raise ValueError("rows needed exceed rows_capacity")
    return h


def set_threads(n: int) -> int:
    """Threads for the token loops of dispatch and combine (the layout is
    serial); returns the count now in effect.  Results do not depend on it."""
    lib = _load()
    lib.oracle_set_threads(int(n))
    return int(lib.oracle_get_threads())


def dispatch(x: np.ndarray, pair_to_row: np.ndarray, K: int, quant: int, rows: int,
             topk_w: Optional[np.ndarray] = None, out_x: Optional[np.ndarray] = None,
             out_scale: Optional[np.ndarray] = None,
             out_row_weight: Optional[np.ndarray] = None):
    """Permute (and optionally quantize) bf16 rows x [T, H] into `rows` rows.

    Output buffers may be passed pre-filled (e.g. with a sentinel) to check
    that unwritten rows stay untouched; otherwise they are zero-filled.
    Returns (out_x, out_scale, out_row_weight).
    """
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    NB = H // 128
    if out_x is None:
        out_x = np.zeros((rows, H), np.uint16 if quant == QUANT_NONE else np.uint8)
    if out_scale is None and quant == QUANT_FP8_F32:
        out_scale = np.zeros((rows, NB), np.float32)
    if out_scale is None and quant == QUANT_FP8_UE8M0:
        out_scale = np.zeros((rows, (NB + 3) // 4), np.uint32)
    if out_scale is None and quant == QUANT_MXFP8:
        out_scale = np.zeros((rows, H // 32), np.uint8)
    w = None if topk_w is None else _c(topk_w, np.float32)
    for a in (out_x, out_scale, out_row_weight):
        assert a is None or a.flags["C_CONTIGUOUS"]
    lib.oracle_dispatch(T, K, H, quant, _ptr(x), _ptr(w), _ptr(_c(pair_to_row, np.int32)),
                        _ptr(out_x), _ptr(out_scale), _ptr(out_row_weight))
    return out_x, out_scale, out_row_weight


def combine(y: np.ndarray, topk_w: np.ndarray, pair_to_row: np.ndarray) -> np.ndarray:
    """Weighted top-k reduction: bf16 y [rows, H] -> bf16 out [T, H] (uint16 bits)."""
    lib = _load()
    y = _c(y, np.uint16)
    w = _c(topk_w, np.float32)
    T, K = w.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.uint16)
    lib.oracle_combine(T, K, H, _ptr(y), _ptr(w), _ptr(_c(pair_to_row, np.int32)), _ptr(out))
    return out


def _dispatched_buffers(rows, H, quant, out_x, out_scale):
    NB = H // 128
    if out_x is None:
        out_x = np.zeros((rows, H), np.uint16 if quant == QUANT_NONE else np.uint8)
    if out_scale is None and quant == QUANT_FP8_F32:
        out_scale = np.zeros((rows, NB), np.float32)
    if out_scale is None and quant == QUANT_FP8_UE8M0:
        out_scale = np.zeros((rows, (NB + 3) // 4), np.uint32)
    if out_scale is None and quant == QUANT_MXFP8:
        out_scale = np.zeros((rows, H // 32), np.uint8)
    for a in (out_x, out_scale):
        assert a is None or a.flags["C_CONTIGUOUS"]
    return out_x, out_scale


def rank_rows_capacity(T: int, K: int, R: int) -> int:
    """Rows a per-rank (deduplicated) buffer needs: T * min(K, R)."""
    return T * min(K, R)


def rank_layout(topk_idx: np.ndarray, E: int, R: int, rows_cap: Optional[int] = None) -> dict:
    """Per-rank token counts, offsets and the (token, rank) <-> row maps."""
    lib = _load()
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    if rows_cap is None:
        rows_cap = rank_rows_capacity(T, K, R)
    h = dict(rank_token_count=np.zeros(R, np.int32), rank_token_offset=np.zeros(R + 1, np.int32),
             token_rank_row=np.zeros(T * R, np.int32), rank_row_to_token=np.zeros(rows_cap, np.int32))
    rc = lib.oracle_rank_layout(T, K, E, R, rows_cap, _ptr(idx), _ptr(h["rank_token_count"]),
                                _ptr(h["rank_token_offset"]), _ptr(h["token_rank_row"]),
                                _ptr(h["rank_row_to_token"]))
    if rc != 0:
        raise ValueError("per-rank rows exceed rows_cap")
    return h


def dispatch_dedup(x: np.ndarray, token_rank_row: np.ndarray, R: int, quant: int, rows: int,
                   out_x: Optional[np.ndarray] = None, out_scale: Optional[np.ndarray] = None):
    """Each token row (quantized as in dispatch) once per rank it is in.
    Returns (send_x, send_scale)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    out_x, out_scale = _dispatched_buffers(rows, H, quant, out_x, out_scale)
    lib.oracle_dispatch_dedup(T, R, H, quant, _ptr(x), _ptr(_c(token_rank_row, np.int32)),
                              _ptr(out_x), _ptr(out_scale))
    return out_x, out_scale


def expand(topk_idx: np.ndarray, E: int, R: int, quant: int, send_x: np.ndarray,
           send_scale: Optional[np.ndarray], token_rank_row: np.ndarray,
           pair_to_row: np.ndarray, rows: int, out_x: Optional[np.ndarray] = None,
           out_scale: Optional[np.ndarray] = None):
    """Receive-side expansion of per-rank rows into the per-expert layout.
    Returns (out_x, out_scale)."""
    lib = _load()
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    send_x = np.ascontiguousarray(send_x)
    H = send_x.shape[1]
    out_x, out_scale = _dispatched_buffers(rows, H, quant, out_x, out_scale)
    ss = None if send_scale is None else np.ascontiguousarray(send_scale)
    lib.oracle_expand(T, K, E, R, H, quant, _ptr(idx), _ptr(send_x), _ptr(ss),
                      _ptr(_c(token_rank_row, np.int32)), _ptr(_c(pair_to_row, np.int32)),
                      _ptr(out_x), _ptr(out_scale))
    return out_x, out_scale


def combine_partial(topk_idx: np.ndarray, E: int, R: int, y: np.ndarray, topk_w: np.ndarray,
                    pair_to_row: np.ndarray, token_rank_row: np.ndarray, rank_rows: int,
                    out: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-(token, rank) bf16 partial sums [rank_rows, H] (uint16 bits)."""
    lib = _load()
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    y = _c(y, np.uint16)
    H = y.shape[1]
    if out is None:
        out = np.zeros((rank_rows, H), np.uint16)
    assert out.flags["C_CONTIGUOUS"]
    lib.oracle_combine_partial(T, K, E, R, H, _ptr(idx), _ptr(y), _ptr(_c(topk_w, np.float32)),
                               _ptr(_c(pair_to_row, np.int32)), _ptr(_c(token_rank_row, np.int32)),
                               _ptr(out))
    return out


def combine_reduce(partial: np.ndarray, token_rank_row: np.ndarray, R: int) -> np.ndarray:
    """Sum of a token's per-rank partials in ascending rank: bf16 out [T, H]."""
    lib = _load()
    partial = _c(partial, np.uint16)
    H = partial.shape[1]
    trr = _c(token_rank_row, np.int32).reshape(-1)
    T = trr.size // R
    out = np.zeros((T, H), np.uint16)
    lib.oracle_combine_reduce(T, R, H, _ptr(partial), _ptr(trr), _ptr(out))
    return out


def bf16_rne(a: np.ndarray) -> np.ndarray:
    lib = _load()
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_bf16_rne_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_encode(a: np.ndarray) -> np.ndarray:
    lib = _load()
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib.oracle_e4m3_encode_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def ue8m0_exponent(a: np.ndarray) -> np.ndarray:
    lib = _load()
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.int32)
    lib.oracle_ue8m0_exponent_array(_ptr(a), _ptr(out), a.size)
    return out


def mx_exponent(a: np.ndarray) -> np.ndarray:
    """OCP MX shared exponent for E4M3 elements: largest s with 2^(s+8) <= a."""
    lib = _load()
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.int32)
    lib.oracle_mx_exponent_array(_ptr(a), _ptr(out), a.size)
    return out


# ---- adapters for grouped-GEMM consumers --------------------------------------

def row_expert(expert_offset: np.ndarray, recv_count: np.ndarray, rows: int) -> np.ndarray:
    """Expert of each row that holds a received pair, -1 elsewhere: int32 [rows]."""
    lib = _load()
    off, rc = _c(expert_offset, np.int32), _c(recv_count, np.int32)
    out = np.zeros(rows, np.int32)
    lib.oracle_row_expert(rc.size, _ptr(off), _ptr(rc), rows, _ptr(out))
    return out


def repack_masked_to_contiguous(x: np.ndarray, scale: Optional[np.ndarray], recv_count: np.ndarray,
                                C: int, align: int, quant: int, out_rows: int,
                                out_x: Optional[np.ndarray] = None, out_scale: Optional[np.ndarray] = None):
    """Masked slab rows (+ scales) -> contiguous segments padded to `align`.
    Returns (out_x, out_scale, out_offset [E+1], out_row_expert [out_rows])."""
    lib = _load()
    x = np.ascontiguousarray(x)
    H = x.shape[1]
    rc = _c(recv_count, np.int32)
    E = rc.size
    out_x, out_scale = _dispatched_buffers(out_rows, H, quant, out_x, out_scale)
    off = np.zeros(E + 1, np.int32)
    rex = np.zeros(out_rows, np.int32)
    sc = None if scale is None else np.ascontiguousarray(scale)
    rc_ = lib.oracle_repack_masked_to_contiguous(E, C, align, H, quant, _ptr(rc), _ptr(x), _ptr(sc), out_rows,
                                                 _ptr(out_x), _ptr(out_scale), _ptr(off), _ptr(rex))
    if rc_ != 0:
        raise ValueError("contiguous segments exceed out_rows")
    return out_x, out_scale, off, rex


def repack_contiguous_to_masked(y: np.ndarray, recv_count: np.ndarray, offset: np.ndarray, C: int,
                                out: Optional[np.ndarray] = None) -> np.ndarray:
    """Contiguous bf16 expert outputs -> the masked slab [E*C, H]."""
    lib = _load()
    y = _c(y, np.uint16)
    H = y.shape[1]
    rc = _c(recv_count, np.int32)
    E = rc.size
    if out is None:
        out = np.zeros((E * C, H), np.uint16)
    assert out.flags["C_CONTIGUOUS"]
    lib.oracle_repack_contiguous_to_masked(E, C, H, _ptr(rc), _ptr(_c(offset, np.int32)), _ptr(y), _ptr(out))
    return out


def scales_mn_major(scale_words: np.ndarray) -> np.ndarray:
    """Row-major 32-bit scales [rows, S] -> MN-major [S, ld], ld = rows rounded up to 4."""
    lib = _load()
    a = np.ascontiguousarray(scale_words).view(np.uint32)
    rows, S = a.shape
    ld = (rows + 3) // 4 * 4
    out = np.zeros((S, ld), np.uint32)
    lib.oracle_scales_mn_major(rows, S, _ptr(a), _ptr(out))
    return out
