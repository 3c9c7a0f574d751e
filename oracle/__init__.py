"""CPU oracle for the W4A16 skinny matmul -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrappers over oracle/oracle.c (plain C, double precision).  Only
tests/, the smoke check and the bench's CPU baseline leg may import this
package; the GPU library never does, and the oracle never imports it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB: an instrumented build of the same source (sanitizer runs)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16.restype = ctypes.c_double
        lib.oracle_code.argtypes = [vp, i64]
        lib.oracle_code.restype = i32
        lib.oracle_matmul.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, i32]
        lib.oracle_gather.argtypes = [vp, i64, vp, vp, i64, vp, i64, i32, vp, vp, i32]
        lib.oracle_matmul_dequant_first.argtypes = [vp, vp, vp, i64, i64, i32, vp]
        lib.oracle_argmax.argtypes = [vp, vp, i64, i32, vp, vp, vp]
        lib.oracle_topk.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        lib.oracle_greedy_accept.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.oracle_draft_union.argtypes = [vp, i64, vp, i64, i64, vp]
        lib.oracle_draft_union.restype = i64
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


def matmul(packed, scales, x, nthreads: int | None = None, want_abs: bool = True):
    """y[T][N] (float64) and A[T][N] = sum_k |w*x| for the whole matrix."""
    packed, pp = _c(packed, np.uint8)
    scales, sp = _c(scales, np.uint16)
    x, xp = _c(x, np.uint16)
    N = packed.shape[0]
    K = packed.shape[1] * 2
    T = x.shape[0]
    assert x.shape[1] == K and scales.shape == (N, K // 128)
    y = np.empty((T, N), np.float64)
    a = np.empty((T, N), np.float64) if want_abs else None
    _load().oracle_matmul(pp, sp, xp, N, K, T, y.ctypes.data, a.ctypes.data if a is not None else None,
                          nthreads or default_threads())
    return y, a


def gather(row_ids, packed, scales, x, nthreads: int | None = None):
    """y[T][n_ids] and A[T][n_ids] for weight rows row_ids[i] (NaN if out of range)."""
    row_ids, rp = _c(row_ids, np.int32)
    packed, pp = _c(packed, np.uint8)
    scales, sp = _c(scales, np.uint16)
    x, xp = _c(x, np.uint16)
    n_rows = packed.shape[0]
    K = packed.shape[1] * 2
    T = x.shape[0]
    n = row_ids.shape[0]
    y = np.empty((T, n), np.float64)
    a = np.empty((T, n), np.float64)
    _load().oracle_gather(rp, n, pp, sp, n_rows, xp, K, T, y.ctypes.data, a.ctypes.data,
                          nthreads or default_threads())
    return y, a


def matmul_dequant_first(packed, scales, x):
    packed, pp = _c(packed, np.uint8)
    scales, sp = _c(scales, np.uint16)
    x, xp = _c(x, np.uint16)
    N = packed.shape[0]
    K = packed.shape[1] * 2
    T = x.shape[0]
    y = np.empty((T, N), np.float64)
    _load().oracle_matmul_dequant_first(pp, sp, xp, N, K, T, y.ctypes.data)
    return y


def argmax(y, ids=None, lib=None):
    """Per row t of y[T][n]: (id, value, gap to the best other id).

    lib: a ctypes handle of another build of oracle.c exporting the same
    oracle_argmax (the mutation pins load deliberately broken copies)."""
    y, yp = _c(y, np.float64)
    T, n = y.shape
    if ids is not None:
        ids, ip = _c(ids, np.int32)
        assert ids.shape == (n,)
    else:
        ip = None
    out_id = np.empty(T, np.int32)
    out_val = np.empty(T, np.float64)
    gap = np.empty(T, np.float64)
    if lib is None:
        lib = _load()
    else:
        lib.oracle_argmax.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_argmax(yp, ip, n, T, out_id.ctypes.data, out_val.ctypes.data, gap.ctypes.data)
    return out_id, out_val, gap


def bf16(bits: int) -> float:
    return float(_load().oracle_bf16(bits))


def code(packed_row, k: int) -> int:
    packed_row, p = _c(packed_row, np.uint8)
    return int(_load().oracle_code(p, k))


def topk(y, k: int, ids=None):
    """Per row t of y[T][n]: the k best (id, value) pairs, score descending,
    equal scores by ascending id; NaN scores never count; (-1, NaN) padding."""
    y, yp = _c(y, np.float64)
    T, n = y.shape
    if ids is not None:
        ids, ip = _c(ids, np.int32)
        assert ids.shape == (n,)
    else:
        ip = None
    out_id = np.empty((T, k), np.int32)
    out_val = np.empty((T, k), np.float64)
    _load().oracle_topk(yp, ip, n, T, k, out_id.ctypes.data, out_val.ctypes.data)
    return out_id, out_val


def greedy_accept(target, draft, n_seq: int, rows: int):
    """Accepted drafts per sequence and the emitted tokens (target choices of
    rows 0..a, then -1)."""
    target, tp = _c(target, np.int32)
    draft, dp = _c(draft, np.int32)
    assert target.size == n_seq * rows and draft.size == n_seq * (rows - 1)
    acc = np.empty(n_seq, np.int32)
    tok = np.empty((n_seq, rows), np.int32)
    _load().oracle_greedy_accept(tp, dp if draft.size else None, n_seq, rows, acc.ctypes.data, tok.ctypes.data)
    return acc, tok


def draft_union(base, seq, n_rows: int):
    """(ids of n_base + n_seq slots, union length): the base list, then the
    in-range sequence ids not seen before in order of first appearance; -1 after."""
    base, bp = _c(base, np.int32)
    seq, sp = _c(seq, np.int32)
    out = np.empty(base.size + seq.size, np.int32)
    m = _load().oracle_draft_union(bp if base.size else None, base.size, sp if seq.size else None, seq.size, n_rows,
                                   out.ctypes.data)
    return out, int(m)
