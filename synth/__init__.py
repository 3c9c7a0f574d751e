"""Seeded synthetic inputs (host numpy arrays) and the workload shapes.

Holds no matmul arithmetic: it draws random numbers and stores them in the
input formats (packed nibble bytes, bf16 bit patterns as uint16, int32 ids).
The CPU oracle's tests, the GPU parity tests and the bench all take their
inputs from here, so both sides of every comparison read identical bits.

Shapes are those of a 27B-class dense decoder (hidden size 5,120 and a
248,320-token vocabulary, as on the swift-qwen3.8-rtx3090 project page,
"Body, heads and drafter", and the qwen-warp/llamAmpere article's byte
table), with the projection sizes of the synthetic workloads.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SYNTH_LIB: an instrumented build of the same source (sanitizer runs)
_LIB_PATH = os.environ.get("SYNTH_LIB") or os.path.join(HERE, "libsynth.so")
_lib = None

SEED = 20261202
GROUP = 128

# name -> (N output rows, K reduction length)
PROJECTIONS = {
    "qkv": (7168, 5120),
    "o": (5120, 5120),
    "gate_up": (34816, 5120),
    "down": (5120, 17408),
}
PROJ_ORDER = ("qkv", "o", "gate_up", "down")
SMALL = (1024, 1024)          # single small matmul, the case the oracle runs in full
LM_HEAD = (248320, 5120)      # full-vocabulary output head
DRAFT_IDS = 32768             # draft-vocabulary rows gathered from the head
LAYERS = 64                   # decoder layers in the full weight pass

# tensor ids (each weight tensor and each activation block owns a stream)
TID_SMALL = 5000
TID_LM_HEAD = 1000
RID_DRAFT = 2000


def tid_layer(layer: int, proj: str) -> int:
    return 8 * layer + PROJ_ORDER.index(proj)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # noqa: F401  (same package)
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        lib.synth_codes.argtypes = [u64, u64, vp, u64, i32]
        lib.synth_scales.argtypes = [u64, u64, vp, u64, i32]
        lib.synth_normal_bf16.argtypes = [u64, u64, vp, u64, i32]
        lib.synth_distinct_ids.argtypes = [u64, u64, vp, i64, i64]
        lib.synth_distinct_ids.restype = i32
        lib.synth_codes_range.argtypes = [u64, u64, vp, u64, u64]
        lib.synth_scales_range.argtypes = [u64, u64, vp, u64, u64]
        lib.synth_bf16_from_double.argtypes = [ctypes.c_double]
        lib.synth_bf16_from_double.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_from_double(v: float) -> int:
    return int(_load().synth_bf16_from_double(float(v)))


def codes(tid: int, n_rows: int, k: int, seed: int = SEED, out: np.ndarray | None = None) -> np.ndarray:
    """Packed codes [n_rows][k/2] uint8 of weight tensor `tid`."""
    n = n_rows * (k // 2)
    a = np.empty(n, dtype=np.uint8) if out is None else out.reshape(-1)
    assert a.size == n and a.dtype == np.uint8 and a.flags.c_contiguous
    _load().synth_codes(seed, 4 * tid + 0, a.ctypes.data, n, _threads())
    return a.reshape(n_rows, k // 2)


def scales(tid: int, n_rows: int, k: int, seed: int = SEED, out: np.ndarray | None = None) -> np.ndarray:
    """bf16 scales [n_rows][k/128] (uint16 bit patterns) of weight tensor `tid`."""
    n = n_rows * (k // GROUP)
    a = np.empty(n, dtype=np.uint16) if out is None else out.reshape(-1)
    assert a.size == n and a.dtype == np.uint16 and a.flags.c_contiguous
    _load().synth_scales(seed, 4 * tid + 1, a.ctypes.data, n, _threads())
    return a.reshape(n_rows, k // GROUP)


def activations(xid: int, t: int, k: int, seed: int = SEED) -> np.ndarray:
    """bf16 activations [t][k] (uint16 bit patterns), rows independent N(0,1)."""
    a = np.empty(t * k, dtype=np.uint16)
    _load().synth_normal_bf16(seed, 4 * xid + 2, a.ctypes.data, a.size, _threads())
    return a.reshape(t, k)


def distinct_ids(rid: int, n_ids: int, n_rows: int, seed: int = SEED) -> np.ndarray:
    """n_ids distinct row ids from [0, n_rows), int32, in draw order."""
    a = np.empty(n_ids, dtype=np.int32)
    rc = _load().synth_distinct_ids(seed, 4 * rid + 3, a.ctypes.data, n_ids, n_rows)
    if rc != 0:
        raise ValueError("bad arguments for distinct_ids")
    return a


def weight(tid: int, n_rows: int, k: int, seed: int = SEED):
    return codes(tid, n_rows, k, seed), scales(tid, n_rows, k, seed)


def weight_rows(tid: int, rows, k: int, seed: int = SEED):
    """Rows `rows` of weight tensor `tid` (row-major [n_rows][k/2] codes and
    [n_rows][k/128] scales), the same bits as weight(...)[0][rows] and
    [1][rows], generated without the other rows."""
    rows = np.asarray(rows, dtype=np.int64)
    kb, g = k // 2, k // GROUP
    p = np.empty((rows.size, kb), dtype=np.uint8)
    s = np.empty((rows.size, g), dtype=np.uint16)
    lib = _load()
    for i, r in enumerate(rows):
        lib.synth_codes_range(seed, 4 * tid + 0, p[i].ctypes.data, int(r) * kb, kb)
        lib.synth_scales_range(seed, 4 * tid + 1, s[i].ctypes.data, int(r) * g, g)
    return p, s


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)

