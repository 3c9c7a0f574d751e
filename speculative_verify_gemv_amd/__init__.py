"""Python binding of libw4a16 (the W4A16 skinny matmul for MI355X).

Argument marshalling only: every step of the computation runs in the gfx950
kernels behind the C ABI declared in include/w4a16.h.  PyTorch provides device
memory and the current stream.  There is no fallback: if the library is not
built, or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB: an instrumented build of the same sources (host sanitizer runs)
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(HERE, "libw4a16.so")

GROUP = 128
MAX_T = 16
MAX_TOPK = 32
VARIANTS = {"auto": 0, "dot": 1, "mfma": 2}

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load_library():
    """Loads libw4a16.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(speculative_verify_gemv_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        lib.w4a16_matmul.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
        lib.w4a16_matmul.restype = i32
        lib.w4a16_head_gather.argtypes = [vp, i64, vp, vp, i64, vp, i64, i32, vp, vp, vp, vp, sz, vp]
        lib.w4a16_head_gather.restype = i32
        lib.w4a16_head_gather_noalloc.argtypes = [vp, i64, vp, vp, i64, vp, i64, i32, vp, vp, vp, vp]
        lib.w4a16_head_gather_noalloc.restype = i32
        lib.w4a16_workspace_bytes.argtypes = [i64, i32]
        lib.w4a16_workspace_bytes.restype = sz
        lib.w4a16_set_tile.argtypes = [i32, ctypes.c_char_p]
        lib.w4a16_set_tile.restype = i32
        lib.w4a16_set_variant.argtypes = [i32]
        lib.w4a16_set_variant.restype = i32
        lib.w4a16_get_variant.argtypes = []
        lib.w4a16_get_variant.restype = i32
        lib.w4a16_status_string.argtypes = [i32]
        lib.w4a16_status_string.restype = ctypes.c_char_p
        lib.w4a16_abi_version.argtypes = []
        lib.w4a16_abi_version.restype = i32
        lib.w4a16_batch_table_bytes.argtypes = [i32]
        lib.w4a16_batch_table_bytes.restype = sz
        lib.w4a16_batch_plan.argtypes = [vp, i32, i32, vp, sz]
        lib.w4a16_batch_plan.restype = i32
        lib.w4a16_matmul_batch.argtypes = [vp, vp, vp]
        lib.w4a16_matmul_batch.restype = i32
        lib.w4a16_tiled_tile_bytes.argtypes = [i64]
        lib.w4a16_tiled_tile_bytes.restype = sz
        lib.w4a16_tiled_bytes.argtypes = [i64, i64]
        lib.w4a16_tiled_bytes.restype = sz
        lib.w4a16_repack_tiled.argtypes = [vp, vp, i64, i64, vp, sz, vp]
        lib.w4a16_repack_tiled.restype = i32
        lib.w4a16_repack_tiled_rows.argtypes = [vp, vp, i64, i64, vp, i64, vp, sz, vp]
        lib.w4a16_repack_tiled_rows.restype = i32
        lib.w4a16_matmul_tiled.argtypes = [vp, vp, vp, i64, i64, i32, vp]
        lib.w4a16_matmul_tiled.restype = i32
        lib.w4a16_head_gather_tiled.argtypes = [vp, i64, vp, i64, vp, i64, i32, vp, vp, vp, vp, sz, vp]
        lib.w4a16_head_gather_tiled.restype = i32
        lib.w4a16_topk_workspace_bytes.argtypes = [i64, i32, i32]
        lib.w4a16_topk_workspace_bytes.restype = sz
        lib.w4a16_topk.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
        lib.w4a16_topk.restype = i32
        lib.w4a16_greedy_accept.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        lib.w4a16_greedy_accept.restype = i32
        lib.w4a16_draft_union.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp]
        lib.w4a16_draft_union.restype = i32
        lib.w4a16_batch_workspace_bytes.argtypes = [vp]
        lib.w4a16_batch_workspace_bytes.restype = sz
        lib.w4a16_matmul_batch_ws.argtypes = [vp, vp, vp, sz, vp]
        lib.w4a16_matmul_batch_ws.restype = i32
        lib.w4a16_stream_read.argtypes = [vp, sz, vp, i32, vp]
        lib.w4a16_stream_read.restype = i32
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().w4a16_status_string(status).decode()


def abi_version() -> int:
    return load_library().w4a16_abi_version()


def set_variant(name: str) -> None:
    s = load_library().w4a16_set_variant(VARIANTS[name])
    if s:
        raise W4A16Error(s, "set_variant")


def set_tile(spec: str | None, batch: bool = False) -> None:
    """Measurement helper: force the tiling of later single (or grouped)
    launches, e.g. "split,1,8"; None restores the planner's choice."""
    s = load_library().w4a16_set_tile(1 if batch else 0, None if spec is None else spec.encode())
    if s:
        raise W4A16Error(s, "set_tile")


def get_variant() -> str:
    v = load_library().w4a16_get_variant()
    return {i: n for n, i in VARIANTS.items()}[v]


def workspace_bytes(n_out: int, T: int) -> int:
    return int(load_library().w4a16_workspace_bytes(n_out, T))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Context in which the tensors a call allocates (outputs, scratch) belong
    to the stream its kernels run on, so that the caching allocator orders
    their reuse after that work."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check_bits(t: torch.Tensor, what: str) -> None:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what} must hold bf16 bit patterns (bfloat16/int16/uint16), got {t.dtype}")
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous CUDA tensor")


def _check_weight(packed: torch.Tensor, scales: torch.Tensor):
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not (packed.is_cuda and packed.is_contiguous()):
        raise ValueError("packed must be a contiguous CUDA uint8 tensor [rows][K/2]")
    _check_bits(scales, "scales")
    rows, kh = packed.shape
    K = 2 * kh
    if scales.shape != (rows, K // GROUP):
        raise ValueError(f"scales must be [rows][K/128] = {(rows, K // GROUP)}, got {tuple(scales.shape)}")
    return rows, K


def matmul(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """y[T][N] (float32) = x * W^T with W given by packed int4 codes and bf16 group scales."""
    N, K = _check_weight(packed, scales)
    _check_bits(x, "x")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T][{K}]")
    T = x.shape[0]
    if out is None:
        with _on(stream):
            out = torch.empty((T, N), dtype=torch.float32, device=packed.device)
    elif out.dtype != torch.float32 or out.shape != (T, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor [T][N]")
    s = load_library().w4a16_matmul(_ptr(packed), _ptr(scales), _ptr(x), _ptr(out), N, K, T, _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_matmul")
    return out


def _gather_outputs(n: int, T: int, device, scores: bool, argmax: bool, out, workspace):
    y = None
    if scores:
        y = out if out is not None else torch.empty((T, n), dtype=torch.float32, device=device)
    ids = vals = None
    ws_bytes = 0
    if argmax:
        ids = torch.empty(T, dtype=torch.int32, device=device)
        vals = torch.empty(T, dtype=torch.float32, device=device)
        ws_bytes = workspace_bytes(n, T)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device)
        ws_bytes = workspace.numel() * workspace.element_size()
    return y, ids, vals, workspace, ws_bytes


def _row_ids(row_ids, n_rows: int) -> int:
    if row_ids is None:
        return n_rows
    if row_ids.dtype != torch.int32 or row_ids.dim() != 1 or not (row_ids.is_cuda and row_ids.is_contiguous()):
        raise ValueError("row_ids must be a contiguous CUDA int32 vector")
    return row_ids.shape[0]


def head_gather(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, row_ids: torch.Tensor | None = None,
                scores: bool = True, argmax: bool = False, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None):
    """Scores rows row_ids (all rows if None) of an output head; optional per-row argmax.

    Returns (y [T][n] float32 or None, argmax_id [T] int32 or None, argmax_val [T] float32 or None).
    """
    n_rows, K = _check_weight(packed, scales)
    _check_bits(x, "x")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T][{K}]")
    T = x.shape[0]
    n = _row_ids(row_ids, n_rows)
    with _on(stream):
        y, ids, vals, workspace, ws_bytes = _gather_outputs(n, T, packed.device, scores, argmax, out, workspace)
    s = load_library().w4a16_head_gather(_ptr(row_ids), n, _ptr(packed), _ptr(scales), n_rows, _ptr(x), K, T,
                                         _ptr(y), _ptr(ids), _ptr(vals), _ptr(workspace), ws_bytes,
                                         _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_head_gather")
    return y, ids, vals


NOALLOC_SCRATCH_BYTES = 2 << 20


def head_gather_noalloc(packed: torch.Tensor, scales: torch.Tensor, x: torch.Tensor,
                        row_ids: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        argmax_id: torch.Tensor | None = None, argmax_val: torch.Tensor | None = None, stream=None):
    """head_gather() through w4a16_head_gather_noalloc: the library allocates
    nothing (the argmax partials live in its static device scratch); the
    caller passes every output it wants (out [T][n] float32, argmax_id [T]
    int32, argmax_val [T] float32), so the call itself allocates nothing
    either.  Calls that may overlap on one GPU race on the scratch."""
    n_rows, K = _check_weight(packed, scales)
    _check_bits(x, "x")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T][{K}]")
    T = x.shape[0]
    n = _row_ids(row_ids, n_rows)
    for t, shape, dt, what in ((out, (T, n), torch.float32, "out"), (argmax_id, (T,), torch.int32, "argmax_id"),
                               (argmax_val, (T,), torch.float32, "argmax_val")):
        if t is not None and (t.dtype != dt or tuple(t.shape) != shape or not (t.is_cuda and t.is_contiguous())):
            raise ValueError(f"{what} must be a contiguous CUDA {dt} tensor of shape {shape}")
    s = load_library().w4a16_head_gather_noalloc(_ptr(row_ids), n, _ptr(packed), _ptr(scales), n_rows, _ptr(x), K,
                                                 T, _ptr(out), _ptr(argmax_id), _ptr(argmax_val), _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_head_gather_noalloc")


class TiledWeight:
    """A weight in the tiled layout (one uint8 device buffer) with its shape."""

    def __init__(self, data: torch.Tensor, N: int, K: int):
        self.data, self.N, self.K = data, N, K

    @property
    def device(self):
        return self.data.device


def tiled_bytes(N: int, K: int) -> int:
    return int(load_library().w4a16_tiled_bytes(N, K))


def repack_tiled(packed: torch.Tensor, scales: torch.Tensor, stream=None) -> TiledWeight:
    """Tiled-layout copy of a row-major weight (runs on the GPU)."""
    N, K = _check_weight(packed, scales)
    nbytes = tiled_bytes(N, K)
    with _on(stream):
        data = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    s = load_library().w4a16_repack_tiled(_ptr(packed), _ptr(scales), N, K, _ptr(data), nbytes, _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_repack_tiled")
    return TiledWeight(data, N, K)


def repack_tiled_rows(packed: torch.Tensor, scales: torch.Tensor, row_ids: torch.Tensor, stream=None) -> TiledWeight:
    """Tiled-layout copy of rows row_ids of a row-major weight (a fixed-list
    head slice); row i of the result is input row row_ids[i]."""
    n_rows, K = _check_weight(packed, scales)
    if row_ids.dtype != torch.int32 or row_ids.dim() != 1 or not (row_ids.is_cuda and row_ids.is_contiguous()):
        raise ValueError("row_ids must be a contiguous CUDA int32 vector")
    n = row_ids.shape[0]
    nbytes = tiled_bytes(n, K)
    with _on(stream):
        data = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    s = load_library().w4a16_repack_tiled_rows(_ptr(packed), _ptr(scales), n_rows, K, _ptr(row_ids), n, _ptr(data),
                                               nbytes, _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_repack_tiled_rows")
    return TiledWeight(data, n, K)


def matmul_tiled(w: TiledWeight, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """matmul() on a tiled weight."""
    _check_bits(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [T][{w.K}]")
    T = x.shape[0]
    with _on(stream):
        y = out if out is not None else torch.empty((T, w.N), dtype=torch.float32, device=w.device)
    if y.dtype != torch.float32 or y.shape != (T, w.N) or not (y.is_cuda and y.is_contiguous()):
        raise ValueError("out must be a contiguous CUDA float32 tensor [T][N]")
    s = load_library().w4a16_matmul_tiled(_ptr(w.data), _ptr(x), _ptr(y), w.N, w.K, T, _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_matmul_tiled")
    return y


def head_gather_tiled(w: TiledWeight, x: torch.Tensor, row_ids: torch.Tensor | None = None, scores: bool = True,
                      argmax: bool = False, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None):
    """head_gather() on a tiled weight."""
    _check_bits(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [T][{w.K}]")
    T = x.shape[0]
    n = _row_ids(row_ids, w.N)
    with _on(stream):
        y, ids, vals, workspace, ws_bytes = _gather_outputs(n, T, w.device, scores, argmax, out, workspace)
    s = load_library().w4a16_head_gather_tiled(_ptr(row_ids), n, _ptr(w.data), w.N, _ptr(x), w.K, T, _ptr(y),
                                               _ptr(ids), _ptr(vals), _ptr(workspace), ws_bytes, _stream(stream))
    if s:
        raise W4A16Error(s, "w4a16_head_gather_tiled")
    return y, ids, vals


class _Problem(ctypes.Structure):
    _fields_ = [("packed_u4", ctypes.c_void_p), ("scales_bf16", ctypes.c_void_p), ("x_bf16", ctypes.c_void_p),
                ("y_f32", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("argmax_id", ctypes.c_void_p), ("argmax_val", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class Batch:
    """A planned grouped launch over independent matmuls with the same T.

    problems: list of (packed, scales, x, y) CUDA tensors, or (TiledWeight,
    None, x, y); either may carry three more entries (argmax_id int32 [T],
    argmax_val float32 [T] or None, workspace uint8 of workspace_bytes(N, T))
    for the per-row argmax of that problem's outputs.  The tensors must stay
    alive and in place while the batch is used; the plan is a host table plus
    its device copy (both held here).
    """

    def __init__(self, problems, T: int):
        lib = load_library()
        arr = (_Problem * len(problems))()
        self._keep = []
        for i, prob in enumerate(problems):
            packed, scales, x, y = prob[:4]
            am_id, am_val, ws = (tuple(prob[4:7]) + (None, None, None))[:3]
            if isinstance(packed, TiledWeight):
                N, K, layout, pp, sp = packed.N, packed.K, 1, packed.data.data_ptr(), None
            else:
                N, K = _check_weight(packed, scales)
                layout, pp, sp = 0, packed.data_ptr(), scales.data_ptr()
            _check_bits(x, "x")
            if x.shape != (T, K) or y.dtype != torch.float32 or y.shape != (T, N) or not y.is_contiguous():
                raise ValueError(f"problem {i}: x must be [T][K] and y float32 [T][N]")
            if am_id is not None:
                if am_id.dtype != torch.int32 or am_id.numel() != T or not am_id.is_cuda:
                    raise ValueError(f"problem {i}: argmax_id must be a CUDA int32 tensor of T entries")
                if am_val is not None and (am_val.dtype != torch.float32 or am_val.numel() != T):
                    raise ValueError(f"problem {i}: argmax_val must be a CUDA float32 tensor of T entries")
                if ws is None or not ws.is_cuda:
                    raise ValueError(f"problem {i}: argmax needs a CUDA workspace")
            arr[i] = _Problem(pp, sp, x.data_ptr(), y.data_ptr(), N, K, layout, 0,
                              _ptr(am_id), _ptr(am_val), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size())
            self._keep.append(tuple(prob))
        nbytes = lib.w4a16_batch_table_bytes(len(problems))
        if nbytes == 0:
            raise ValueError("batch size out of range")
        self.host = torch.empty(nbytes, dtype=torch.uint8)
        s = lib.w4a16_batch_plan(ctypes.cast(arr, ctypes.c_void_p), len(problems), T, self.host.data_ptr(), nbytes)
        if s:
            raise W4A16Error(s, "w4a16_batch_plan")
        self.device = self.host.to(problems[0][2].device, non_blocking=False)
        self.T = T
        self.count = len(problems)
        # no plan needs an activation workspace: the workgroups copy the bf16
        # activations straight into LDS (w4a16_batch_workspace_bytes is 0)
        self.workspace = None
        if lib.w4a16_batch_workspace_bytes(self.host.data_ptr()) != 0:
            raise RuntimeError("the library planned an activation workspace; this binding passes none")

    def run(self, stream=None) -> None:
        """One grouped launch (w4a16_matmul_batch) on `stream` (default: the current stream)."""
        s = load_library().w4a16_matmul_batch(self.host.data_ptr(), self.device.data_ptr(), _stream(stream))
        if s:
            raise W4A16Error(s, "w4a16_matmul_batch")


def topk_workspace_bytes(n: int, T: int, k: int) -> int:
    return int(load_library().w4a16_topk_workspace_bytes(n, T, k))


def topk(scores: torch.Tensor, k: int, row_ids: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         stream=None):
    """Per row t of scores [T][n] (float32): the k best (id, value) pairs,
    score descending, equal scores by ascending vocabulary id (row_ids[i], or
    i); NaN scores and negative ids never count; (-1, NaN) padding.
    Returns (ids [T][k] int32, values [T][k] float32)."""
    if scores.dtype != torch.float32 or scores.dim() != 2 or not (scores.is_cuda and scores.is_contiguous()):
        raise ValueError("scores must be a contiguous CUDA float32 tensor [T][n]")
    T, n = scores.shape
    if row_ids is not None and (row_ids.dtype != torch.int32 or row_ids.shape != (n,) or not row_ids.is_cuda
                                or not row_ids.is_contiguous()):
        raise ValueError("row_ids must be a contiguous CUDA int32 vector of n entries")
    nbytes = topk_workspace_bytes(n, T, k)
    if nbytes == 0:
        raise ValueError("topk: size out of range")
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=scores.device)
        ids = torch.empty((T, k), dtype=torch.int32, device=scores.device)
        vals = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    st = load_library().w4a16_topk(scores.data_ptr(), n, T, _ptr(row_ids), k, ids.data_ptr(), vals.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream))
    if st:
        raise W4A16Error(st, "w4a16_topk")
    return ids, vals


def greedy_accept(target_ids: torch.Tensor, draft_ids: torch.Tensor | None, n_seq: int, rows: int, stream=None):
    """Greedy verification of n_seq sequences of `rows` verify rows: returns
    (accepted drafts [n_seq] int32, emitted tokens [n_seq][rows] int32, -1 after
    the target model's token)."""
    for t, what in ((target_ids, "target_ids"), (draft_ids, "draft_ids")):
        if t is not None and (t.dtype != torch.int32 or not (t.is_cuda and t.is_contiguous())):
            raise ValueError(f"{what} must be a contiguous CUDA int32 tensor")
    if target_ids.numel() != n_seq * rows or (draft_ids is not None and draft_ids.numel() != n_seq * (rows - 1)):
        raise ValueError("target_ids must hold n_seq*rows ids and draft_ids n_seq*(rows-1)")
    with _on(stream):
        acc = torch.empty(n_seq, dtype=torch.int32, device=target_ids.device)
        tok = torch.empty((n_seq, rows), dtype=torch.int32, device=target_ids.device)
    st = load_library().w4a16_greedy_accept(target_ids.data_ptr(), _ptr(draft_ids), n_seq, rows, acc.data_ptr(),
                                            tok.data_ptr(), _stream(stream))
    if st:
        raise W4A16Error(st, "w4a16_greedy_accept")
    return acc, tok


def draft_union(base_ids: torch.Tensor | None, seq_ids: torch.Tensor | None, n_rows: int, stream=None):
    """Draft-head id list on the device: base ids, then the sequence's new
    in-range ids in order of first appearance, then -1.  Returns (ids
    [n_base + n_seq] int32, length [1] int32), both on the device."""
    for t, what in ((base_ids, "base_ids"), (seq_ids, "seq_ids")):
        if t is not None and (t.dtype != torch.int32 or t.dim() != 1 or not (t.is_cuda and t.is_contiguous())):
            raise ValueError(f"{what} must be a contiguous CUDA int32 vector")
    nb = 0 if base_ids is None else base_ids.numel()
    ns = 0 if seq_ids is None else seq_ids.numel()
    device = (base_ids if base_ids is not None else seq_ids).device
    with _on(stream):
        out = torch.empty(nb + ns, dtype=torch.int32, device=device)
        length = torch.empty(1, dtype=torch.int32, device=device)
    st = load_library().w4a16_draft_union(_ptr(base_ids) if nb else None, nb, _ptr(seq_ids) if ns else None, ns,
                                          n_rows, out.data_ptr(), length.data_ptr(), _stream(stream))
    if st:
        raise W4A16Error(st, "w4a16_draft_union")
    return out, length


def stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None) -> None:
    """Measurement helper: read all of src (a contiguous CUDA tensor whose
    byte size is a multiple of 16) once with nontemporal 16-byte loads over
    `workgroups` workgroups; sink is a CUDA int32 tensor of at least
    workgroups * 256 elements.  Its rate is the streaming-read ceiling."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32):
        raise ValueError("src must be a contiguous CUDA tensor and sink a CUDA int32 tensor")
    if sink.numel() < workgroups * 256:
        raise ValueError("sink must hold workgroups * 256 words")
    nbytes = src.numel() * src.element_size()
    st = load_library().w4a16_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), workgroups, _stream(stream))
    if st:
        raise W4A16Error(st, "w4a16_stream_read")
