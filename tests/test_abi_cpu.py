"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/w4a16.h declares, and rejects bad arguments on the host
(nothing reaches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
LIB = os.environ.get("W4A16_LIB") or os.path.join(ROOT, "speculative_verify_gemv_amd", "libw4a16.so")

OK, NULLP, SHAPE, ALIGN, WS, UNSUP, HIP, VARIANT, SCRATCH = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libw4a16.so not built")
    l = ctypes.CDLL(LIB)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    l.w4a16_matmul.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    l.w4a16_matmul.restype = i32
    l.w4a16_head_gather.argtypes = [vp, i64, vp, vp, i64, vp, i64, i32, vp, vp, vp, vp, sz, vp]
    l.w4a16_head_gather.restype = i32
    l.w4a16_workspace_bytes.argtypes = [i64, i32]
    l.w4a16_workspace_bytes.restype = sz
    l.w4a16_status_string.argtypes = [i32]
    l.w4a16_status_string.restype = ctypes.c_char_p
    l.w4a16_set_variant.argtypes = [i32]
    l.w4a16_set_variant.restype = i32
    l.w4a16_get_variant.restype = i32
    l.w4a16_tiled_tile_bytes.argtypes = [i64]
    l.w4a16_tiled_tile_bytes.restype = sz
    l.w4a16_tiled_bytes.argtypes = [i64, i64]
    l.w4a16_tiled_bytes.restype = sz
    l.w4a16_repack_tiled.argtypes = [vp, vp, i64, i64, vp, sz, vp]
    l.w4a16_repack_tiled.restype = i32
    l.w4a16_matmul_tiled.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    l.w4a16_matmul_tiled.restype = i32
    l.w4a16_head_gather_tiled.argtypes = [vp, i64, vp, i64, vp, i64, i32, vp, vp, vp, vp, sz, vp]
    l.w4a16_head_gather_tiled.restype = i32
    l.w4a16_batch_table_bytes.argtypes = [i32]
    l.w4a16_batch_table_bytes.restype = sz
    l.w4a16_batch_plan.argtypes = [vp, i32, i32, vp, sz]
    l.w4a16_batch_plan.restype = i32
    return l


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"w4a16_matmul", "w4a16_head_gather", "w4a16_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in w4a16.h but not exported"


def test_abi_version_and_strings(lib):
    assert lib.w4a16_abi_version() == 6
    for s in range(9):
        assert lib.w4a16_status_string(s)
    assert lib.w4a16_status_string(99) == b"unknown status"


A = 0x10000  # fake, suitably aligned device addresses: never dereferenced on a rejected call


def mm(lib, p=A, s=A, x=A, y=A, N=64, K=256, T=1):
    return lib.w4a16_matmul(p, s, x, y, N, K, T, None)


def test_matmul_rejections(lib):
    assert mm(lib, p=None) == NULLP
    assert mm(lib, s=None) == NULLP
    assert mm(lib, x=None) == NULLP
    assert mm(lib, y=None) == NULLP
    assert mm(lib, N=0) == SHAPE
    assert mm(lib, N=2**31) == SHAPE
    assert mm(lib, K=0) == SHAPE
    assert mm(lib, K=100) == SHAPE
    assert mm(lib, K=129) == SHAPE
    assert mm(lib, K=2**21) == SHAPE
    assert mm(lib, T=0) == SHAPE
    assert mm(lib, T=17) == SHAPE
    assert mm(lib, p=A + 8) == ALIGN
    assert mm(lib, x=A + 2) == ALIGN
    assert mm(lib, s=A + 1) == ALIGN
    assert mm(lib, y=A + 2) == ALIGN


def hg(lib, ids=A, n_ids=10, p=A, s=A, n_rows=100, x=A, K=256, T=2, y=A, am=None, av=None, ws=None, wsb=0):
    return lib.w4a16_head_gather(ids, n_ids, p, s, n_rows, x, K, T, y, am, av, ws, wsb, None)


def test_head_gather_rejections(lib):
    assert hg(lib, p=None) == NULLP
    assert hg(lib, y=None, am=None) == NULLP
    assert hg(lib, av=A) == NULLP                  # value without id
    assert hg(lib, n_ids=0) == SHAPE
    assert hg(lib, n_rows=0) == SHAPE
    assert hg(lib, ids=None, n_ids=10, n_rows=100) == SHAPE   # identity needs n_ids == n_rows
    assert hg(lib, T=17) == SHAPE
    assert hg(lib, K=200) == SHAPE
    assert hg(lib, ids=A + 2) == ALIGN
    assert hg(lib, am=A + 1) == ALIGN
    assert hg(lib, am=A) == WS                     # argmax without workspace
    need = lib.w4a16_workspace_bytes(10, 2)
    assert need > 0
    assert hg(lib, am=A, ws=A, wsb=need - 1) == WS
    assert hg(lib, am=A, ws=A + 8, wsb=need) == WS  # workspace must be 16-byte aligned


def test_workspace_bytes(lib):
    assert lib.w4a16_workspace_bytes(0, 1) == 0
    assert lib.w4a16_workspace_bytes(10, 0) == 0
    assert lib.w4a16_workspace_bytes(10, 17) == 0
    assert lib.w4a16_workspace_bytes(248320, 4) == 248320 // 16 * 4 * 8
    assert lib.w4a16_workspace_bytes(17, 1) == 2 * 8


def test_variant_selection(lib):
    assert lib.w4a16_set_variant(7) == VARIANT
    for v in (1, 2, 0):
        assert lib.w4a16_set_variant(v) == OK and lib.w4a16_get_variant() == v


def test_valid_call_without_gpu_fails_cleanly(lib):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert mm(lib) in (HIP, UNSUP)


def test_tiled_byte_counts(lib):
    # a tile: G blocks of 16 rows x 64 code bytes, plus 256 scale bytes per 8 groups
    assert lib.w4a16_tiled_tile_bytes(5120) == 40 * 1024 + 5 * 256
    assert lib.w4a16_tiled_tile_bytes(1152) == 9 * 1024 + 2 * 256      # G = 9: a short last chunk
    assert lib.w4a16_tiled_tile_bytes(128) == 1024 + 256
    assert lib.w4a16_tiled_tile_bytes(100) == 0
    # G % 8 == 0: exactly the row-major codes + scales (0.515625 B per weight)
    assert lib.w4a16_tiled_bytes(248320, 5120) == 248320 * 5120 // 2 + 2 * 248320 * 40
    assert lib.w4a16_tiled_bytes(17, 128) == 2 * (1024 + 256)           # rows padded to 32
    assert lib.w4a16_tiled_bytes(0, 128) == 0


def test_tiled_rejections(lib):
    need = lib.w4a16_tiled_bytes(64, 256)
    rp = lambda p=A, s=A, N=64, K=256, t=A, tb=need: lib.w4a16_repack_tiled(p, s, N, K, t, tb, None)
    assert rp(p=None) == NULLP and rp(s=None) == NULLP and rp(t=None) == NULLP
    assert rp(N=0) == SHAPE and rp(K=200) == SHAPE
    assert rp(t=A + 8) == ALIGN and rp(p=A + 8) == ALIGN and rp(s=A + 1) == ALIGN
    assert rp(tb=need - 1) == WS
    mt = lambda w=A, x=A, y=A, N=64, K=256, T=2: lib.w4a16_matmul_tiled(w, x, y, N, K, T, None)
    assert mt(w=None) == NULLP and mt(x=None) == NULLP and mt(y=None) == NULLP
    assert mt(N=0) == SHAPE and mt(K=129) == SHAPE and mt(T=17) == SHAPE
    assert mt(w=A + 4) == ALIGN and mt(x=A + 2) == ALIGN and mt(y=A + 2) == ALIGN
    gt = lambda ids=A, n_ids=10, w=A, n_rows=100, x=A, K=256, T=2, y=A, am=None, av=None, ws=None, wsb=0: \
        lib.w4a16_head_gather_tiled(ids, n_ids, w, n_rows, x, K, T, y, am, av, ws, wsb, None)
    assert gt(w=None) == NULLP and gt(y=None) == NULLP and gt(av=A) == NULLP
    assert gt(w=A + 8) == ALIGN and gt(ids=A + 2) == ALIGN
    assert gt(n_ids=0) == SHAPE and gt(ids=None) == SHAPE
    assert gt(am=A) == WS


class Problem(ctypes.Structure):
    _fields_ = [("packed_u4", ctypes.c_void_p), ("scales_bf16", ctypes.c_void_p), ("x_bf16", ctypes.c_void_p),
                ("y_f32", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("argmax_id", ctypes.c_void_p), ("argmax_val", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


def plan(lib, probs, T=4):
    arr = (Problem * len(probs))(*probs)
    nbytes = lib.w4a16_batch_table_bytes(len(probs))
    buf = (ctypes.c_uint64 * (nbytes // 8 + 1))()
    return lib.w4a16_batch_plan(ctypes.cast(arr, ctypes.c_void_p), len(probs), T, ctypes.addressof(buf), nbytes)


def test_batch_plan_layouts(lib):
    """Planning is host-only, so it runs here: both layouts accepted, bad fields rejected."""
    assert ctypes.sizeof(Problem) == 88
    row = Problem(A, A, A, A, 7168, 5120, 0, 0)
    tiled = Problem(A, None, A, A, 5120, 17408, 1, 0)
    assert plan(lib, [row, tiled]) == OK
    assert plan(lib, [Problem(A, None, A, A, 64, 256, 0, 0)]) == NULLP      # row-major needs scales
    assert plan(lib, [Problem(A, A, A, A, 64, 256, 2, 0)]) == SHAPE         # unknown layout
    assert plan(lib, [Problem(A, A, A, A, 64, 256, 1, 5)]) == SHAPE         # reserved must be 0
    assert plan(lib, [Problem(A + 8, None, A, A, 64, 256, 1, 0)]) == ALIGN  # tiled buffer 16-byte aligned


def test_batch_plan_argmax_fields(lib):
    """A problem's argmax: workspace of w4a16_workspace_bytes(N, T) bytes,
    16-byte aligned; argmax_val needs argmax_id; ids and values 4-byte aligned."""
    T, N, K = 4, 248320, 5120
    need = lib.w4a16_workspace_bytes(N, T)
    assert need == (N + 15) // 16 * T * 8
    head = lambda am=A, av=A, ws=A, wb=need: Problem(A, None, A, A, N, K, 1, 0, am, av, ws, wb)
    body = Problem(A, None, A, A, 7168, 5120, 1, 0)
    assert plan(lib, [body, head()], T) == OK
    assert plan(lib, [body, head(av=None)], T) == OK
    assert plan(lib, [body, head(am=None, av=None, ws=None, wb=0)], T) == OK   # no argmax: workspace unused
    assert plan(lib, [head(am=None)], T) == NULLP                              # value without id
    assert plan(lib, [head(ws=None)], T) == WS and plan(lib, [head(wb=need - 1)], T) == WS
    assert plan(lib, [head(ws=A + 8)], T) == WS
    assert plan(lib, [head(am=A + 2)], T) == ALIGN and plan(lib, [head(av=A + 1)], T) == ALIGN


def test_epilogue_arguments_rejected_on_the_host(lib):
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.w4a16_topk_workspace_bytes.argtypes = [i64, i32, i32]
    lib.w4a16_topk_workspace_bytes.restype = sz
    lib.w4a16_topk.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.w4a16_topk.restype = i32
    lib.w4a16_greedy_accept.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.w4a16_greedy_accept.restype = i32
    wsb = lib.w4a16_topk_workspace_bytes
    assert wsb(248320, 4, 32) == 4 * 122 * 32 * 8      # 2048 scores per first-stage chunk
    assert wsb(1, 1, 1) == 8
    assert wsb(0, 1, 1) == 0 and wsb(10, 17, 1) == 0 and wsb(10, 1, 33) == 0 and wsb(10, 1, 0) == 0
    need = wsb(1000, 2, 8)
    tk = lambda s=A, n=1000, T=2, ids=None, k=8, ti=A, tv=A, ws=A, b=need: \
        lib.w4a16_topk(s, n, T, ids, k, ti, tv, ws, b, None)
    assert tk(s=None) == NULLP and tk(ti=None) == NULLP
    assert tk(n=0) == SHAPE and tk(T=0) == SHAPE and tk(T=17) == SHAPE and tk(k=0) == SHAPE and tk(k=33) == SHAPE
    assert tk(s=A + 2) == ALIGN and tk(ids=A + 1) == ALIGN and tk(ti=A + 2) == ALIGN
    assert tk(ws=None) == WS and tk(b=need - 1) == WS and tk(ws=A + 8) == WS
    ga = lambda t=A, d=A, S=4, R=4, acc=A, tok=A: lib.w4a16_greedy_accept(t, d, S, R, acc, tok, None)
    assert ga(t=None) == NULLP and ga(acc=None) == NULLP and ga(d=None) == NULLP
    assert ga(S=0) == SHAPE and ga(R=0) == SHAPE and ga(R=17) == SHAPE
    assert ga(t=A + 2) == ALIGN and ga(tok=A + 1) == ALIGN


def test_draft_union_arguments_rejected_on_the_host(lib):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.w4a16_draft_union.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp]
    lib.w4a16_draft_union.restype = i32
    du = lambda b=A, nb=32768, s=A, ns=100, n=248320, o=A, m=A: lib.w4a16_draft_union(b, nb, s, ns, n, o, m, None)
    assert du(o=None) == NULLP and du(m=None) == NULLP and du(b=None) == NULLP and du(s=None) == NULLP
    assert du(nb=-1) == SHAPE and du(ns=4097) == SHAPE and du(nb=0, ns=0) == SHAPE
    assert du(n=0) == SHAPE and du(n=524289) == SHAPE
    assert du(b=A + 2) == ALIGN and du(o=A + 1) == ALIGN and du(m=A + 2) == ALIGN


def test_stream_read_arguments_rejected_on_the_host(lib):
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.w4a16_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.w4a16_stream_read.restype = i32
    sr = lambda s=A, n=1 << 20, k=A, w=2048: lib.w4a16_stream_read(s, n, k, w, None)
    assert sr(s=None) == NULLP and sr(k=None) == NULLP
    assert sr(n=0) == SHAPE and sr(n=1000) == SHAPE and sr(w=0) == SHAPE and sr(w=65537) == SHAPE
    assert sr(s=A + 8) == ALIGN and sr(k=A + 2) == ALIGN


def test_batch_workspace_planning_and_checks(lib):
    """Grouped launches need no activation workspace at any T (the
    workgroups copy the bf16 activations straight into LDS):
    w4a16_batch_workspace_bytes is 0, and w4a16_matmul_batch_ws accepts a
    NULL workspace and checks the tables as w4a16_matmul_batch does, before
    touching the device."""
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.w4a16_batch_workspace_bytes.argtypes = [vp]
    lib.w4a16_batch_workspace_bytes.restype = sz
    lib.w4a16_matmul_batch_ws.argtypes = [vp, vp, vp, sz, vp]
    lib.w4a16_matmul_batch_ws.restype = i32
    shapes = [(7168, 5120), (5120, 17408), (17, 128)]
    probs = [Problem(A, None, A, A, n, k, 1, 0) for n, k in shapes]

    def table(T):
        arr = (Problem * len(probs))(*probs)
        nbytes = lib.w4a16_batch_table_bytes(len(probs))
        buf = (ctypes.c_uint64 * (nbytes // 8 + 1))()
        assert lib.w4a16_batch_plan(ctypes.cast(arr, vp), len(probs), T, ctypes.addressof(buf), nbytes) == OK
        return buf

    for T in (1, 4, 8, 9, 12, 16):
        tb = table(T)
        assert lib.w4a16_batch_workspace_bytes(ctypes.addressof(tb)) == 0
        run = lambda ws=None, n=0, t=ctypes.addressof(tb), d=A: lib.w4a16_matmul_batch_ws(t, d, ws, n, None)
        assert run(t=None) == NULLP and run(d=None) == NULLP and run(d=A + 8) == ALIGN
        assert run() in (UNSUP, HIP) and run(ws=A, n=64) in (UNSUP, HIP)  # the device check is next
    junk = (ctypes.c_uint64 * 16)()
    assert lib.w4a16_batch_workspace_bytes(ctypes.addressof(junk)) == 0
    assert lib.w4a16_batch_workspace_bytes(None) == 0


def test_head_gather_noalloc_limits(lib):
    """The allocation-free head call checks its arguments like
    w4a16_head_gather, needs no workspace, and refuses (before the device
    is touched) argmax partials larger than its static scratch."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = lib.w4a16_head_gather_noalloc
    f.argtypes = [vp, i64, vp, vp, i64, vp, i64, i32, vp, vp, vp, vp]
    f.restype = i32
    call = lambda ids=A, n_ids=10, p=A, s=A, n_rows=100, x=A, K=256, T=2, y=A, am=None, av=None: \
        f(ids, n_ids, p, s, n_rows, x, K, T, y, am, av, None)
    assert call(p=None) == NULLP and call(y=None) == NULLP and call(av=A) == NULLP
    assert call(n_ids=0) == SHAPE and call(T=17) == SHAPE and call(ids=A + 2) == ALIGN
    limit = 2 << 20
    assert lib.w4a16_workspace_bytes(262144, 16) == limit
    assert call(n_ids=262145, n_rows=300000, T=16, am=A) == SCRATCH
    assert call(n_ids=262145, n_rows=300000, T=16, am=None) in (UNSUP, HIP)  # no argmax: no scratch used
    assert call(n_ids=262144, n_rows=300000, T=16, am=A) in (UNSUP, HIP)     # exactly the limit
    assert call(am=A) in (UNSUP, HIP)                                       # no workspace needed


def test_tile_override_parsing(lib):
    """The measurement tile override: bad specs and batch values are rejected,
    valid ones accepted, NULL or "" restores the planner's choice."""
    f = lib.w4a16_set_tile
    f.argtypes = [ctypes.c_int32, ctypes.c_char_p]
    assert f(2, b"split,1,8") == SHAPE
    for spec in (b"split,3,8", b"split,1,9", b"run,0,4", b"run,17,4", b"shared,1,17", b"bogus,1,1", b"split,1"):
        assert f(0, spec) == SHAPE, spec
    for batch in (0, 1):
        for spec in (b"split,1,8", b"shared,4,2", b"run,16,16"):
            assert f(batch, spec) == OK, spec
        assert f(batch, b"") == OK and f(batch, None) == OK


def test_batch_plan_kernel_layout(lib):
    """The table records which kernels a grouped launch runs: built for the
    tiled layout (every problem tiled), for row-major weights (every problem
    row-major) or for either (a mix); runs of tiles only for one layout, and
    a table that asks for runs over both is refused before the device."""
    lib.w4a16_matmul_batch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.w4a16_matmul_batch.restype = ctypes.c_int32
    K_SHARED, K_RUN = 3, 4  # the header's variant codes

    def header(probs, T):
        arr = (Problem * len(probs))(*probs)
        nbytes = lib.w4a16_batch_table_bytes(len(probs))
        buf = (ctypes.c_uint64 * (nbytes // 8 + 1))()
        assert lib.w4a16_batch_plan(ctypes.cast(arr, ctypes.c_void_p), len(probs), T, ctypes.addressof(buf),
                                    nbytes) == OK
        words = (ctypes.c_int32 * 16).from_buffer(buf)
        return buf, words  # words[4] variant, words[5] rt, words[6] kernel layout

    row = [Problem(A, A, A, A, 7168, 5120, 0, 0), Problem(A, A, A, A, 5120, 17408, 0, 0)]
    tiled = [Problem(A, None, A, A, 7168, 5120, 1, 0), Problem(A, None, A, A, 5120, 17408, 1, 0)]
    mixed = [row[0], tiled[1]]
    for T in (1, 2, 4, 8, 16):
        _, w = header(row, T)
        assert w[6] == 2 and w[4] == (K_SHARED if T <= 2 else K_RUN)
        _, w = header(tiled, T)
        assert w[6] == 1 and w[4] == (K_SHARED if T <= 2 else K_RUN)
        buf, w = header(mixed, T)
        assert w[6] == 0 and w[4] == K_SHARED
        w[4] = K_RUN  # runs over a mix of layouts: refused
        assert lib.w4a16_matmul_batch(ctypes.addressof(buf), A, None) == SHAPE
        w[4], w[6] = K_SHARED, 3  # an unknown kernel layout: refused
        assert lib.w4a16_matmul_batch(ctypes.addressof(buf), A, None) == SHAPE
