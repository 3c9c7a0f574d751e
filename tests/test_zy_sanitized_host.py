"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle.c), the input generator (synth.c) and the host side of
libw4a16 (argument checks, planning, batch tables, the C ABI; its GPU code is
built as usual) are built instrumented into _build/sanitize/<source hash>/,
and the CPU test suite runs again in a child process that loads those builds
(ORACLE_LIB, SYNTH_LIB, W4A16_LIB) with the sanitizer runtime preloaded.  Any
report (an out-of-bounds access, a use after free, a signed overflow, a bad
shift, a misaligned access ...) aborts the child and fails this test.  The
first run after a source change builds for a minute or two (and removes the
builds of earlier sources); later runs reuse the build.  Leak checking is
off: the Python interpreter itself is not instrumented and keeps its
allocations until exit.
"""
import ctypes
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.environ.get("W4A16_SANITIZED") == "1"
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")

# instrumentation of the host code; for hipcc each flag goes to the host
# compilation only, the GPU code is compiled as in the product build
C_SAN = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
HIP_HOST_SAN = ["-g", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _sources():
    files = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c")]
    files += sorted(glob.glob(os.path.join(ROOT, "speculative_verify_gemv_amd", "csrc", "*")))
    files += sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    return files


def _source_hash():
    h = hashlib.sha256()
    for f in _sources():
        h.update(f.encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(C_SAN + HIP_HOST_SAN).encode())
    return h.hexdigest()[:16]


def _runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(out_dir):
    # builds of earlier sources are of no further use (about 150-250 MB each)
    parent = os.path.dirname(out_dir)
    if os.path.isdir(parent):
        for name in os.listdir(parent):
            if os.path.join(parent, name) != out_dir:
                shutil.rmtree(os.path.join(parent, name), ignore_errors=True)
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    from synth import build as synth_build
    from speculative_verify_gemv_amd import build as lib_build

    os.makedirs(out_dir, exist_ok=True)
    libs = {"ORACLE_LIB": os.path.join(out_dir, "liboracle.so"), "SYNTH_LIB": os.path.join(out_dir, "libsynth.so"),
            "W4A16_LIB": os.path.join(out_dir, "libw4a16.so")}
    if all(os.path.exists(p) for p in libs.values()):
        return libs
    oracle_build.build(cc=CLANG, extra=C_SAN, lib=libs["ORACLE_LIB"])
    synth_build.build(cc=CLANG, extra=C_SAN, lib=libs["SYNTH_LIB"])
    lib_build.build(extra=HIP_HOST_SAN, lib=libs["W4A16_LIB"], obj_dir=os.path.join(out_dir, "obj"))
    return libs


@pytest.mark.skipif(CHILD, reason="the instrumented run itself")
def test_cpu_suite_under_address_and_undefined_behaviour_sanitizers():
    if not os.path.exists(CLANG):
        pytest.skip("no clang with sanitizer runtimes")
    runtime = _runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime")
    libs = _build(os.path.join(ROOT, "_build", "sanitize", _source_hash()))
    env = dict(os.environ, **libs)
    env.update(W4A16_SANITIZED="1", LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out


@pytest.mark.skipif(not CHILD, reason="runs inside the instrumented run only")
def test_the_instrumented_builds_are_the_ones_loaded():
    """In the child: the sanitizer runtime is in the process, and the oracle,
    the generator and the library are the instrumented builds."""
    import oracle
    import synth
    import speculative_verify_gemv_amd as w4a16

    assert ctypes.CDLL(None).__getattr__("__asan_init") is not None
    assert oracle._LIB_PATH == os.environ["ORACLE_LIB"]
    assert synth._LIB_PATH == os.environ["SYNTH_LIB"]
    assert w4a16.LIB_PATH == os.environ["W4A16_LIB"]
    for path in (os.environ["ORACLE_LIB"], os.environ["SYNTH_LIB"], os.environ["W4A16_LIB"]):
        lib = ctypes.CDLL(path)
        assert lib is not None
    # the instrumented library reaches the sanitizer runtime
    maps = open("/proc/self/maps").read()
    assert "libclang_rt.asan" in maps and os.environ["W4A16_LIB"] in maps
