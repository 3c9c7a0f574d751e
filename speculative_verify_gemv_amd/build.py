"""Compile the HIP library libw4a16.so for gfx950 (hipcc, in-tree).

The kernel templates are instantiated once per activation-row count T
(w4a16_kernels_tt.hip built sixteen times with -DW4A16_TT=1..16); those
objects, the planning / dispatch unit and the C ABI unit compile in
parallel and are linked into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
OBJ_DIR = os.path.join(ROOT, "_build", "w4a16")
MAX_T = 16

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def _units(obj_dir=OBJ_DIR):
    """(source, object, extra flags) of every translation unit."""
    units = [(os.path.join(CSRC, "w4a16_kernels_tt.hip"), os.path.join(obj_dir, f"kernels_t{t}.o"),
              [f"-DW4A16_TT={t}"]) for t in range(1, MAX_T + 1)]
    units.append((os.path.join(CSRC, "w4a16_kernels.hip"), os.path.join(obj_dir, "kernels.o"), []))
    units.append((os.path.join(CSRC, "w4a16_epilogue.hip"), os.path.join(obj_dir, "epilogue.o"), []))
    units.append((os.path.join(CSRC, "w4a16_api.hip"), os.path.join(obj_dir, "api.o"), []))
    return units


def build(verbose: bool = False, extra=(), link_extra=(), lib: str = LIB, obj_dir: str = OBJ_DIR) -> str:
    """Builds the library; extra / link_extra are added to every compile / to
    the link, lib and obj_dir place another build (an instrumented one) beside
    the product's."""
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src, obj, flags in _units(obj_dir):
        jobs.append([hipcc(), *HIPCC_FLAGS, *extra, *flags, *inc, "-c", "-o", obj, src])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(lambda c: _run(c, verbose), jobs))
    failed = [(c, e) for c, (rc, e) in zip(jobs, results) if rc != 0]
    for c, e in failed:
        sys.stderr.write(f"{c[-1]}:\n{e}\n")
    if failed:
        raise RuntimeError("hipcc failed building libw4a16.so")
    if verbose:
        for rc, e in results:
            if e.strip():
                sys.stderr.write(e + "\n")
    tmp = lib + ".tmp"
    rc, err = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, "-o", tmp,
                    *[obj for _, obj, _ in _units(obj_dir)]], verbose)
    if rc != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed linking libw4a16.so")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
