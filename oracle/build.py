"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only: only the tests, the smoke check and the bench's CPU
baseline leg load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, cc: str = "gcc", extra=(), lib: str = LIB) -> str:
    """extra flags and another output place an instrumented build beside this one."""
    src = os.path.join(HERE, "oracle.c")
    tmp = lib + ".tmp"
    # -ffp-contract=off: no fused multiply-adds, every operation rounds as written.
    cmd = [cc, *extra, "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
