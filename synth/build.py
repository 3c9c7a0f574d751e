"""Compile the seeded input generator (plain C, gcc) into synth/libsynth.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")


def build(verbose: bool = False, cc: str = "gcc", extra=(), lib: str = LIB) -> str:
    """extra flags and another output place an instrumented build beside this one."""
    src = os.path.join(HERE, "synth.c")
    tmp = lib + ".tmp"
    cmd = [cc, *extra, "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
