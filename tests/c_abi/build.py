"""Compile tests/c_abi/abi_check.c (a plain-C client of libw4a16, checked
against the oracle) into _build/abi_check with gcc.  Test infrastructure:
run by tests/test_gpu_c_abi.py."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "abi_check")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           "-I" + os.path.join(ROOT, "include"), "-o", OUT + ".tmp", os.path.join(HERE, "abi_check.c"),
           "-L" + os.path.join(ROOT, "speculative_verify_gemv_amd"), "-lw4a16",
           "-L" + os.path.join(ROOT, "oracle"), "-loracle", f"-L{rocm}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../speculative_verify_gemv_amd", "-Wl,-rpath,$ORIGIN/../oracle",
           f"-Wl,-rpath,{rocm}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
