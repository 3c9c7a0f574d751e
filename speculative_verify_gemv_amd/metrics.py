"""Reporting arithmetic of the bench (host-side, no GPU).

Decode reads every weight once per cycle, so its speed is bounded by bytes
over bandwidth: with G gigabytes read per cycle, peak bandwidth B, the
fraction eta of it the kernels reach and tau tokens committed per cycle,
tokens/s <= eta * B * tau / G (qwen-warp/llamAmpere article, "The
arithmetic every claim answers to"; the formula itself was lost from the
extracted text, its symbols are defined in the same paragraph and its
printed examples fix this reading).
"""

import hashlib
import os
import re

GROUP = 128

# the sources whose compiled form the committed counter summaries describe
KERNEL_SOURCES = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", f)
                  for f in ("w4a16_device.h", "w4a16_internal.h", "w4a16_kernels.hip", "w4a16_kernels_tt.hip",
                            "w4a16_api.hip")]


def kernel_source_hash() -> str:
    """sha256 of the kernel sources with comments and blank space removed (a
    comment edit does not change the kernels the counters were taken on)."""
    text = ""
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.strip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def weight_bytes(n_rows: int, k: int) -> int:
    """Bytes of a W4A16 group-128 weight: 4-bit codes plus one bf16 scale per 128 inputs."""
    return n_rows * k // 2 + 2 * n_rows * (k // GROUP)


def gbps(nbytes: float, ms: float) -> float:
    """GB/s (10^9 bytes per second) for nbytes moved in ms milliseconds."""
    return nbytes / (ms * 1e-3) / 1e9


def fraction_of_peak(achieved_gbps: float, peak_gbps: float) -> float:
    return achieved_gbps / peak_gbps


def decode_ceiling_tok_s(eta: float, peak_gbps: float, gb_per_cycle: float, tokens_per_cycle: float = 1.0) -> float:
    """Upper bound on decode tokens/s: eta * B * tau / G."""
    return eta * peak_gbps * tokens_per_cycle / gb_per_cycle


def cycles_per_s(ms_per_cycle: float) -> float:
    return 1000.0 / ms_per_cycle
