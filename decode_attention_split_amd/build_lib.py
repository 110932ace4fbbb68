"""Builds libgemma_attn.so (HIP, gfx950) in the package directory with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemma_attn.so")
SOURCES = ["api.hip", "decode_valu.hip", "decode_mfma.hip", "merge_append.hip"]
HEADERS = ["ga_device.h", "ga_internal.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False, extra_flags=None, out=None) -> str:
    out = out or LIB
    cmd = (["/opt/rocm/bin/hipcc"] + HIPCC_FLAGS + list(extra_flags or []) +
           ["-I", INCLUDE, "-I", CSRC] + sources() + ["-o", out + ".tmp"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
