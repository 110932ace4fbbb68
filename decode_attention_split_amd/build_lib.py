"""Builds libgemma_attn.so (HIP, gfx950) in the package directory with hipcc.

Every source compiles to its own object in parallel (the vector kernels are split by head
dim over three sources so that their instantiations compile side by side), then one
link makes the shared library.
"""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemma_attn.so")
SOURCES = ["api.hip", "decode_valu.hip", "decode_valu_d128.hip", "decode_valu_d256.hip",
           "decode_valu_d512.hip", "decode_mfma.hip", "decode_rows16.hip", "merge_append.hip",
           "stream_read.hip"]
HEADERS = ["ga_device.h", "ga_internal.h", "ga_mfma.h", "decode_valu_impl.h"]

HIPCC = "/opt/rocm/bin/hipcc"
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source flags.  The multi-token kernel keeps its matrix-core accumulators in ordinary
# VGPRs (it has the room at its occupancy), so the rescale of the accumulators takes no
# copies between AGPRs and VGPRs; the global kernel needs the AGPRs for its 128-register
# accumulator.
SOURCE_FLAGS = {"decode_rows16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False, extra_flags=None, out=None, jobs: int = 0) -> str:
    out = out or LIB
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="ga_build_") as tmp:
        objs, procs = [], []
        pending = list(sources())
        while pending or procs:
            while pending and len(procs) < jobs:
                src = pending.pop(0)
                obj = os.path.join(tmp, os.path.basename(src) + ".o")
                cmd = ([HIPCC] + HIPCC_FLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) +
                       list(extra_flags or []) + ["-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
                if verbose:
                    print(" ".join(cmd), flush=True)
                procs.append((subprocess.Popen(cmd), cmd))
                objs.append(obj)
            proc, cmd = procs.pop(0)
            if proc.wait() != 0:
                for p, _ in procs:
                    p.wait()
                raise subprocess.CalledProcessError(proc.returncode, cmd)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
