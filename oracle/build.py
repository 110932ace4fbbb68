"""Builds oracle/liboracle.so from oracle/oracle.c with the host C compiler.

Test infrastructure only: the library it builds is loaded by the tests, the smoke
check and the benchmark's CPU-baseline leg, never by the GPU library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without fast-math: libm exp/tanh/log and IEEE double arithmetic as written.
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-Wall", "-Wextra", "-fPIC",
           "-shared", "-pthread", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
