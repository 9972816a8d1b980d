"""Build the CPU oracle shared library (test infrastructure only).

Compiles oracle/oracle.c with gcc into oracle/liboracle.so.  Nothing on the GPU
product path links or loads the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
