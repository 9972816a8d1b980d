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


def build_sanitized(out_path: str, verbose: bool = False) -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (every report fatal), for running the oracle's pins under them.  Loading it
    into Python needs the ASan runtime preloaded (see sanitizer_runtime)."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wextra", SRC, "-o", out_path, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out_path


def sanitizer_runtime() -> str:
    """Path of gcc's ASan runtime library (to preload)."""
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
