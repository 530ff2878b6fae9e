"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only: the product path never builds or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")
OUT_SANITIZED = os.path.join(HERE, "liboracle_asan.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """sanitize: a host build with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts), written to liboracle_asan.so; the process that loads
    it must preload the ASan runtime (gcc -print-file-name=libasan.so)."""
    out = OUT_SANITIZED if sanitize else OUT
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"] if sanitize else ["-O2"]
    cmd = (["gcc"] + opt + ["-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
                            "-o", out + ".tmp", SRC, "-lm"])
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
