"""Compile libmk.so (the persistent decode kernel, the MLA attention kernels and their C ABI) for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_kernel.hip", "mk_runtime.hip", "mla.hip"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    cmd = (["hipcc"] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB + ".tmp"])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError("libmk build failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
