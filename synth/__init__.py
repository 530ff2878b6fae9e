"""Seeded synthetic inputs for the MoE decode stack (Philox4x32-10 + Box-Muller).

A module of its own, holding none of the decode step's arithmetic: it serves
both the GPU path (device fills into torch-allocated memory) and the oracle's
tests (host fills into numpy arrays).  Each tensor has its own Philox stream,
so any one tensor, or any one expert, can be regenerated on either side.

bf16 tensors are carried on the host as uint16 bit patterns.
"""
import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsynth.so")
F32, BF16 = 0, 1

# stream kinds (one Philox stream per tensor: layer, kind, index)
K_G1, K_WQ, K_WK, K_WV, K_WO, K_G2, K_WR, K_BR = 1, 2, 3, 4, 5, 6, 7, 8
K_WGATE, K_WUP, K_WDOWN, K_SGATE, K_SUP, K_SDOWN = 9, 10, 11, 12, 13, 14
K_HIDDEN, K_KCACHE, K_VCACHE = 20, 21, 22
K_MLA_CACHE, K_MLA_Q = 23, 24  # latent cache rows and absorbed queries of the MLA attention

_lib = None


def build(verbose=False):
    """Compile libsynth.so (host + gfx950 device code)."""
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "synth.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("synth build failed:\n" + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        u64, dbl, vp = C.c_uint64, C.c_double, C.c_void_p
        L.synth_philox4x32_10.argtypes = [C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), C.POINTER(C.c_uint32)]
        for name in ("synth_fill_normal_host", "synth_fill_uniform_host"):
            getattr(L, name).argtypes = [vp, C.c_int, u64, u64, u64, dbl, dbl]
            getattr(L, name).restype = C.c_int
        for name in ("synth_fill_normal_device", "synth_fill_uniform_device"):
            getattr(L, name).argtypes = [vp, C.c_int, u64, u64, u64, dbl, dbl, vp]
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def stream_id(layer: int, kind: int, index: int = 0) -> int:
    """Philox stream of one tensor: layer (or -1 for per-step inputs), kind, index."""
    return (((layer + 1) & 0xFFFFFFFF) << 32) | ((kind & 0xFFFF) << 16) | (index & 0xFFFF)


def philox(ctr, key):
    c = (C.c_uint32 * 4)(*ctr)
    k = (C.c_uint32 * 2)(*key)
    o = (C.c_uint32 * 4)()
    lib().synth_philox4x32_10(c, k, o)
    return tuple(o)


def _np_dtype(dtype):
    return np.uint16 if dtype == BF16 else np.float32


def host_normal(shape, dtype, seed, stream, mean=0.0, std=1.0):
    a = np.empty(shape, dtype=_np_dtype(dtype))
    rc = lib().synth_fill_normal_host(a.ctypes.data, dtype, a.size, seed, stream, mean, std)
    assert rc == 0
    return a


def host_uniform(shape, dtype, seed, stream, lo, hi):
    a = np.empty(shape, dtype=_np_dtype(dtype))
    rc = lib().synth_fill_uniform_host(a.ctypes.data, dtype, a.size, seed, stream, lo, hi)
    assert rc == 0
    return a


def device_normal(ptr, n, dtype, seed, stream, mean=0.0, std=1.0, hip_stream=None):
    rc = lib().synth_fill_normal_device(C.c_void_p(ptr), dtype, n, seed, stream, mean, std,
                                        C.c_void_p(hip_stream) if hip_stream else None)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_device failed ({rc})")


def device_uniform(ptr, n, dtype, seed, stream, lo, hi, hip_stream=None):
    rc = lib().synth_fill_uniform_device(C.c_void_p(ptr), dtype, n, seed, stream, lo, hi,
                                         C.c_void_p(hip_stream) if hip_stream else None)
    if rc != 0:
        raise RuntimeError(f"synth_fill_uniform_device failed ({rc})")


def bf16_bits_to_f32(a):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
