"""ctypes binding of libmk.so (include/mk.h): argument marshalling only.

Every step of the decode path runs in the HIP kernels of libmk.so; there is no
Python or CPU fallback.  Loading fails loudly when the library is not built.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_UNSUPPORTED = -2
MK_ERR_DEVICE = -3
MK_ERR_HIP = -4
MK_ERR_TIMEOUT = -5
MK_F32, MK_BF16 = 0, 1

EXPORTS = ("mk_create", "mk_decode_step", "mk_decode_step_phased", "mk_decode_step_noalloc", "mk_destroy", "mk_sync",
           "mk_set_trace", "mk_set_timing", "mk_set_watchdog", "mk_get_info", "mk_strerror", "mk_last_error")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MK_NOALLOC_SCRATCH_BYTES


class MkError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class mk_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("n_shared", C.c_int32), ("d_ff", C.c_int32), ("dtype", C.c_int32),
                ("has_router_bias", C.c_int32), ("rms_eps", C.c_float), ("has_attn", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("rope_theta", C.c_float), ("rows", C.c_int32), ("rows_per_seq", C.c_int32),
                ("kv_capacity", C.c_int32)]


class mk_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "moe_norm", "w_router",
                                          "b_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")]


class mk_kv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n_seq", C.c_int32), ("capacity", C.c_int32)]


class mk_info(C.Structure):
    _fields_ = [("n_cu", C.c_int32), ("threads", C.c_int32), ("lds_bytes", C.c_int32),
                ("barriers_per_step", C.c_int32), ("attn_splits", C.c_int32), ("launches_per_step", C.c_int32),
                ("workspace_bytes", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                              "python -m moe_layer_stack_amd.build")
        L = C.CDLL(LIB_PATH)
        L.mk_create.argtypes = [C.POINTER(mk_config), C.POINTER(mk_layer_weights), C.POINTER(C.c_void_p)]
        L.mk_decode_step.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(mk_kv_cache), C.c_void_p,
                                     C.c_void_p]
        L.mk_decode_step_phased.argtypes = L.mk_decode_step.argtypes
        L.mk_decode_step_noalloc.argtypes = L.mk_decode_step.argtypes
        L.mk_destroy.argtypes = [C.c_void_p]
        L.mk_sync.argtypes = [C.c_void_p, C.c_void_p]
        L.mk_set_trace.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.mk_set_timing.argtypes = [C.c_void_p, C.c_void_p]
        L.mk_set_watchdog.argtypes = [C.c_void_p, C.c_int64]
        L.mk_get_info.argtypes = [C.c_void_p, C.POINTER(mk_info)]
        L.mk_strerror.argtypes = [C.c_int]
        L.mk_strerror.restype = C.c_char_p
        L.mk_last_error.argtypes = []
        L.mk_last_error.restype = C.c_char_p
        for f in ("mk_create", "mk_decode_step", "mk_decode_step_phased", "mk_decode_step_noalloc", "mk_destroy",
                  "mk_sync", "mk_set_trace", "mk_set_timing", "mk_set_watchdog", "mk_get_info"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != MK_OK:
        raise MkError(rc, f"{mk_strerror(rc)}: {mk_last_error()}")
    return rc


def mk_strerror(status: int) -> str:
    return lib().mk_strerror(status).decode()


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


def mk_create(cfg: mk_config, layers) -> C.c_void_p:
    """layers: sequence of mk_layer_weights (device pointers).  Returns the handle."""
    arr = (mk_layer_weights * len(layers))(*layers)
    h = C.c_void_p()
    _check(lib().mk_create(C.byref(cfg), arr, C.byref(h)))
    return h


def mk_decode_step(h, hidden_in: int, positions: int, kv, hidden_out: int, stream: int = 0) -> int:
    kvp = C.byref(kv) if kv is not None else None
    return _check(lib().mk_decode_step(h, C.c_void_p(hidden_in), C.c_void_p(positions), kvp,
                                       C.c_void_p(hidden_out), C.c_void_p(stream) if stream else None))


def mk_decode_step_phased(h, hidden_in: int, positions: int, kv, hidden_out: int, stream: int = 0) -> int:
    kvp = C.byref(kv) if kv is not None else None
    return _check(lib().mk_decode_step_phased(h, C.c_void_p(hidden_in), C.c_void_p(positions), kvp,
                                              C.c_void_p(hidden_out), C.c_void_p(stream) if stream else None))


def mk_decode_step_noalloc(h, hidden_in: int, positions: int, kv, hidden_out: int, stream: int = 0) -> int:
    kvp = C.byref(kv) if kv is not None else None
    return _check(lib().mk_decode_step_noalloc(h, C.c_void_p(hidden_in), C.c_void_p(positions), kvp,
                                               C.c_void_p(hidden_out), C.c_void_p(stream) if stream else None))


def mk_destroy(h) -> int:
    return _check(lib().mk_destroy(h))


def mk_sync(h, stream: int = 0) -> int:
    """Returns the status (does not raise), so callers can test device-side errors."""
    return lib().mk_sync(h, C.c_void_p(stream) if stream else None)


def mk_set_trace(h, ids: int = 0, w: int = 0, logits: int = 0) -> int:
    return _check(lib().mk_set_trace(h, C.c_void_p(ids or None), C.c_void_p(w or None),
                                     C.c_void_p(logits or None)))


def mk_set_timing(h, stamps: int = 0) -> int:
    return _check(lib().mk_set_timing(h, C.c_void_p(stamps or None)))


def mk_set_watchdog(h, ticks: int) -> int:
    return _check(lib().mk_set_watchdog(h, C.c_int64(int(ticks))))


def mk_get_info(h) -> mk_info:
    info = mk_info()
    _check(lib().mk_get_info(h, C.byref(info)))
    return info
