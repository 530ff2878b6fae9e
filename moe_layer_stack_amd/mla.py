"""ctypes binding of the MLA attention calls (include/mk_mla.h) in libmk.so:
argument marshalling only; the attention runs in the library's HIP kernels."""
import ctypes as C

from ._lib import MK_OK, MkError, lib as _mk_lib, mk_strerror

MLA_EXPORTS = ("mk_mla_create", "mk_mla_attention", "mk_mla_sync", "mk_mla_get_info", "mk_mla_destroy",
               "mk_mla_last_error")
MLA_LATENT_DIM, MLA_ROPE_DIM = 512, 64


class mk_mla_config(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("latent_dim", C.c_int32), ("rope_dim", C.c_int32), ("rows", C.c_int32),
                ("rows_per_seq", C.c_int32), ("n_seq", C.c_int32), ("capacity", C.c_int32), ("scale", C.c_float)]


class mk_mla_info(C.Structure):
    _fields_ = [("splits", C.c_int32), ("workgroups", C.c_int32), ("workspace_bytes", C.c_int64)]


_done = False


def lib():
    global _done
    L = _mk_lib()
    if not _done:
        L.mk_mla_create.argtypes = [C.POINTER(mk_mla_config), C.POINTER(C.c_void_p)]
        L.mk_mla_attention.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.mk_mla_sync.argtypes = [C.c_void_p, C.c_void_p]
        L.mk_mla_get_info.argtypes = [C.c_void_p, C.POINTER(mk_mla_info)]
        L.mk_mla_destroy.argtypes = [C.c_void_p]
        L.mk_mla_last_error.argtypes = []
        L.mk_mla_last_error.restype = C.c_char_p
        for f in ("mk_mla_create", "mk_mla_attention", "mk_mla_sync", "mk_mla_get_info", "mk_mla_destroy"):
            getattr(L, f).restype = C.c_int
        _done = True
    return L


def mk_mla_last_error() -> str:
    return lib().mk_mla_last_error().decode()


def _check(rc):
    if rc != MK_OK:
        raise MkError(rc, f"{mk_strerror(rc)}: {mk_mla_last_error()}")
    return rc


def mk_mla_create(cfg: mk_mla_config) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib().mk_mla_create(C.byref(cfg), C.byref(h)))
    return h


def mk_mla_attention(h, q: int, cache: int, positions: int, out: int, stream: int = 0) -> int:
    """q, cache, positions, out: device addresses (see include/mk_mla.h)."""
    return _check(lib().mk_mla_attention(h, C.c_void_p(q), C.c_void_p(cache), C.c_void_p(positions),
                                         C.c_void_p(out), C.c_void_p(stream)))


def mk_mla_sync(h, stream: int = 0) -> int:
    return lib().mk_mla_sync(h, C.c_void_p(stream))


def mk_mla_get_info(h) -> mk_mla_info:
    info = mk_mla_info()
    _check(lib().mk_mla_get_info(h, C.byref(info)))
    return info


def mk_mla_destroy(h) -> int:
    return lib().mk_mla_destroy(h)
