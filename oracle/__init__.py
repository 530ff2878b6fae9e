"""Python binding of the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the product package never imports it.

Arrays are numpy: activations float64, weights float32 or bf16 carried as
uint16 bit patterns (the dtype of the array selects the widening).  Matrices
are [out][in] row-major, as documented in oracle.h.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
_lib = None


class Dims(C.Structure):
    _fields_ = [("d", C.c_int), ("n_experts", C.c_int), ("top_k", C.c_int), ("d_ff", C.c_int),
                ("n_shared", C.c_int), ("wdtype", C.c_int), ("rms_eps", C.c_double),
                ("n_heads", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("rope_theta", C.c_double)]


class Layer(C.Structure):
    _fields_ = [("g1", C.c_void_p), ("wq", C.c_void_p), ("wk", C.c_void_p), ("wv", C.c_void_p),
                ("wo", C.c_void_p), ("g2", C.c_void_p), ("wr", C.c_void_p),
                ("br", C.POINTER(C.c_float)),
                ("w_gate", C.POINTER(C.c_void_p)), ("w_up", C.POINTER(C.c_void_p)),
                ("w_down", C.POINTER(C.c_void_p)),
                ("s_gate", C.POINTER(C.c_void_p)), ("s_up", C.POINTER(C.c_void_p)),
                ("s_down", C.POINTER(C.c_void_p))]


class KV(C.Structure):
    _fields_ = [("n_seq", C.c_int), ("capacity", C.c_int),
                ("k", C.POINTER(C.c_uint16)), ("v", C.POINTER(C.c_uint16))]


def lib():
    """Load liboracle.so, building it first if it is not there."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", _build.OUT)
        if path == _build.OUT and not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        dp = C.POINTER(C.c_double)
        ip = C.POINTER(C.c_int)
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_double_to_bf16.restype = C.c_uint16
        L.orc_double_to_bf16.argtypes = [C.c_double]
        L.orc_rmsnorm.argtypes = [C.c_int, dp, C.c_void_p, C.c_int, C.c_double, dp]
        L.orc_matvec.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_int, dp, dp]
        L.orc_silu.restype = C.c_double
        L.orc_silu.argtypes = [C.c_double]
        L.orc_softmax.argtypes = [C.c_int, dp, dp]
        L.orc_topk.argtypes = [C.c_int, C.c_int, dp, ip, ip, dp]
        L.orc_expert.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, dp, dp]
        L.orc_rope.argtypes = [C.c_int, C.c_double, C.c_int, dp]
        L.orc_attn_block.argtypes = [C.POINTER(Dims), C.POINTER(Layer), C.c_int, C.c_int,
                                     C.POINTER(C.c_int32), C.POINTER(KV), dp, dp]
        L.orc_route.argtypes = [C.POINTER(Dims), C.POINTER(Layer), C.c_int, dp, ip, dp, ip, dp, dp]
        L.orc_moe_block.argtypes = [C.POINTER(Dims), C.POINTER(Layer), C.c_int, dp, ip, dp, dp]
        L.orc_forward.argtypes = [C.POINTER(Dims), C.c_int, C.POINTER(Layer), C.c_int, C.c_int,
                                  C.POINTER(C.c_int32), C.POINTER(KV), C.POINTER(C.c_float),
                                  C.POINTER(C.c_float), dp, ip, dp, dp]
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_mla_attention.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double,
                                        dp, C.POINTER(C.c_uint16), C.POINTER(C.c_int32), dp]
        for f in ("orc_attn_block", "orc_route", "orc_moe_block", "orc_forward", "orc_num_threads",
                  "orc_set_threads", "orc_mla_attention"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------- helpers
def _dtype_of(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"weights must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _dp(a):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _ip(a):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(C.POINTER(C.c_int))


def _vp(a):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return C.c_void_p(a.ctypes.data)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops from now on (results do not
    depend on it); returns the count in effect."""
    return lib().orc_set_threads(int(n))


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def double_to_bf16(x: float) -> int:
    return lib().orc_double_to_bf16(float(x))


def rmsnorm(x, g, eps):
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g)
    out = np.empty_like(x)
    lib().orc_rmsnorm(x.size, _dp(x), _vp(g), _dtype_of(g), eps, _dp(out))
    return out


def matvec(w, x):
    w = np.ascontiguousarray(w)
    x = np.ascontiguousarray(x, dtype=np.float64)
    n_out, n_in = w.shape
    assert x.size == n_in
    y = np.empty(n_out, dtype=np.float64)
    lib().orc_matvec(n_out, n_in, _vp(w), _dtype_of(w), _dp(x), _dp(y))
    return y


def silu(u):
    return lib().orc_silu(float(u))


def softmax(z):
    z = np.ascontiguousarray(z, dtype=np.float64)
    p = np.empty_like(z)
    lib().orc_softmax(z.size, _dp(z), _dp(p))
    return p


def topk(p, k, forced=None):
    p = np.ascontiguousarray(p, dtype=np.float64)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    f = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    lib().orc_topk(p.size, k, _dp(p), None if f is None else _ip(f), _ip(ids), _dp(w))
    return ids, w


def expert(wg, wu, wd, x):
    wg, wu, wd = (np.ascontiguousarray(a) for a in (wg, wu, wd))
    F, d = wg.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(d, dtype=np.float64)
    lib().orc_expert(d, F, _vp(wg), _vp(wu), _vp(wd), _dtype_of(wg), _dp(x), _dp(y))
    return y


def rope(x, pos, theta):
    x = np.array(x, dtype=np.float64, copy=True)
    lib().orc_rope(x.size, theta, int(pos), _dp(x))
    return x


# ---------------------------------------------------------------- stacks
class OracleLayer:
    """Holds the numpy arrays of one layer and the ctypes struct pointing at them.

    Any expert entry may be None (e.g. experts not selected in a large run);
    the oracle returns ORC_EPTR if it needs one that is missing."""

    def __init__(self, g2, wr, br, w_gate, w_up, w_down, s_gate=(), s_up=(), s_down=(),
                 g1=None, wq=None, wk=None, wv=None, wo=None):
        self.arrays = dict(g1=g1, wq=wq, wk=wk, wv=wv, wo=wo, g2=g2, wr=wr, br=br)
        self.w_gate, self.w_up, self.w_down = list(w_gate), list(w_up), list(w_down)
        self.s_gate, self.s_up, self.s_down = list(s_gate), list(s_up), list(s_down)
        for a in (g1, wq, wk, wv, wo, g2, wr):
            if a is not None:
                assert a.flags.c_contiguous
        if br is not None:
            assert br.dtype == np.float32
        self._refresh()

    def _ptrarr(self, lst):
        arr = (C.c_void_p * max(1, len(lst)))()
        for i, a in enumerate(lst):
            arr[i] = None if a is None else np.ascontiguousarray(a).ctypes.data
        return arr

    def _refresh(self):
        a = self.arrays
        self._pg, self._pu, self._pd = (self._ptrarr(x) for x in (self.w_gate, self.w_up, self.w_down))
        self._sg, self._su, self._sd = (self._ptrarr(x) for x in (self.s_gate, self.s_up, self.s_down))
        br = a["br"]
        self.struct = Layer(_vp(a["g1"]), _vp(a["wq"]), _vp(a["wk"]), _vp(a["wv"]), _vp(a["wo"]),
                            _vp(a["g2"]), _vp(a["wr"]),
                            None if br is None else br.ctypes.data_as(C.POINTER(C.c_float)),
                            C.cast(self._pg, C.POINTER(C.c_void_p)), C.cast(self._pu, C.POINTER(C.c_void_p)),
                            C.cast(self._pd, C.POINTER(C.c_void_p)),
                            C.cast(self._sg, C.POINTER(C.c_void_p)), C.cast(self._su, C.POINTER(C.c_void_p)),
                            C.cast(self._sd, C.POINTER(C.c_void_p)))

    def set_experts(self, w_gate, w_up, w_down):
        self.w_gate, self.w_up, self.w_down = list(w_gate), list(w_up), list(w_down)
        self._refresh()


class OracleKV:
    """Per-layer bf16 KV cache [n_seq][G][capacity][hd] as uint16 bits."""

    def __init__(self, k, v):
        assert k.dtype == np.uint16 and v.dtype == np.uint16 and k.shape == v.shape
        self.k = np.ascontiguousarray(k)
        self.v = np.ascontiguousarray(v)
        self.struct = KV(k.shape[0], k.shape[2], self.k.ctypes.data_as(C.POINTER(C.c_uint16)),
                         self.v.ctypes.data_as(C.POINTER(C.c_uint16)))


def make_dims(d, n_experts, top_k, d_ff, n_shared, wdtype, rms_eps=1e-6, n_heads=0, n_kv_heads=0,
              head_dim=0, rope_theta=1e6):
    return Dims(d, n_experts, top_k, d_ff, n_shared, wdtype, rms_eps, n_heads, n_kv_heads, head_dim,
                rope_theta)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def attn_block(dims, layer, h, positions, kv, rows_per_seq=1):
    h = np.ascontiguousarray(h, dtype=np.float64)
    M = h.shape[0]
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    out = np.empty_like(h)
    _check(lib().orc_attn_block(C.byref(dims), C.byref(layer.struct), M, rows_per_seq,
                                pos.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(kv.struct), _dp(h),
                                _dp(out)), "attn_block")
    return out


def route(dims, layer, h, forced=None):
    h = np.ascontiguousarray(h, dtype=np.float64)
    M = h.shape[0]
    E, k = dims.n_experts, dims.top_k
    logits = np.empty((M, E), dtype=np.float64)
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float64)
    margin = np.empty(M, dtype=np.float64)
    f = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    _check(lib().orc_route(C.byref(dims), C.byref(layer.struct), M, _dp(h), None if f is None else _ip(f),
                           _dp(logits), _ip(ids), _dp(w), _dp(margin)), "route")
    return logits, ids, w, margin


def moe_block(dims, layer, h, ids, w):
    h = np.ascontiguousarray(h, dtype=np.float64)
    out = np.empty_like(h)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    _check(lib().orc_moe_block(C.byref(dims), C.byref(layer.struct), h.shape[0], _dp(h), _ip(ids), _dp(w),
                               _dp(out)), "moe_block")
    return out


def forward(dims, layers, hidden_in, positions=None, kvs=None, rows_per_seq=1):
    """Whole step; returns (hidden_out fp32, trace dict)."""
    hin = np.ascontiguousarray(hidden_in, dtype=np.float32)
    M, d = hin.shape
    L = len(layers)
    E, k = dims.n_experts, dims.top_k
    arr = (Layer * max(1, L))(*[ly.struct for ly in layers])
    if kvs is not None:
        kvarr = (KV * max(1, L))(*[kv.struct for kv in kvs])
        kvp = C.cast(kvarr, C.POINTER(KV))
    else:
        kvp = None
    pos = np.zeros(M, dtype=np.int32) if positions is None else np.ascontiguousarray(positions, dtype=np.int32)
    out = np.empty_like(hin)
    logits = np.empty((L, M, E), dtype=np.float64)
    ids = np.empty((L, M, k), dtype=np.int32)
    w = np.empty((L, M, k), dtype=np.float64)
    margin = np.empty((L, M), dtype=np.float64)
    _check(lib().orc_forward(C.byref(dims), L, C.cast(arr, C.POINTER(Layer)), M, rows_per_seq,
                             pos.ctypes.data_as(C.POINTER(C.c_int32)), kvp,
                             hin.ctypes.data_as(C.POINTER(C.c_float)), out.ctypes.data_as(C.POINTER(C.c_float)),
                             _dp(logits), _ip(ids), _dp(w), _dp(margin)), "forward")
    return out, dict(logits=logits, ids=ids, w=w, margin=margin)


def mla_attention(q, cache, positions, latent_dim, scale, rows_per_seq=1):
    """MLA attention at decode over a latent cache (orc_mla_attention):
    q [M][H][Dc + Dr] (float64), cache [n_seq][capacity][Dc + Dr] bf16 bits
    (uint16), positions [M]; returns out [M][H][Dc] float64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    cache = np.ascontiguousarray(cache, dtype=np.uint16)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    M, H, Dk = q.shape
    n_seq, cap, Dk2 = cache.shape
    if Dk2 != Dk or not 0 < latent_dim <= Dk:
        raise ValueError("q and cache rows differ in width, or latent_dim is out of range")
    out = np.empty((M, H, latent_dim), dtype=np.float64)
    _check(lib().orc_mla_attention(M, rows_per_seq, H, latent_dim, Dk - latent_dim, n_seq, cap, float(scale), _dp(q),
                                   cache.ctypes.data_as(C.POINTER(C.c_uint16)),
                                   pos.ctypes.data_as(C.POINTER(C.c_int32)), _dp(out)), "mla_attention")
    return out
