"""The C ABI on the CPU: the library loads, exports every function that
include/mk.h and include/mk_mla.h declare, and rejects bad arguments before
touching a device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mk():
    import moe_layer_stack_amd as mk
    from moe_layer_stack_amd import build
    if not os.path.exists(os.path.join(ROOT, "moe_layer_stack_amd", "libmk.so")):
        build.build()
    mk.lib()
    return mk


def declared(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(mk_[a-z_]+|synth_[a-z0-9_]+)\s*\(", src))


def test_every_declared_function_is_exported(mk):
    names = declared("mk.h")
    assert {"mk_create", "mk_decode_step", "mk_destroy"} <= names
    L = C.CDLL(os.path.join(ROOT, "moe_layer_stack_amd", "libmk.so"))
    for n in names:
        assert hasattr(L, n), n
    assert set(mk.EXPORTS) == names


def test_every_declared_mla_function_is_exported(mk):
    from moe_layer_stack_amd import mla
    names = declared("mk_mla.h")
    assert {"mk_mla_create", "mk_mla_attention", "mk_mla_destroy"} <= names
    L = C.CDLL(os.path.join(ROOT, "moe_layer_stack_amd", "libmk.so"))
    for n in names:
        assert hasattr(L, n), n
    assert set(mla.MLA_EXPORTS) == names
    # mk_mla_config: 7 int32 + 1 float; mk_mla_info: 2 int32 + 1 int64
    assert C.sizeof(mla.mk_mla_config) == 32
    assert C.sizeof(mla.mk_mla_info) == 16


def test_mla_create_rejects_bad_configs_before_the_device(mk):
    from moe_layer_stack_amd import mla
    L = mla.lib()
    h = C.c_void_p()
    assert L.mk_mla_create(None, C.byref(h)) == mk.MK_ERR_INVALID_ARG
    good = dict(n_heads=64, latent_dim=512, rope_dim=64, rows=8, rows_per_seq=1, n_seq=8, capacity=4160, scale=0.072)
    for bad, want in ((dict(rows=0), mk.MK_ERR_INVALID_ARG), (dict(rows_per_seq=3), mk.MK_ERR_INVALID_ARG),
                      (dict(n_seq=4), mk.MK_ERR_INVALID_ARG), (dict(scale=0.0), mk.MK_ERR_INVALID_ARG),
                      (dict(scale=float("nan")), mk.MK_ERR_INVALID_ARG), (dict(latent_dim=256), mk.MK_ERR_UNSUPPORTED),
                      (dict(rope_dim=32), mk.MK_ERR_UNSUPPORTED), (dict(n_heads=8), mk.MK_ERR_UNSUPPORTED),
                      (dict(n_heads=256), mk.MK_ERR_UNSUPPORTED), (dict(rows=72, n_seq=72), mk.MK_ERR_UNSUPPORTED),
                      (dict(capacity=(1 << 21) + 1), mk.MK_ERR_UNSUPPORTED)):
        cfg = mla.mk_mla_config(**{**good, **bad})
        assert L.mk_mla_create(C.byref(cfg), C.byref(h)) == want, bad
        assert h.value is None
    assert L.mk_mla_destroy(None) == mk.MK_OK


def test_synth_exports(syn):
    L = C.CDLL(syn.LIB)
    for n in declared("synth.h"):
        assert hasattr(L, n), n


def test_struct_sizes_match_header(mk):
    # mk_config: 17 x 4-byte fields; mk_layer_weights: 14 pointers; mk_kv_cache: 2 pointers + 2 ints
    assert C.sizeof(mk.mk_config) == 17 * 4
    assert C.sizeof(mk.mk_layer_weights) == 14 * 8
    assert C.sizeof(mk.mk_kv_cache) == 24
    assert C.sizeof(mk.mk_info) == 24 + 8


def test_strerror(mk):
    assert mk.mk_strerror(mk.MK_OK) == "success"
    assert "timed out" in mk.mk_strerror(mk.MK_ERR_TIMEOUT)
    assert mk.mk_strerror(-99) == "unknown status"


def _cfg(mk, **kw):
    c = dict(n_layers=2, d_model=256, n_experts=8, top_k=2, n_shared=0, d_ff=512, dtype=mk.MK_F32,
             has_router_bias=0, rms_eps=1e-6, has_attn=0, n_heads=0, n_kv_heads=0, head_dim=0, rope_theta=1e6,
             rows=1, rows_per_seq=1, kv_capacity=0)
    c.update(kw)
    return mk.mk_config(**c)


def _layers(n):
    from moe_layer_stack_amd import mk_layer_weights
    fake = 0x1000
    return [mk_layer_weights(None, None, None, None, None, fake, fake, None, fake, fake, fake, None, None, None)
            for _ in range(n)]


@pytest.mark.parametrize("kw,status", [
    (dict(n_layers=0), -1),
    (dict(dtype=7), -2),
    (dict(d_model=300), -2),           # row not 1/2/4/8 KiB
    (dict(d_ff=100), -2),
    (dict(n_experts=65), -2),
    (dict(top_k=9, n_experts=16), -2),
    (dict(top_k=3, n_experts=2), -2),
    (dict(n_shared=5), -2),
    (dict(rms_eps=0.0), -1),
    (dict(rows=9), -2),                # above 8 rows: a multiple of 8
    (dict(rows=65), -2),
    (dict(rows=16, rows_per_seq=16), -2),  # a launch of 8 rows must hold whole sequences
    (dict(rows=4, rows_per_seq=3), -1),
    (dict(has_attn=1, n_heads=3, n_kv_heads=2, head_dim=128, d_model=256, kv_capacity=16), -1),
    (dict(has_attn=1, n_heads=2, n_kv_heads=1, head_dim=64, kv_capacity=16), -2),
    (dict(dtype=1, d_model=512, d_ff=1024), -2),   # bf16 rows below 2 KiB
    (dict(dtype=1, d_model=1024, d_ff=512), -2),
])
def test_create_rejects_bad_config(mk, kw, status):
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk, **kw), _layers(max(1, kw.get("n_layers", 2))))
    assert ei.value.status == status, str(ei.value)


def test_create_rejects_too_many_queries_per_kv_head(mk):
    # 8 verify rows of one sequence with 8 query heads per kv head: 64 query
    # vectors per (sequence, kv head), above the 32 an attention task set holds
    kw = dict(dtype=1, d_model=1024, d_ff=1024, has_attn=1, n_heads=32, n_kv_heads=4, head_dim=128,
              rows=8, rows_per_seq=8, kv_capacity=64)
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk, **kw), _layers(2))
    assert ei.value.status == -2 and "rows_per_seq * n_heads / n_kv_heads" in mk.mk_last_error()
    # the same with 4 rows per sequence (32 queries) passes validation and
    # stops at the next check, the (absent) attention weights of the stand-in layers
    kw.update(rows_per_seq=4)
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk, **kw), _layers(2))
    assert ei.value.status == mk.MK_ERR_INVALID_ARG and "attention weight pointer" in mk.mk_last_error()


def test_create_rejects_fp32_wide_query_groups(mk):
    kw = dict(dtype=0, d_model=1024, d_ff=512, has_attn=1, n_heads=16, n_kv_heads=2, head_dim=128,
              kv_capacity=64)
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk, **kw), _layers(2))
    assert ei.value.status == -2 and "fp32" in mk.mk_last_error()


def test_create_rejects_null_weights(mk):
    from moe_layer_stack_amd import mk_layer_weights
    lw = [mk_layer_weights() for _ in range(2)]
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk), lw)
    assert ei.value.status == mk.MK_ERR_INVALID_ARG and "NULL" in mk.mk_last_error()


def test_create_requires_bias_when_configured(mk):
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk, has_router_bias=1), _layers(2))
    assert ei.value.status == mk.MK_ERR_INVALID_ARG and "b_router" in mk.mk_last_error()


def test_decode_step_rejects_null_handle(mk):
    with pytest.raises(mk.MkError) as ei:
        mk.mk_decode_step(None, 0x1000, 0x2000, None, 0x3000)
    assert ei.value.status == mk.MK_ERR_INVALID_ARG


def test_destroy_accepts_null(mk):
    assert mk.mk_destroy(None) == mk.MK_OK


def test_create_without_gpu_reports_device(mk):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(mk.MkError) as ei:
        mk.mk_create(_cfg(mk), _layers(2))
    assert ei.value.status == mk.MK_ERR_DEVICE
