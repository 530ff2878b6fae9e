"""MI355X (gfx950) MoE decode megakernel: one persistent HIP kernel per decode
step through a deep stack of MoE transformer layers.

The Python surface is a thin ctypes binding of include/mk.h (and of
include/mk_mla.h in the mla module); every step of the decode path runs in the
HIP kernels of libmk.so.
"""
from ._lib import (EXPORTS, NOALLOC_SCRATCH_BYTES, MK_BF16, MK_ERR_DEVICE, MK_ERR_HIP, MK_ERR_INVALID_ARG, MK_ERR_TIMEOUT,
                   MK_ERR_UNSUPPORTED, MK_F32, MK_OK, MkError, lib, mk_config, mk_create, mk_decode_step,
                   mk_decode_step_noalloc, mk_decode_step_phased, mk_destroy, mk_get_info, mk_info, mk_kv_cache, mk_last_error, mk_layer_weights, mk_set_timing, mk_set_trace,
                   mk_set_watchdog, mk_strerror, mk_sync)

__all__ = ["EXPORTS", "NOALLOC_SCRATCH_BYTES", "MK_BF16", "MK_ERR_DEVICE", "MK_ERR_HIP", "MK_ERR_INVALID_ARG", "MK_ERR_TIMEOUT",
           "MK_ERR_UNSUPPORTED", "MK_F32", "MK_OK", "MkError", "lib", "mk_config", "mk_create", "mk_decode_step",
           "mk_decode_step_noalloc", "mk_decode_step_phased", "mk_destroy", "mk_get_info", "mk_info", "mk_kv_cache", "mk_last_error", "mk_layer_weights",
           "mk_set_timing", "mk_set_trace", "mk_set_watchdog", "mk_strerror", "mk_sync"]
