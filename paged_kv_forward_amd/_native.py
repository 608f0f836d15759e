"""ctypes binding of include/pie.h: the same names, argument marshalling only.

Loading fails loudly when libpie.so has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_double, c_float, c_int, c_int32, c_int64,
                    c_size_t, c_uint32, c_uint64, c_void_p)

HERE = os.path.dirname(os.path.abspath(__file__))
# PIE_LIBRARY may name another build of the same library (the sanitized
# host build of the CPU tests); there is no fallback of any kind.
LIB_PATH = os.environ.get("PIE_LIBRARY") or os.path.join(HERE, "libpie.so")

PIE_OK, PIE_EINVAL, PIE_ENOMEM, PIE_EHIP, PIE_ESTATE = 0, -1, -2, -3, -4
PIE_KV_BF16, PIE_KV_E4M3 = 0, 1
PIE_EPI_ARGMAX, PIE_EPI_GUMBEL_MAX = 0, 1
PIE_FLAG_NO_LAUNCH, PIE_FLAG_LOGITS_DEVICE, PIE_FLAG_SYNC_DEBUG = 1, 2, 4
KERNEL_CLASSES = ["embed", "gemm_qkv", "attn_decode", "attn_prefill", "gemm_o", "gemm_gateup",
                  "gemm_down", "lm_head"]
PIE_K_NUM_CLASSES = len(KERNEL_CLASSES)

EXPORTS = ["pie_kv_page_bytes", "pie_workspace_bytes", "pie_init", "pie_destroy",
           "pie_alloc_working_set", "pie_fork", "pie_free_working_set", "pie_truncate",
           "pie_ws_info", "pie_pool_stats_get", "pie_forward", "pie_last_error",
           "pie_profile_enable", "pie_profile_repeat", "pie_profile_read", "pie_debug_plan", "pie_debug_philox",
           "pie_packed_weight_bytes", "pie_pack_weight", "pie_decode_async", "pie_sync", "pie_prefix_lookup",
           "pie_packed_weight_fp8_bytes", "pie_fp8_scale_count", "pie_pack_weight_fp8", "pie_attach_fp8_weights",
           "pie_forward_static"]
PIE_STATIC_SCRATCH_BYTES = 96 * 1024 * 1024


class pie_model_desc(Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("d_ffn", c_int32),
                ("vocab", c_int32), ("rms_eps", c_float), ("rope_theta", c_float),
                ("kv_dtype", c_int32), ("page_size", c_int32)]


class pie_weights(Structure):
    _fields_ = [("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("attn_norm", POINTER(c_void_p)), ("wq", POINTER(c_void_p)),
                ("wk", POINTER(c_void_p)), ("wv", POINTER(c_void_p)), ("wo", POINTER(c_void_p)),
                ("mlp_norm", POINTER(c_void_p)), ("w_gate", POINTER(c_void_p)),
                ("w_up", POINTER(c_void_p)), ("w_down", POINTER(c_void_p)),
                ("kv_scale", c_void_p)]


class pie_fp8_weights(Structure):
    _fields_ = [(nm, POINTER(c_void_p)) for nm in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
                                                  "sq", "sk", "sv", "so", "s_gate", "s_up", "s_down")] + [
        ("lm_head", c_void_p), ("s_lm_head", c_void_p)]


class pie_limits(Structure):
    _fields_ = [("max_rows", c_int32), ("max_seqs", c_int32), ("max_readout", c_int32),
                ("max_ctx", c_int32)]


class pie_ws_stats(Structure):
    _fields_ = [("len", c_int32), ("frozen_len", c_int32), ("n_pages", c_int32)]


class pie_pool_stats(Structure):
    _fields_ = [("pages_total", c_int64), ("pages_free", c_int64),
                ("pages_ever_allocated", c_int64), ("kv_bytes_copied", c_int64)]


class pie_epilogue(Structure):
    _fields_ = [("kind", c_int32), ("temperature", c_float), ("seed", c_uint64)]


class pie_pass(Structure):
    _fields_ = [("ws", c_uint64), ("tokens", POINTER(c_int32)), ("positions", POINTER(c_int32)),
                ("n_tokens", c_int32), ("readout", POINTER(c_int32)), ("n_readout", c_int32),
                ("epi", POINTER(pie_epilogue)), ("commit", c_int32)]


class pie_plan_view(Structure):
    _fields_ = [("n_rows", c_int32), ("n_seqs", c_int32), ("n_readout", c_int32),
                ("n_page_entries", c_int32)] + [
        (nm, POINTER(c_int32)) for nm in ("tok", "pos", "row_seq", "slot", "seq_row0", "seq_ctx",
                                          "seq_len", "seq_pg0", "pg_id", "pg_valid", "pg_start",
                                          "ro_row", "ro_lane")]


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpie.so is not built: run `python -m paged_kv_forward_amd.build` "
                          "(hipcc, gfx950) first; there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = POINTER
    sig = {
        "pie_kv_page_bytes": (c_size_t, [P(pie_model_desc)]),
        "pie_workspace_bytes": (c_size_t, [P(pie_model_desc), P(pie_limits)]),
        "pie_init": (c_int, [P(pie_model_desc), P(pie_weights), c_void_p, c_size_t, c_void_p,
                             c_size_t, P(pie_limits), c_void_p, P(c_void_p)]),
        "pie_destroy": (c_int, [c_void_p]),
        "pie_alloc_working_set": (c_int, [c_void_p, P(c_uint64)]),
        "pie_fork": (c_int, [c_void_p, c_uint64, P(c_uint64)]),
        "pie_free_working_set": (c_int, [c_void_p, c_uint64]),
        "pie_truncate": (c_int, [c_void_p, c_uint64, c_int32]),
        "pie_ws_info": (c_int, [c_void_p, c_uint64, P(pie_ws_stats), P(c_int32)]),
        "pie_pool_stats_get": (c_int, [c_void_p, P(pie_pool_stats)]),
        "pie_forward": (c_int, [c_void_p, P(pie_pass), c_int32, P(c_int32), c_void_p, c_int32]),
        "pie_forward_static": (c_int, [c_void_p, P(pie_pass), c_int32, P(c_int32), c_void_p, c_int32]),
        "pie_last_error": (c_char_p, []),
        "pie_profile_enable": (c_int, [c_void_p, c_uint32]),
        "pie_profile_repeat": (c_int, [c_void_p, c_int32]),
        "pie_profile_read": (c_int, [c_void_p, P(c_double), P(c_int64)]),
        "pie_debug_plan": (c_int, [c_void_p, P(pie_plan_view)]),
        "pie_debug_philox": (c_int, [c_void_p, c_uint64, c_uint32, c_uint32, c_int32, c_void_p]),
        "pie_packed_weight_bytes": (c_size_t, [c_int32, c_int32]),
        "pie_pack_weight": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
        "pie_decode_async": (c_int, [c_void_p, P(c_uint64), c_int32, c_void_p, c_void_p, P(pie_epilogue),
                                     c_void_p]),
        "pie_sync": (c_int, [c_void_p]),
        "pie_prefix_lookup": (c_int, [c_void_p, P(c_int32), c_int32, P(c_uint64), P(c_int32)]),
        "pie_packed_weight_fp8_bytes": (c_size_t, [c_int32, c_int32]),
        "pie_fp8_scale_count": (c_size_t, [c_int32, c_int32]),
        "pie_pack_weight_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
        "pie_attach_fp8_weights": (c_int, [c_void_p, P(pie_fp8_weights)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


class PieError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d)" % (msg, code))
        self.code = code


def check(rc: int) -> None:
    if rc != PIE_OK:
        raise PieError(rc, lib().pie_last_error().decode(errors="replace"))


def _fn(name):
    def call(*args):
        return getattr(lib(), name)(*args)
    call.__name__ = name
    return call


# The C ABI under its own names.
for _n in EXPORTS:
    globals()[_n] = _fn(_n)
