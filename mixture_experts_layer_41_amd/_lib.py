"""ctypes view of libmoe_mi355x.so (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_SWIGLU = 0, 1
MOE_WEIGHTS_ACT, MOE_WEIGHTS_INT8 = 0, 1

# every symbol include/moe.h declares
EXPORTS = ("moe_status_string", "moe_route", "moe_permute", "moe_expert_ffn",
           "moe_expert_ffn_int8", "moe_combine", "moe_aux_stats", "moe_forward",
           "moe_forward_static", "moe_forward_train", "moe_backward")
MOE_STATIC_SCRATCH_BYTES = 64 << 20


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("d_ffn", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("add_residual", ctypes.c_int32),
        ("weight_format", ctypes.c_int32),
        ("router_temperature", ctypes.c_float),
    ]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "router_bias", "w1", "b1", "w2", "b2",
        "shared_w1", "shared_b1", "shared_w2", "shared_b2",
        "w1_scale", "w2_scale", "shared_w1_scale", "shared_w2_scale")]


class MoeAux(ctypes.Structure):
    _fields_ = [
        ("load_balance", ctypes.c_double),
        ("z_loss", ctypes.c_double),
        ("weighted", ctypes.c_double),
        ("n_dropped", ctypes.c_int64),
        ("capacity", ctypes.c_int64),
        ("n_kept", ctypes.c_int64),
        ("lb_squares", ctypes.c_double),
        ("kl_uniform", ctypes.c_double),
        ("freq_penalty", ctypes.c_double),
    ]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "scores", "token_lse", "topk_idx", "topk_w", "expert_counts", "expert_offsets",
        "perm_token", "inv_row", "y_perm", "preact", "shared_preact")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dw_router", "drouter_bias", "dw1", "db1", "dw2", "db2", "dws1", "dsb1", "dws2",
        "dsb2")]


class MoeLossWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in ("load_balance", "z_loss", "lb_squares", "kl_uniform")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)
    cfgp = ctypes.POINTER(MoeConfig)
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    sigs = {
        "moe_route": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_expert_ffn": [cfgp, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_expert_ffn_int8": [cfgp, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine": [cfgp, vp, vp, vp, vp, vp, vp, vp],
        "moe_aux_stats": [cfgp, vp, vp, vp, ctypes.c_size_t, vp, vp],
        "moe_forward": [cfgp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_forward_static": [cfgp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp, vp, vp, vp],
        "moe_forward_train": [cfgp, ctypes.POINTER(MoeWeights), vp, vp, vp, ctypes.POINTER(MoeSaved),
                              vp, vp, sz, vp],
        "moe_backward": [cfgp, ctypes.POINTER(MoeWeights), vp, ctypes.POINTER(MoeSaved), vp,
                         ctypes.POINTER(MoeLossWeights), ctypes.POINTER(MoeGrads), vp, sz, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = L
    return L


def check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())
