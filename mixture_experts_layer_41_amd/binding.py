"""Thin Python binding of the C ABI, same names as the library's entry points.

Argument marshalling only: tensors are allocated with torch on the current
CUDA (HIP) device, their data pointers and torch's current stream are passed
to the library, and every step of the layer runs in the library's kernels.
bf16 tensors are torch.bfloat16; float32 ones torch.float32; indices int32;
INT8 weight codes torch.int8 with float32 row scales.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MoeAux, MoeConfig, MoeGrads, MoeLossWeights, MoeSaved, MoeWeights, check, lib

_TORCH_DT = {_lib.MOE_DTYPE_F32: torch.float32, _lib.MOE_DTYPE_BF16: torch.bfloat16}


def make_config(T, d, E, k, f, S=0, dtype="bf16", act="swiglu", capacity_factor=0.0,
                add_residual=False, weights="act", temperature=1.0) -> MoeConfig:
    return MoeConfig(
        n_tokens=int(T), d_model=int(d), n_experts=int(E), top_k=int(k), d_ffn=int(f),
        n_shared=int(S),
        dtype=_lib.MOE_DTYPE_BF16 if dtype == "bf16" else _lib.MOE_DTYPE_F32,
        act=_lib.MOE_ACT_SWIGLU if act == "swiglu" else _lib.MOE_ACT_GELU,
        capacity_factor=float(capacity_factor), add_residual=int(bool(add_residual)),
        weight_format=_lib.MOE_WEIGHTS_INT8 if weights == "int8" else _lib.MOE_WEIGHTS_ACT,
        router_temperature=float(temperature))


def config_of(layer) -> MoeConfig:
    """MoeConfig from any object with T, d, E, k, f, S, dtype, act,
    capacity_factor and add_residual attributes (and optionally weights:
    "act" or "int8", and router_temperature)."""
    return make_config(layer.T, layer.d, layer.E, layer.k, layer.f, layer.S, layer.dtype,
                       layer.act, layer.capacity_factor, layer.add_residual,
                       getattr(layer, "weights", "act"), getattr(layer, "router_temperature", 1.0))


def torch_dtype(cfg: MoeConfig) -> torch.dtype:
    return _TORCH_DT[cfg.dtype]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev():
    return torch.device("cuda", torch.cuda.current_device())


def _i32(*shape):
    return torch.empty(*shape, dtype=torch.int32, device=_dev())


def _f32(*shape):
    return torch.empty(*shape, dtype=torch.float32, device=_dev())


# ---------------------------------------------------------------------------


def moe_route(cfg: MoeConfig, x, w_router, router_bias=None, router_noise=None):
    """Returns (topk_idx [T,k] i32, topk_w [T,k] f32, token_lse [T] f32, route_ws)."""
    L = lib()
    T, k = cfg.n_tokens, cfg.top_k
    idx, w, lse = _i32(T, k), _f32(T, k), _f32(T)

    def q(ws, nb):
        return L.moe_route(ctypes.byref(cfg), _p(x), _p(w_router), _p(router_bias),
                           _p(router_noise), _p(idx), _p(w), _p(lse), ws, nb, _stream())
    q.__name__ = "moe_route"
    n = ctypes.c_size_t(0)
    check("moe_route", q(None, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=_dev())
    check("moe_route", q(_p(ws), ctypes.byref(n)))
    return idx, w, lse, ws


def moe_permute(cfg: MoeConfig, topk_idx, topk_w=None, x=None, want_perm_w=False,
                want_x_perm=False):
    """Returns a dict with expert_counts [E], expert_offsets [E+1],
    perm_token [T*k], perm_w [T*k] or None, inv_row [T,k], x_perm [T*k,d] or
    None, n_dropped [1] (all device tensors)."""
    L = lib()
    T, k, E = cfg.n_tokens, cfg.top_k, cfg.n_experts
    out = {
        "expert_counts": _i32(E), "expert_offsets": _i32(E + 1), "perm_token": _i32(T * k),
        "perm_w": _f32(T * k) if want_perm_w else None, "inv_row": _i32(T, k),
        "x_perm": (torch.empty(T * k, cfg.d_model, dtype=torch_dtype(cfg), device=_dev())
                   if want_x_perm else None),
        "n_dropped": _i32(1),
    }

    def call(ws, nb):
        return L.moe_permute(ctypes.byref(cfg), _p(topk_idx), _p(topk_w), _p(x),
                             _p(out["expert_counts"]), _p(out["expert_offsets"]),
                             _p(out["perm_token"]), _p(out["perm_w"]), _p(out["inv_row"]),
                             _p(out["x_perm"]), _p(out["n_dropped"]), ws, nb, _stream())
    n = ctypes.c_size_t(0)
    check("moe_permute", call(None, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=_dev())
    check("moe_permute", call(_p(ws), ctypes.byref(n)))
    return out


def moe_expert_ffn(cfg: MoeConfig, n_groups, n_seg, rows_max, a, a_rows, group_offsets, w1, b1,
                   w2, b2, out=None):
    """out [rows_max, d] = grouped expert FFN (rows outside every group untouched)."""
    L = lib()
    if out is None:
        out = torch.zeros(max(int(rows_max), 1), cfg.d_model, dtype=torch_dtype(cfg), device=_dev())

    def call(ws, nb):
        return L.moe_expert_ffn(ctypes.byref(cfg), int(n_groups), int(n_seg), int(rows_max), _p(a),
                                _p(a_rows), _p(group_offsets), _p(w1), _p(b1), _p(w2), _p(b2),
                                _p(out), ws, nb, _stream())
    n = ctypes.c_size_t(0)
    check("moe_expert_ffn", call(None, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=_dev())
    check("moe_expert_ffn", call(_p(ws), ctypes.byref(n)))
    return out


def moe_expert_ffn_int8(cfg: MoeConfig, n_groups, n_seg, rows_max, a, a_rows, group_offsets, w1,
                        w1_scale, b1, w2, w2_scale, b2, out=None):
    """moe_expert_ffn with INT8 weight codes (torch.int8) and float32 row
    scales."""
    L = lib()
    if out is None:
        out = torch.zeros(max(int(rows_max), 1), cfg.d_model, dtype=torch_dtype(cfg), device=_dev())

    def call(ws, nb):
        return L.moe_expert_ffn_int8(ctypes.byref(cfg), int(n_groups), int(n_seg), int(rows_max),
                                     _p(a), _p(a_rows), _p(group_offsets), _p(w1), _p(w1_scale),
                                     _p(b1), _p(w2), _p(w2_scale), _p(b2), _p(out), ws, nb,
                                     _stream())
    n = ctypes.c_size_t(0)
    check("moe_expert_ffn_int8", call(None, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=_dev())
    check("moe_expert_ffn_int8", call(_p(ws), ctypes.byref(n)))
    return out


class ExpertFFN:
    """A prepared moe_expert_ffn (or, with w1_scale / w2_scale, INT8
    moe_expert_ffn_int8) call: workspace and output allocated once, so
    repeated calls allocate nothing and cost one library call each."""

    def __init__(self, cfg: MoeConfig, n_groups, n_seg, rows_max, a, a_rows, group_offsets, w1, b1,
                 w2, b2, out=None, w1_scale=None, w2_scale=None):
        self.cfg = cfg
        self.q8 = w1_scale is not None
        self.out = out if out is not None else torch.empty(
            max(int(rows_max), 1), cfg.d_model, dtype=torch_dtype(cfg), device=_dev())
        self._keep = (a, a_rows, group_offsets, w1, b1, w2, b2, w1_scale, w2_scale)
        if self.q8:
            self._head = (int(n_groups), int(n_seg), int(rows_max), _p(a), _p(a_rows),
                          _p(group_offsets), _p(w1), _p(w1_scale), _p(b1), _p(w2), _p(w2_scale),
                          _p(b2), _p(self.out))
            self._fn = lib().moe_expert_ffn_int8
        else:
            self._head = (int(n_groups), int(n_seg), int(rows_max), _p(a), _p(a_rows),
                          _p(group_offsets), _p(w1), _p(b1), _p(w2), _p(b2), _p(self.out))
            self._fn = lib().moe_expert_ffn
        n = ctypes.c_size_t(0)
        check(self._fn.__name__, self._fn(ctypes.byref(cfg), *self._head, None, ctypes.byref(n), None))
        self.ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=_dev())
        self._n = ctypes.c_size_t(self.ws.numel())
        self._ws = _p(self.ws)

    def __call__(self):
        self._n.value = self.ws.numel()
        check(self._fn.__name__, self._fn(ctypes.byref(self.cfg), *self._head, self._ws,
                                          ctypes.byref(self._n), _stream()))
        return self.out


def moe_combine(cfg: MoeConfig, y_perm, inv_row, topk_w, shared_y=None, residual=None, y=None):
    L = lib()
    if y is None:
        y = torch.empty(cfg.n_tokens, cfg.d_model, dtype=torch_dtype(cfg), device=_dev())
    check("moe_combine", L.moe_combine(ctypes.byref(cfg), _p(y_perm), _p(inv_row), _p(topk_w),
                                       _p(shared_y), _p(residual), _p(y), _stream()))
    return y


def aux_to_dict(t: torch.Tensor) -> dict:
    """Decode a device moe_aux record (uint8 tensor) after a synchronise."""
    raw = bytes(t.cpu().numpy().tobytes())
    a = MoeAux.from_buffer_copy(raw[:ctypes.sizeof(MoeAux)])
    return {f: getattr(a, f) for f, _ in MoeAux._fields_}


def new_aux() -> torch.Tensor:
    return torch.zeros(ctypes.sizeof(MoeAux), dtype=torch.uint8, device=_dev())


def moe_aux_stats(cfg: MoeConfig, expert_counts, n_dropped, route_ws, aux=None):
    L = lib()
    aux = new_aux() if aux is None else aux
    check("moe_aux_stats", L.moe_aux_stats(ctypes.byref(cfg), _p(expert_counts), _p(n_dropped),
                                           _p(route_ws), route_ws.numel(), _p(aux), _stream()))
    return aux


@dataclass
class LayerWeights:
    """Device tensors of one layer (None where absent)."""
    w_router: torch.Tensor
    w1: torch.Tensor
    w2: torch.Tensor
    router_bias: torch.Tensor | None = None
    b1: torch.Tensor | None = None
    b2: torch.Tensor | None = None
    shared_w1: torch.Tensor | None = None
    shared_b1: torch.Tensor | None = None
    shared_w2: torch.Tensor | None = None
    shared_b2: torch.Tensor | None = None
    # INT8 expert weights: float32 row scales of w1 / w2 / shared_w1 / shared_w2
    w1_scale: torch.Tensor | None = None
    w2_scale: torch.Tensor | None = None
    shared_w1_scale: torch.Tensor | None = None
    shared_w2_scale: torch.Tensor | None = None

    def c_struct(self) -> MoeWeights:
        return MoeWeights(**{n: (None if getattr(self, n) is None else getattr(self, n).data_ptr())
                             for n, _ in MoeWeights._fields_})


class Forward:
    """A prepared moe_forward call: workspace and outputs allocated once, so
    repeated calls (and HIP graph capture) allocate nothing."""

    def __init__(self, cfg: MoeConfig, weights: LayerWeights, want_routing=True, want_aux=True):
        self.cfg = cfg
        self.weights = weights
        self._w = weights.c_struct()
        T, k, E = cfg.n_tokens, cfg.top_k, cfg.n_experts
        self.y = torch.empty(T, cfg.d_model, dtype=torch_dtype(cfg), device=_dev())
        self.topk_idx = _i32(T, k) if want_routing else None
        self.topk_w = _f32(T, k) if want_routing else None
        self.expert_counts = _i32(E) if want_routing else None
        self.aux = new_aux() if want_aux else None
        n = ctypes.c_size_t(0)
        check("moe_forward", lib().moe_forward(ctypes.byref(cfg), ctypes.byref(self._w), None, None,
                                               None, None, None, None, None, None, ctypes.byref(n),
                                               None))
        self.ws_bytes = int(n.value)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=_dev())

    def __call__(self, x, router_noise=None):
        n = ctypes.c_size_t(self.ws.numel())
        check("moe_forward", lib().moe_forward(
            ctypes.byref(self.cfg), ctypes.byref(self._w), _p(x), _p(router_noise), _p(self.y),
            _p(self.topk_idx),
            _p(self.topk_w), _p(self.expert_counts), _p(self.aux), _p(self.ws), ctypes.byref(n),
            _stream()))
        return self.y


def moe_forward_static(cfg: MoeConfig, weights: LayerWeights, x, router_noise=None, y=None,
                       topk_idx=None, topk_w=None, expert_counts=None, aux=None):
    """moe_forward without a workspace (the library's static scratch array).
    Output tensors may be passed in (then nothing is allocated here either);
    returns (y, topk_idx, topk_w, expert_counts, aux)."""
    T, k, E = cfg.n_tokens, cfg.top_k, cfg.n_experts
    y = torch.empty(T, cfg.d_model, dtype=torch_dtype(cfg), device=_dev()) if y is None else y
    topk_idx = _i32(T, k) if topk_idx is None else topk_idx
    topk_w = _f32(T, k) if topk_w is None else topk_w
    expert_counts = _i32(E) if expert_counts is None else expert_counts
    aux = new_aux() if aux is None else aux
    w = weights.c_struct()
    check("moe_forward_static", lib().moe_forward_static(
        ctypes.byref(cfg), ctypes.byref(w), _p(x), _p(router_noise), _p(y), _p(topk_idx),
        _p(topk_w), _p(expert_counts), _p(aux), _stream()))
    return y, topk_idx, topk_w, expert_counts, aux


def moe_forward(cfg: MoeConfig, weights: LayerWeights, x, router_noise=None):
    """One-shot forward: returns (y, extras dict with topk_idx, topk_w,
    expert_counts, aux (decoded after a synchronise))."""
    f = Forward(cfg, weights)
    y = f(x, router_noise)
    torch.cuda.synchronize()
    return y, {"topk_idx": f.topk_idx, "topk_w": f.topk_w, "expert_counts": f.expert_counts,
               "aux": aux_to_dict(f.aux)}


# ---------------------------------------------------------------------------
# training: forward with saved state, then the backward


class TrainStep:
    """moe_forward_train + moe_backward with their buffers allocated once.

    forward(x, router_noise=None) -> y; backward(dy, aux_scale=1.0,
    loss_weights=None) -> dict of gradient tensors (dx in the activation
    dtype, the rest float32), for the x / noise of the last forward.  The aux
    part of the loss is aux_scale * (0.01 lb + 0.001 z), or loss_weights
    (dict with keys load_balance, z_loss, lb_squares, kl_uniform) when given."""

    def __init__(self, cfg: MoeConfig, weights: LayerWeights):
        self.cfg = cfg
        self.weights = weights
        self._w = weights.c_struct()
        T, k, E, d, f, S = cfg.n_tokens, cfg.top_k, cfg.n_experts, cfg.d_model, cfg.d_ffn, cfg.n_shared
        w1r = 2 * f if cfg.act == _lib.MOE_ACT_SWIGLU else f
        dt = torch_dtype(cfg)
        dev = _dev()
        self.saved = {
            "scores": _f32(T, E), "token_lse": _f32(T), "topk_idx": _i32(T, k), "topk_w": _f32(T, k),
            "expert_counts": _i32(E), "expert_offsets": _i32(E + 1), "perm_token": _i32(T * k),
            "inv_row": _i32(T * k),
            "y_perm": torch.empty(T * k, d, dtype=dt, device=dev),
            "preact": torch.empty(T * k, w1r, dtype=dt, device=dev),
            "shared_preact": torch.empty(T, S * w1r, dtype=dt, device=dev) if S else None,
        }
        self._s = MoeSaved(**{n: (None if v is None else v.data_ptr()) for n, v in self.saved.items()})
        self.y = torch.empty(T, d, dtype=dt, device=dev)
        self.aux = new_aux()
        f32 = dict(dtype=torch.float32, device=dev)
        self.grads = {
            "dx": torch.empty(T, d, dtype=dt, device=dev),
            "dw_router": torch.empty(E, d, **f32),
            "drouter_bias": torch.empty(E, **f32),
            "dw1": torch.empty(E, w1r, d, **f32), "dw2": torch.empty(E, d, f, **f32),
            "db1": torch.empty(E, w1r, **f32) if weights.b1 is not None else None,
            "db2": torch.empty(E, d, **f32) if weights.b2 is not None else None,
        }
        if S:
            self.grads.update({
                "dws1": torch.empty(S, w1r, d, **f32), "dws2": torch.empty(S, d, f, **f32),
                "dsb1": torch.empty(S, w1r, **f32) if weights.shared_b1 is not None else None,
                "dsb2": torch.empty(S, d, **f32) if weights.shared_b2 is not None else None,
            })
        self._g = MoeGrads(**{n: (None if self.grads.get(n) is None else self.grads[n].data_ptr())
                              for n, _ in MoeGrads._fields_})
        L = lib()
        n = ctypes.c_size_t(0)
        check("moe_forward_train", L.moe_forward_train(ctypes.byref(cfg), ctypes.byref(self._w), None,
                                                       None, None, None, None, None, ctypes.byref(n),
                                                       None))
        self.fws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=dev)
        m = ctypes.c_size_t(0)
        check("moe_backward", L.moe_backward(ctypes.byref(cfg), ctypes.byref(self._w), None, None, None,
                                             None, None, None, ctypes.byref(m), None))
        self.bws = torch.empty(max(int(m.value), 1), dtype=torch.uint8, device=dev)
        self.x = None

    def forward(self, x, router_noise=None):
        self.x = x
        n = ctypes.c_size_t(self.fws.numel())
        check("moe_forward_train", lib().moe_forward_train(
            ctypes.byref(self.cfg), ctypes.byref(self._w), _p(x), _p(router_noise), _p(self.y),
            ctypes.byref(self._s), _p(self.aux), _p(self.fws), ctypes.byref(n), _stream()))
        return self.y

    def backward(self, dy, aux_scale=1.0, loss_weights=None):
        if loss_weights is None:
            lw = MoeLossWeights(load_balance=0.01 * aux_scale, z_loss=0.001 * aux_scale)
        else:
            lw = MoeLossWeights(**{k: float(v) for k, v in loss_weights.items()})
        n = ctypes.c_size_t(self.bws.numel())
        check("moe_backward", lib().moe_backward(
            ctypes.byref(self.cfg), ctypes.byref(self._w), _p(self.x), ctypes.byref(self._s), _p(dy),
            ctypes.byref(lw), ctypes.byref(self._g), _p(self.bws), ctypes.byref(n), _stream()))
        return self.grads
