"""Shared helpers of the GPU tests: device upload of generated inputs, the
normwise error, and oracle runs on the same inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from moe_inputs import Bank, make_inputs
from mixture_experts_layer_41_amd import binding as B


def tol_for(cfg):
    """Output tolerance (normwise max-abs error / max-abs reference)."""
    return 1e-4 if cfg.dtype == "f32" else 2e-2


def normwise(a, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / (den if den > 0 else 1.0))


def to_dev(arr, dtype: str):
    """numpy (uint16 bf16 bits, int8 weight codes or float32) -> cuda tensor."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.int8:
        return torch.from_numpy(a).cuda()
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bank_to_dev(bank, dtype: str, threads: int = 16, keep=None):
    """Fill a device tensor from a lazy Bank (or numpy array) one expert at a
    time.  Experts listed in `keep` are also returned as host arrays
    ({e: array}), so a later oracle run does not draw them again."""
    if bank is None:
        return None
    if isinstance(bank, np.ndarray):
        return to_dev(bank, dtype)
    tdt = {np.uint16: torch.bfloat16, np.int8: torch.int8}.get(bank.np_dtype, torch.float32)
    out = torch.empty(bank.full_shape, dtype=tdt, device="cuda")
    from concurrent.futures import ThreadPoolExecutor

    def gen(e):
        return e, bank[e]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        for e, a in ex.map(gen, range(bank.n)):
            out[e].copy_(to_dev(a, dtype))
            if keep is not None and e in keep.get("ids", ()):
                keep.setdefault("arrays", {})[e] = a
    return out


def from_dev(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def gap_accept(cfg):
    return lambda x, w, b, n: oracle.router_gap_ok(x, w, b, cfg.k, cfg.dtype,
                                                   temperature=cfg.router_temperature, noise=n)


def inputs(cfg, materialize=True):
    return make_inputs(cfg, accept=gap_accept(cfg), materialize=materialize)


def weights_to_dev(cfg, t, keep_experts=None) -> B.LayerWeights:
    """Upload a layer's weights.  With lazy banks and keep_experts (a set of
    routed expert ids), the host copies of those experts replace the banks in
    `t` (as dicts), so the oracle can run on them afterwards."""
    dt = cfg.dtype
    rb = t.get("router_bias")
    kept = {}
    banks = {}
    routed_keys = ("w1", "w2", "b1", "b2", "w1_scale", "w2_scale")
    for key in routed_keys + ("ws1", "ws2", "sb1", "sb2", "ws1_scale", "ws2_scale"):
        ids = keep_experts if key in routed_keys else set(range(cfg.S))
        kept[key] = {"ids": ids or set()}
        banks[key] = bank_to_dev(t.get(key), dt, keep=kept[key])
    if keep_experts is not None:
        for key, kk in kept.items():
            if "arrays" in kk:
                t[key] = kk["arrays"]
    return B.LayerWeights(
        w_router=to_dev(t["w_router"], dt),
        router_bias=None if rb is None else torch.from_numpy(np.asarray(rb, np.float32)).cuda(),
        w1=banks["w1"], w2=banks["w2"], b1=banks["b1"], b2=banks["b2"],
        shared_w1=banks["ws1"], shared_w2=banks["ws2"], shared_b1=banks["sb1"], shared_b2=banks["sb2"],
        w1_scale=banks["w1_scale"], w2_scale=banks["w2_scale"],
        shared_w1_scale=banks["ws1_scale"], shared_w2_scale=banks["ws2_scale"],
    )


def routed_experts(cfg, t, rows):
    """Experts the given tokens route to (oracle routing on the CPU)."""
    xd = oracle.decode(t["x"][rows], cfg.dtype)
    wr = oracle.decode(t["w_router"], cfg.dtype)
    rb = t.get("router_bias")
    p, _ = oracle.softmax_lse(oracle.router_logits(xd, wr, None if rb is None else rb.astype(np.float64)))
    return set(int(e) for e in oracle.topk_select(p, cfg.k).reshape(-1))
