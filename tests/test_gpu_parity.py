"""Parity of the HIP library (through its C ABI) with the float64 CPU oracle.

Integer results (top-k indices, counts, offsets, permutation, inverse rows,
drops) must match bit-exactly; the layer output within the normwise
tolerance (1e-4 float32, 2e-2 bfloat16); routing weights, lse and the
auxiliary losses within their relative bounds.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from helpers import (from_dev, inputs, normwise, to_dev, tol_for,
                     weights_to_dev)
from moe_inputs import LayerConfig, get_config
from mixture_experts_layer_41_amd import binding as B

pytestmark = pytest.mark.gpu

# Routing weights come from float32 logits (MFMA or FMA accumulation) against
# float64 ones; with |logit| < ~1 the accumulated error is ~1e-6 absolute,
# and w_j = exp(l_j) / sum exp(l_sel) moves by at most twice that relatively.
W_RTOL = 1e-5
LSE_RTOL = 1e-5
AUX_RTOL = 1e-5
# kl_uniform = ln(1/E) - mean_e ln(P_e + 1e-8): P_e carries the float32
# probabilities' relative error (~1e-6), so the logarithms, and kl, carry
# about that much absolute error whatever kl's size (it is ~0 for balanced
# routing).  freq_penalty comes from the integer counts: exact up to the
# float64 summation order.
KL_ATOL = 1e-5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_oracle(cfg, t, rows=None, want_routed_rows=False):
    return oracle.forward(cfg, t, rows=rows, want_routed_rows=want_routed_rows)


def check_routing(cfg, o, idx, w, lse=None):
    idx = idx.cpu().numpy()
    w = w.cpu().numpy().astype(np.float64)
    k, E = cfg.k, cfg.E
    if k < E:
        assert np.array_equal(idx, o["topk_idx"]), "top-k indices differ"
    else:   # no gap rule at k == E: compare index sets and the weights per expert
        assert (np.sort(idx, 1) == np.arange(E)[None, :]).all()
    wref = np.take_along_axis(o["p"], idx.astype(np.int64), 1)
    wref = wref / wref.sum(1, keepdims=True)
    rel = np.max(np.abs(w - wref) / np.abs(wref))
    assert rel <= W_RTOL, f"routing weights rel err {rel:.3e}"
    if lse is not None:
        l = lse.cpu().numpy().astype(np.float64)
        # relative to max(|lse|, 1): lse near zero carries float32 absolute error
        rl = np.max(np.abs(l - o["lse"]) / np.maximum(np.abs(o["lse"]), 1.0))
        assert rl <= LSE_RTOL, f"lse err {rl:.3e}"


def check_permutation(o, res, T, k, gpu_idx):
    """Counts, offsets, permutation and drops bit-exact; inverse rows compared
    per (token, expert) so that the slot order of equal-probability experts
    (possible only when k == E) does not matter."""
    assert np.array_equal(res["expert_counts"].cpu().numpy(), o["counts"])
    assert np.array_equal(res["expert_offsets"].cpu().numpy(), o["offsets"])
    R = int(o["offsets"][-1])
    assert np.array_equal(res["perm_token"].cpu().numpy()[:R], o["perm_token"])
    assert int(res["n_dropped"].cpu().item()) == o["n_dropped"]
    inv = res["inv_row"].cpu().numpy().reshape(T, k)
    gi = gpu_idx.cpu().numpy().reshape(T, k)
    if np.array_equal(gi, o["topk_idx"]):
        assert np.array_equal(inv, o["inv_row"])
    else:
        for t in range(T):
            ref = {int(e): int(r) for e, r in zip(o["topk_idx"][t], o["inv_row"][t])}
            got = {int(e): int(r) for e, r in zip(gi[t], inv[t])}
            assert got == ref


def check_aux(aux, o):
    assert abs(aux["load_balance"] - o["lb"]) <= AUX_RTOL * abs(o["lb"]), (aux, o["lb"])
    assert abs(aux["z_loss"] - o["z"]) <= AUX_RTOL * abs(o["z"]), (aux, o["z"])
    assert abs(aux["weighted"] - o["weighted"]) <= AUX_RTOL * abs(o["weighted"])
    assert aux["n_dropped"] == o["n_dropped"]
    assert aux["capacity"] == (-1 if o["capacity"] is None else o["capacity"])
    assert abs(aux["lb_squares"] - o["lb_squares"]) <= AUX_RTOL * abs(o["lb_squares"])
    assert abs(aux["kl_uniform"] - o["kl_uniform"]) <= KL_ATOL, (aux["kl_uniform"], o["kl_uniform"])
    assert abs(aux["freq_penalty"] - o["freq_penalty"]) <= 1e-12 + 1e-9 * o["freq_penalty"]


# ---------------------------------------------------------------------------
# small shapes: every step through its own entry point, then the full layer

SMALL = [
    # name, T, d, E, k, f, S, dtype, act, cf, expert_bias, router_bias, residual
    ("f32_gelu_ragged", 77, 24, 5, 2, 40, 0, "f32", "gelu", 0.0, "random", "none", False),
    ("f32_swiglu_shared", 130, 32, 6, 3, 24, 2, "f32", "swiglu", 0.0, "random", "none", True),
    ("f32_gelu_cap", 200, 16, 4, 2, 16, 1, "f32", "gelu", 0.6, "random", "zipf", False),
    ("bf16_swiglu_ragged", 333, 72, 7, 2, 136, 0, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_swiglu_tiles", 1000, 256, 8, 2, 200, 1, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_gelu_bias", 300, 64, 12, 3, 72, 2, "bf16", "gelu", 1.0, "random", "none", True),
    ("bf16_cap_drop", 640, 128, 16, 2, 64, 0, "bf16", "swiglu", 0.5, "none", "zipf", False),
    ("bf16_k_eq_E", 64, 64, 8, 8, 64, 0, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_E1", 50, 40, 1, 1, 48, 0, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_T1_E200", 1, 128, 200, 6, 64, 1, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_E512", 96, 2048, 512, 8, 32, 0, "bf16", "swiglu", 0.0, "none", "none", False),
    ("f32_k1", 90, 16, 3, 1, 16, 0, "f32", "gelu", 0.0, "random", "none", False),
    ("bf16_cap1", 40, 32, 4, 2, 32, 0, "bf16", "swiglu", 0.25, "none", "none", False),
    # k above 8: picks past the register-held ones, generic combine and scatter paths
    ("bf16_k12_cap", 300, 64, 16, 12, 64, 1, "bf16", "swiglu", 1.0, "none", "none", True),
    ("f32_k10", 100, 32, 12, 10, 32, 0, "f32", "gelu", 0.0, "random", "none", False),
    # more than 1024 rows per group: the wide-tile grouped GEMM, ragged group
    # ends inside a 256-row tile, shared experts summed along K, GELU with
    # biases, capacity drops
    ("bf16_wide_swiglu_shared2", 3000, 512, 2, 1, 384, 2, "bf16", "swiglu", 0.0, "none", "none", False),
    ("bf16_wide_gelu_bias", 2600, 256, 2, 1, 512, 1, "bf16", "gelu", 0.0, "random", "none", True),
    ("bf16_wide_cap_zipf", 4100, 256, 4, 2, 256, 0, "bf16", "swiglu", 1.0, "none", "zipf", False),
    # 8 column tiles on both products: the wide kernel's grouped tile order
    # (groups of 8 row tiles, the last group ragged: 10 row tiles)
    ("bf16_wide_grouped_order", 2050, 2048, 2, 1, 1024, 0, "bf16", "swiglu", 0.0, "none", "none", False),
    # d = 384: the down product's last column tile is half a tile
    ("bf16_wide_half_tile", 2300, 384, 2, 1, 256, 1, "bf16", "swiglu", 0.0, "none", "none", True),
    # SwiGLU with expert biases on the wide tiles (gate and up halves of the
    # bias slice; the shared pair's two down biases summed), with the half
    # column tile: the bias of its columns past d clamped
    ("bf16_wide_swiglu_bias", 2400, 384, 2, 1, 256, 2, "bf16", "swiglu", 0.0, "random", "none", False),
    # decode-sized groups with expert biases: the 32-row decode tiles (many
    # groups: 32 x 256; the one shared group of 100 rows: 32 x 128)
    ("bf16_decode_tiles_bias", 100, 256, 16, 2, 128, 1, "bf16", "swiglu", 0.0, "random", "none", False),
    ("bf16_decode_tiles_gelu", 120, 512, 8, 1, 256, 2, "bf16", "gelu", 0.0, "random", "none", True),
    # decode tiles over groups of 23-41 rows: groups of at most 32 rows are
    # one row tile (weights streamed with the nontemporal hint), larger ones
    # two (weights cached), in one launch
    ("bf16_decode_mixed_rows", 256, 256, 16, 2, 128, 1, "bf16", "swiglu", 0.0, "none", "none", False),
]


def small_cfg(row, seed):
    (name, T, d, E, k, f, S, dt, act, cf, eb, rb, res) = row
    return LayerConfig(name, T=T, d=d, E=E, k=k, f=f, S=S, dtype=dt, act=act, capacity_factor=cf,
                       router_bias=rb if rb != "zipf" else "zipf", expert_bias=eb,
                       add_residual=res, seed=seed)


@pytest.mark.parametrize("row", SMALL, ids=[r[0] for r in SMALL])
def test_small_shapes_all_steps(row):
    cfg = small_cfg(row, seed=500 + SMALL.index(row))
    say(f"[case] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} S={cfg.S} {cfg.dtype}")
    t = inputs(cfg)
    o = run_oracle(cfg, t, want_routed_rows=True)
    c = B.config_of(cfg)
    W = weights_to_dev(cfg, t)
    x = to_dev(t["x"], cfg.dtype)

    # moe_route
    idx, w, lse, route_ws = B.moe_route(c, x, W.w_router, W.router_bias)
    torch.cuda.synchronize()
    check_routing(cfg, o, idx, w, lse)

    # moe_permute (on the GPU's own indices, which equal the oracle's)
    pr = B.moe_permute(c, idx, w, x, want_perm_w=True, want_x_perm=True)
    torch.cuda.synchronize()
    check_permutation(o, pr, cfg.T, cfg.k, idx)
    R = int(o["offsets"][-1])
    xd = oracle.decode(t["x"], cfg.dtype)
    assert np.array_equal(from_dev(pr["x_perm"][:R]), xd[o["perm_token"]])
    inv = pr["inv_row"].cpu().numpy().reshape(cfg.T, cfg.k)
    wg = w.cpu().numpy()
    pw = pr["perm_w"].cpu().numpy()
    kept = inv >= 0
    assert np.array_equal(pw[inv[kept]], wg[kept])

    # moe_aux_stats
    aux = B.aux_to_dict(B.moe_aux_stats(c, pr["expert_counts"], pr["n_dropped"], route_ws))
    check_aux(aux, o)

    # moe_expert_ffn (routed), against the oracle's unweighted expert rows
    y_perm = B.moe_expert_ffn(c, cfg.E, 1, cfg.T * cfg.k, x, pr["perm_token"],
                              pr["expert_offsets"], W.w1, W.b1, W.w2, W.b2)
    torch.cuda.synchronize()
    if R:
        err = normwise(from_dev(y_perm[:R]), o["routed_rows"])
        assert err <= tol_for(cfg), f"expert rows normwise err {err:.3e}"

    # shared experts as one group of n_seg = S
    shared_y = None
    if cfg.S:
        shared_y = B.moe_expert_ffn(c, 1, cfg.S, cfg.T, x, None, None, W.shared_w1, W.shared_b1,
                                    W.shared_w2, W.shared_b2)
        torch.cuda.synchronize()
        err = normwise(from_dev(shared_y), o["shared_y"])
        assert err <= tol_for(cfg), f"shared normwise err {err:.3e}"

    # moe_combine
    y = B.moe_combine(c, y_perm, pr["inv_row"], w, shared_y, x if cfg.add_residual else None)
    torch.cuda.synchronize()
    err = normwise(from_dev(y), o["y"])
    assert err <= tol_for(cfg), f"combine normwise err {err:.3e}"

    # moe_forward, and determinism of two runs
    F = B.Forward(c, W)
    y1 = F(x).clone()
    y2 = F(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1,
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2)
    err = normwise(from_dev(y1), o["y"])
    assert err <= tol_for(cfg), f"forward normwise err {err:.3e}"
    check_routing(cfg, o, F.topk_idx, F.topk_w)
    assert np.array_equal(F.expert_counts.cpu().numpy(), o["counts"])
    check_aux(B.aux_to_dict(F.aux), o)
    say(f"[ok] {cfg.name} y_err={err:.2e}")


# ---------------------------------------------------------------------------
# the named workloads at full size: routing, permutation and aux in full; the
# output on every token, except for the two 65536-token layers, whose output
# is compared on a sample that covers every row tile of every expert: the
# tokens in the first and last row of each 128-row block of each expert's
# rows (the grouped GEMMs use tiles of 128 or 256 rows, so every tile of
# either size, each expert's last partial tile included, has compared rows)

FULL = {"c1": "all", "c2": "all", "c2n": "all", "c3": "all", "c4": "tiles", "c4cap": "tiles",
        "c5": "all", "c5q": "all"}
LAZY = ("c5", "c5q")  # expert weights generated one expert at a time


def tile_cover_rows(cfg, t, block=128):
    """Tokens in the first and last row of every `block`-row block of every
    expert's kept rows, with the oracle's own routing, dispatch order and
    capacity."""
    xd = oracle.decode(t["x"], cfg.dtype)
    wr = oracle.decode(t["w_router"], cfg.dtype)
    rb = t.get("router_bias")
    logits = oracle.router_scores(
        oracle.router_logits(xd, wr, None if rb is None else np.asarray(rb, np.float32).astype(np.float64)),
        cfg.router_temperature, t.get("router_noise"))
    p, _ = oracle.softmax_lse(logits)
    idx = oracle.topk_select(p, cfg.k)
    cap = oracle.capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
    offsets, perm_token, _, _, _ = oracle.dispatch(idx, cfg.E, cap)
    rows = set()
    for e in range(cfg.E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        for b in range(r0, r1, block):
            rows.add(int(perm_token[b]))
            rows.add(int(perm_token[min(b + block, r1) - 1]))
    rows.update((0, cfg.T - 1))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", list(FULL))
def test_named_workload_full_size(name):
    cfg = get_config(name)
    say(f"[case] {name}: {cfg.name}")
    t = inputs(cfg, materialize=(name not in LAZY))
    rows = tile_cover_rows(cfg, t) if FULL[name] == "tiles" else None
    if rows is not None:
        say(f"[rows] {name}: {len(rows)} tokens cover every 128-row block of every expert")
    c = B.config_of(cfg)
    say(f"[upload] {name}")
    keep = set(range(cfg.E)) if name in LAZY else None
    W = weights_to_dev(cfg, t, keep_experts=keep)
    say(f"[oracle] {name}")
    o = run_oracle(cfg, t, rows=rows)
    x = to_dev(t["x"], cfg.dtype)
    noise = to_dev(t.get("router_noise"), "f32")
    F = B.Forward(c, W)
    say(f"[forward] {name}")
    y = F(x, noise)
    torch.cuda.synchronize()
    check_routing(cfg, o, F.topk_idx, F.topk_w)
    assert np.array_equal(F.expert_counts.cpu().numpy(), o["counts"])
    aux = B.aux_to_dict(F.aux)
    check_aux(aux, o)
    yg = from_dev(y) if rows is None else from_dev(y[torch.as_tensor(rows, device="cuda")])
    err = normwise(yg, o["y"])
    assert err <= tol_for(cfg), f"{name} normwise err {err:.3e}"
    # the standalone permutation on the same indices
    pr = B.moe_permute(c, F.topk_idx)
    torch.cuda.synchronize()
    check_permutation(o, pr, cfg.T, cfg.k, F.topk_idx)
    say(f"[ok] {name} y_err={err:.2e} over {cfg.T if rows is None else len(rows)} tokens "
        f"lb={aux['load_balance']:.6f} z={aux['z_loss']:.6f} dropped={aux['n_dropped']}")


# ---------------------------------------------------------------------------
# 8-bit expert weights: INT8 codes with float32 row scales (bf16 activations)

SMALL_Q8 = [
    # name, T, d, E, k, f, S, act, cf, expert_bias, router_bias, residual
    ("q8_swiglu", 200, 128, 8, 2, 128, 0, "swiglu", 0.0, "none", "none", False),
    ("q8_gelu_bias_shared2", 150, 256, 6, 3, 128, 2, "gelu", 0.0, "random", "none", True),
    ("q8_cap_drop_shared", 300, 128, 16, 2, 256, 1, "swiglu", 1.0, "none", "zipf", False),
    ("q8_k10", 64, 128, 12, 10, 128, 0, "swiglu", 0.0, "none", "none", False),
    # decode-shaped (12 rows per expert) with K = 512 and 256: the INT8
    # weight stream's two-deep prefetch over several loop turns
    ("q8_decode_k512", 96, 512, 32, 4, 256, 1, "swiglu", 0.0, "random", "none", False),
]


@pytest.mark.parametrize("row", SMALL_Q8, ids=[r[0] for r in SMALL_Q8])
def test_int8_weights_small(row):
    (name, T, d, E, k, f, S, act, cf, eb, rb, res) = row
    cfg = LayerConfig(name, T=T, d=d, E=E, k=k, f=f, S=S, dtype="bf16", act=act,
                      capacity_factor=cf, router_bias=rb, expert_bias=eb, add_residual=res,
                      weights="int8", seed=700 + SMALL_Q8.index(row))
    say(f"[case] {name} T={T} d={d} E={E} k={k} f={f} S={S} int8 weights")
    t = inputs(cfg)
    o = run_oracle(cfg, t, want_routed_rows=True)
    c = B.config_of(cfg)
    W = weights_to_dev(cfg, t)
    x = to_dev(t["x"], cfg.dtype)

    # the expert FFN entry point with INT8 weights, routed and shared
    idx, w, _, _ = B.moe_route(c, x, W.w_router, W.router_bias)
    pr = B.moe_permute(c, idx, w, x)
    torch.cuda.synchronize()
    check_permutation(o, pr, T, k, idx)
    R = int(o["offsets"][-1])
    y_perm = B.moe_expert_ffn_int8(c, E, 1, T * k, x, pr["perm_token"], pr["expert_offsets"],
                                   W.w1, W.w1_scale, W.b1, W.w2, W.w2_scale, W.b2)
    torch.cuda.synchronize()
    if R:
        err = normwise(from_dev(y_perm[:R]), o["routed_rows"])
        assert err <= tol_for(cfg), f"expert rows normwise err {err:.3e}"
    if S:
        sy = B.moe_expert_ffn_int8(c, 1, S, T, x, None, None, W.shared_w1, W.shared_w1_scale,
                                   W.shared_b1, W.shared_w2, W.shared_w2_scale, W.shared_b2)
        torch.cuda.synchronize()
        err = normwise(from_dev(sy), o["shared_y"])
        assert err <= tol_for(cfg), f"shared normwise err {err:.3e}"

    # the whole layer, twice (deterministic)
    F = B.Forward(c, W)
    y1 = F(x).clone()
    y2 = F(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    err = normwise(from_dev(y1), o["y"])
    assert err <= tol_for(cfg), f"forward normwise err {err:.3e}"
    check_routing(cfg, o, F.topk_idx, F.topk_w)
    check_aux(B.aux_to_dict(F.aux), o)
    say(f"[ok] {name} y_err={err:.2e}")


# ---------------------------------------------------------------------------
# router temperature and noise: the scores are logits / tau + noise

VARIANTS = [
    # name, T, d, E, k, f, S, dtype, tau, noise std, router bias, cf
    ("f32_tau_half", 150, 32, 8, 2, 32, 0, "f32", 0.5, 0.0, "none", 0.0),
    ("f32_tau2_noise", 200, 48, 10, 3, 32, 1, "f32", 2.0, 0.5, "zipf", 0.0),
    ("bf16_noise_cap", 700, 128, 16, 2, 128, 0, "bf16", 1.0, 1.0, "none", 1.0),
    ("bf16_tau1.5_noise_E64", 1200, 256, 64, 6, 64, 2, "bf16", 1.5, 1.0, "zipf", 0.0),
    # decode-sized: the router's K split and separate selection kernel
    ("bf16_decode_tau_noise", 64, 2048, 128, 8, 128, 1, "bf16", 1.5, 1.0, "none", 0.0),
    # batches that fill the chip: the router's LDS-staged logits pipeline
    # (32- and 64-token blocks, ragged last block, 1 and 3 K chunks, 64 and
    # 128 experts)
    ("bf16_staged_tau_noise_E64", 16400, 192, 64, 6, 64, 1, "bf16", 1.5, 1.0, "zipf", 0.0),
    ("bf16_staged_E128_cap", 32800, 64, 128, 8, 32, 0, "bf16", 0.7, 0.5, "none", 1.0),
]


@pytest.mark.parametrize("row", VARIANTS, ids=[r[0] for r in VARIANTS])
def test_router_temperature_and_noise(row):
    (name, T, d, E, k, f, S, dt, tau, sd, rb, cf) = row
    cfg = LayerConfig(name, T=T, d=d, E=E, k=k, f=f, S=S, dtype=dt, act="swiglu",
                      capacity_factor=cf, router_bias=rb, router_temperature=tau,
                      router_noise_std=sd, seed=800 + VARIANTS.index(row))
    say(f"[case] {name} T={T} d={d} E={E} k={k} tau={tau} noise={sd}")
    t = inputs(cfg)
    o = run_oracle(cfg, t)
    c = B.config_of(cfg)
    W = weights_to_dev(cfg, t)
    x = to_dev(t["x"], cfg.dtype)
    noise = to_dev(t["router_noise"], "f32")

    idx, w, lse, route_ws = B.moe_route(c, x, W.w_router, W.router_bias, noise)
    torch.cuda.synchronize()
    check_routing(cfg, o, idx, w, lse)
    pr = B.moe_permute(c, idx, w)
    aux = B.aux_to_dict(B.moe_aux_stats(c, pr["expert_counts"], pr["n_dropped"], route_ws))
    check_permutation(o, pr, T, k, idx)
    check_aux(aux, o)

    F = B.Forward(c, W)
    y = F(x, noise)
    torch.cuda.synchronize()
    check_routing(cfg, o, F.topk_idx, F.topk_w)
    check_aux(B.aux_to_dict(F.aux), o)
    err = normwise(from_dev(y), o["y"])
    assert err <= tol_for(cfg), f"forward normwise err {err:.3e}"
    say(f"[ok] {name} y_err={err:.2e} kl={aux['kl_uniform']:.3e} freq={aux['freq_penalty']:.3e}")
