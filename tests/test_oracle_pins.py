"""Pins of the CPU oracle against facts fixed outside the oracle itself:
closed forms, brute force on tiny inputs, library routines (torch float64 on
the CPU, scipy) for special cases, invariants, and the parameter arithmetic a
page prints.  CPU only.

Page keys as in the oracle header: [P1] Naive-N0.5-Flash blog, [P2] MoE
explainer (mqxn.cn), [P3] small-MoE tutorial (lshu.cn), [P4] OpenMythos blog,
[P5] FLAME-MoE summary.
"""

import itertools
import json
import math
import os
from dataclasses import dataclass

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

import oracle
from moe_inputs import LayerConfig, f32_to_bf16_bits, get_config, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@dataclass
class Cfg:
    T: int
    d: int
    E: int
    k: int
    f: int
    S: int = 0
    dtype: str = "f32"
    act: str = "swiglu"
    capacity_factor: float = 0.0
    add_residual: bool = False


def f32(a):
    return np.asarray(a, dtype=np.float32)


def rand_tensors(cfg, seed, bias=False, router_bias=None):
    """Small float32 tensors for oracle-only pins."""
    r = np.random.default_rng(seed)
    rows = 2 * cfg.f if cfg.act == "swiglu" else cfg.f
    t = {
        "x": f32(r.standard_normal((cfg.T, cfg.d))),
        "w_router": f32(r.standard_normal((cfg.E, cfg.d)) * 0.5),
        "router_bias": None if router_bias is None else f32(router_bias),
        "w1": f32(r.standard_normal((cfg.E, rows, cfg.d)) * 0.3),
        "w2": f32(r.standard_normal((cfg.E, cfg.d, cfg.f)) * 0.3),
        "b1": f32(r.standard_normal((cfg.E, rows)) * 0.1) if bias else None,
        "b2": f32(r.standard_normal((cfg.E, cfg.d)) * 0.1) if bias else None,
        "ws1": f32(r.standard_normal((cfg.S, rows, cfg.d)) * 0.3) if cfg.S else None,
        "ws2": f32(r.standard_normal((cfg.S, cfg.d, cfg.f)) * 0.3) if cfg.S else None,
        "sb1": None, "sb2": None,
    }
    return t


def torch_ffn(x, w1, b1, w2, b2, act):
    """Expert FFN through torch's float64 CPU library routines."""
    x = torch.as_tensor(x, dtype=torch.float64)
    w1 = torch.as_tensor(np.asarray(w1, dtype=np.float64))
    w2 = torch.as_tensor(np.asarray(w2, dtype=np.float64))
    b1 = None if b1 is None else torch.as_tensor(np.asarray(b1, dtype=np.float64))
    b2 = None if b2 is None else torch.as_tensor(np.asarray(b2, dtype=np.float64))
    if act == "gelu":
        h = F.gelu(F.linear(x, w1, b1), approximate="none")
    else:
        gu = F.linear(x, w1, b1)
        g, u = gu.chunk(2, dim=-1)
        h = F.silu(g) * u
    return F.linear(h, w2, b2).numpy()


# ---------------------------------------------------------------------------
# worked example with closed-form values (hand-derived)


def test_worked_example_closed_form():
    """x = [1, 0]; router rows give logits [0, ln 2, ln 3].

    p = [1/6, 1/3, 1/2], lse = ln 6, top-2 = [2, 1], w = [3/5, 2/5];
    f = [0, 1/2, 1/2], P = p -> lb = 3 * (1/2 * 1/3 + 1/2 * 1/2) = 5/4,
    z = (ln 6)^2.  SwiGLU expert 2 with one hidden unit: gate weight 2, up
    weight 3 on x[0] -> h = 3 * silu(2) = 6 / (1 + e^-2); W2 column [1, -1].
    Expert 1: gate 1, up 1 -> h = 1 / (1 + e^-1); W2 column [2, 0].
    """
    cfg = Cfg(T=1, d=2, E=3, k=2, f=1)
    ln2, ln3 = math.log(2.0), math.log(3.0)
    t = {
        "x": f32([[1.0, 0.0]]),
        "w_router": f32([[0.0, 5.0], [ln2, -1.0], [ln3, 7.0]]),
        "router_bias": None,
        "w1": f32([[[9.0, 0.0], [9.0, 0.0]],      # expert 0 (not selected)
                   [[1.0, 0.0], [1.0, 0.0]],      # expert 1: gate 1, up 1
                   [[2.0, 0.0], [3.0, 0.0]]]),    # expert 2: gate 2, up 3
        "w2": f32([[[5.0], [5.0]], [[2.0], [0.0]], [[1.0], [-1.0]]]),
        "b1": None, "b2": None, "ws1": None, "ws2": None,
    }
    o = oracle.forward(cfg, t)
    tol = 1e-6  # float32 storage of ln 2, ln 3
    assert np.allclose(o["p"][0], [1 / 6, 1 / 3, 1 / 2], atol=tol)
    assert abs(o["lse"][0] - math.log(6.0)) < tol
    assert o["topk_idx"].tolist() == [[2, 1]]
    assert np.allclose(o["topk_w"][0], [3 / 5, 2 / 5], atol=tol)
    assert o["counts"].tolist() == [0, 1, 1]
    assert abs(o["lb"] - 5 / 4) < tol
    assert abs(o["z"] - math.log(6.0) ** 2) < 1e-5
    assert abs(o["weighted"] - (0.01 * 5 / 4 + 0.001 * math.log(6.0) ** 2)) < 1e-6
    h2 = 6.0 / (1.0 + math.exp(-2.0))
    h1 = 1.0 / (1.0 + math.exp(-1.0))
    y = 3 / 5 * np.array([h2, -h2]) + 2 / 5 * np.array([2 * h1, 0.0])
    assert np.allclose(o["y"][0], y, atol=1e-6)
    # dispatch of the single token: expert 1 row 0, expert 2 row 1
    assert o["offsets"].tolist() == [0, 0, 1, 2]
    assert o["perm_token"].tolist() == [0, 0]
    assert o["inv_row"].tolist() == [[1, 0]]


# ---------------------------------------------------------------------------
# activations against library routines and exact identities


def test_gelu_is_exact_erf_form():
    z = np.linspace(-6, 6, 241)
    g = oracle.moe_oracle._gelu(z)
    assert np.allclose(g, z * scipy.stats.norm.cdf(z), rtol=1e-13, atol=1e-15)
    assert np.allclose(g - oracle.moe_oracle._gelu(-z), z, atol=1e-13)   # gelu(z) - gelu(-z) = z
    assert oracle.moe_oracle._gelu(np.array([0.0]))[0] == 0.0
    # not the tanh approximation
    tanh_form = 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert np.max(np.abs(g - tanh_form)) > 1e-5


def test_silu_identities():
    z = np.linspace(-20, 20, 401)
    s = oracle.moe_oracle._silu(z)
    assert np.allclose(s, z * scipy.special.expit(z), rtol=1e-13, atol=1e-15)
    assert np.allclose(s - oracle.moe_oracle._silu(-z), z, atol=1e-12)
    assert oracle.moe_oracle._silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# routing: brute force, logit-form identity, special cases


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_tiny(seed):
    """Top-k set = unique maximiser of the sum of logits over k-subsets, in
    descending-probability order; weights = softmax over the selected logits
    ([P2 §4.1] takes top-k on logits then a softmax over the k)."""
    r = np.random.default_rng(seed)
    T, E = 8, 2 + seed % 5
    k = 1 + seed % min(3, E)
    cfg = Cfg(T=T, d=5, E=E, k=k, f=3)
    t = rand_tensors(cfg, seed)
    o = oracle.forward(cfg, t)
    logits = t["x"].astype(np.float64) @ t["w_router"].astype(np.float64).T
    for tok in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(logits[tok, i] for i in S))
        chosen = sorted(best, key=lambda i: -logits[tok, i])
        assert o["topk_idx"][tok].tolist() == chosen
        den = sum(math.exp(logits[tok, i]) for i in chosen)
        w = [math.exp(logits[tok, i]) / den for i in chosen]
        assert np.allclose(o["topk_w"][tok], w, rtol=1e-12)
        # full softmax and lse against torch
        lt = torch.as_tensor(logits[tok])
        assert np.allclose(o["p"][tok], torch.softmax(lt, 0).numpy(), rtol=1e-12)
        assert abs(o["lse"][tok] - torch.logsumexp(lt, 0).item()) < 1e-12


def test_zero_router_uniform():
    """W_r = 0: p = 1/E, lse = ln E, idx = 0..k-1, w = 1/k, lb = 1,
    z = (ln E)^2."""
    cfg = Cfg(T=16, d=4, E=6, k=3, f=2)
    t = rand_tensors(cfg, 3)
    t["w_router"] = np.zeros_like(t["w_router"])
    o = oracle.forward(cfg, t)
    assert np.allclose(o["p"], 1 / 6, rtol=1e-15)
    assert np.allclose(o["lse"], math.log(6), rtol=1e-15)
    assert (o["topk_idx"] == np.arange(3)[None, :]).all()
    assert np.allclose(o["topk_w"], 1 / 3, rtol=1e-15)
    assert abs(o["lb"] - 1.0) < 1e-14
    assert abs(o["z"] - math.log(6) ** 2) < 1e-13


def test_k1_weight_is_one_and_dominant_expert_lb_tends_to_E():
    cfg = Cfg(T=32, d=4, E=5, k=1, f=2)
    bias = np.array([60.0, 0, 0, 0, 0])
    t = rand_tensors(cfg, 4, router_bias=bias)
    o = oracle.forward(cfg, t)
    assert (o["topk_w"] == 1.0).all()
    assert (o["topk_idx"][:, 0] == 0).all()
    assert abs(o["lb"] - 5.0) < 1e-9          # f_0 = 1, P_0 -> 1


def test_k_equals_E_weights_are_full_softmax():
    cfg = Cfg(T=10, d=4, E=4, k=4, f=2)
    t = rand_tensors(cfg, 5)
    o = oracle.forward(cfg, t)
    p_sorted = np.take_along_axis(o["p"], o["topk_idx"], axis=1)
    assert np.allclose(o["topk_w"], p_sorted, rtol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_weight_invariants(seed):
    cfg = Cfg(T=64, d=8, E=7, k=3, f=4)
    o = oracle.forward(cfg, rand_tensors(cfg, seed))
    assert np.allclose(o["topk_w"].sum(axis=1), 1.0, atol=1e-12)
    assert (np.diff(o["topk_w"], axis=1) <= 0).all()
    assert o["counts"].sum() == cfg.T * cfg.k
    for row in o["topk_idx"]:
        assert len(set(row.tolist())) == cfg.k


# ---------------------------------------------------------------------------
# FFN closed forms and dense-mixture equivalence


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_single_expert_closed_form(act):
    """E = 1, k = 1: y = FFN(x) exactly (weight 1), via torch float64."""
    cfg = Cfg(T=9, d=6, E=1, k=1, f=5, act=act)
    t = rand_tensors(cfg, 7, bias=True)
    o = oracle.forward(cfg, t)
    ref = torch_ffn(t["x"], t["w1"][0], t["b1"][0], t["w2"][0], t["b2"][0], act)
    assert np.allclose(o["y"], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_dense_mixture_k_equals_E(act):
    """k = E: y = sum_e p_e FFN_e(x), computed densely with torch."""
    cfg = Cfg(T=12, d=5, E=4, k=4, f=3, act=act)
    t = rand_tensors(cfg, 8, bias=True)
    o = oracle.forward(cfg, t)
    x = torch.as_tensor(t["x"], dtype=torch.float64)
    p = torch.softmax(x @ torch.as_tensor(t["w_router"], dtype=torch.float64).T, dim=1).numpy()
    ref = sum(p[:, e:e + 1] * torch_ffn(t["x"], t["w1"][e], t["b1"][e], t["w2"][e], t["b2"][e], act)
              for e in range(cfg.E))
    assert np.allclose(o["y"], ref, rtol=1e-12, atol=1e-13)


def test_shared_experts_equal_one_wide_ffn():
    """S SwiGLU experts of width f (weight 1 each) = one SwiGLU FFN of width
    S*f with stacked gate rows, stacked up rows and concatenated down columns."""
    cfg = Cfg(T=7, d=6, E=3, k=1, f=4, S=3)
    t = rand_tensors(cfg, 9)
    o = oracle.forward(cfg, t)
    f = cfg.f
    gate = np.concatenate([t["ws1"][s][:f] for s in range(cfg.S)])
    up = np.concatenate([t["ws1"][s][f:] for s in range(cfg.S)])
    down = np.concatenate([t["ws2"][s] for s in range(cfg.S)], axis=1)
    ref = torch_ffn(t["x"], np.concatenate([gate, up]), None, down, None, "swiglu")
    assert np.allclose(o["shared_y"], ref, rtol=1e-12, atol=1e-13)


def test_linearity_in_w2():
    cfg = Cfg(T=20, d=6, E=4, k=2, f=5)
    t = rand_tensors(cfg, 10)
    o1 = oracle.forward(cfg, t)
    t2 = dict(t, w2=t["w2"] * np.float32(2.0))
    o2 = oracle.forward(cfg, t2)
    assert np.array_equal(o2["y"], 2.0 * o1["y"])


def test_residual_matches_explainer_assert():
    """[P2 §4.1]: output == expert outputs + x."""
    cfg = Cfg(T=11, d=6, E=4, k=2, f=5)
    t = rand_tensors(cfg, 11)
    o = oracle.forward(cfg, t)
    o_res = oracle.forward(Cfg(**{**cfg.__dict__, "add_residual": True}), t)
    assert np.allclose(o_res["y"], o["y"] + t["x"].astype(np.float64), atol=1e-5)


# ---------------------------------------------------------------------------
# counts, capacity, permutation


def test_capacity_exact_values():
    assert oracle.capacity(1.25, 4096, 2, 16) == 640
    assert oracle.capacity(1.0, 65536, 6, 64) == 6144
    assert oracle.capacity(0.0, 100, 2, 4) is None
    assert oracle.capacity(-1.0, 100, 2, 4) is None
    assert oracle.capacity(0.5, 6, 1, 3) == 1          # exactly integral: no round-up
    # binary64 reading: 0.1 is slightly above 1/10, so 0.1 * 30 / 3 > 1
    assert oracle.capacity(0.1, 30, 1, 3) == 2
    with pytest.raises(ValueError):
        oracle.capacity(float("nan"), 10, 1, 2)


def _check_perm_structure(o, T, k, E):
    off, pt, inv = o["offsets"], o["perm_token"], o["inv_row"]
    R = int(off[-1])
    assert R + o["n_dropped"] == T * k
    assert len(pt) == R
    rows = inv[inv >= 0]
    assert sorted(rows.tolist()) == list(range(R))       # bijection onto kept rows
    for e in range(E):
        seg = pt[off[e]:off[e + 1]]
        assert (np.diff(seg) > 0).all()                   # strictly increasing tokens
        for r in range(off[e], off[e + 1]):
            tt = pt[r]
            j = int(np.nonzero(o["topk_idx"][tt] == e)[0][0])
            assert inv[tt, j] == r


def test_capacity_one_keeps_lowest_token():
    cfg = Cfg(T=8, d=4, E=4, k=2, f=2, capacity_factor=0.25)   # C = ceil(0.25*16/4) = 1
    t = rand_tensors(cfg, 12)
    o = oracle.forward(cfg, t)
    assert o["capacity"] == 1
    _check_perm_structure(o, cfg.T, cfg.k, cfg.E)
    for e in range(cfg.E):
        toks = np.nonzero((o["topk_idx"] == e).any(axis=1))[0]
        seg = o["perm_token"][o["offsets"][e]:o["offsets"][e + 1]].tolist()
        assert seg == ([int(toks.min())] if len(toks) else [])


def test_huge_capacity_equals_no_capacity():
    cfg = Cfg(T=40, d=6, E=5, k=2, f=3)
    t = rand_tensors(cfg, 13)
    a = oracle.forward(cfg, t)
    b = oracle.forward(Cfg(**{**cfg.__dict__, "capacity_factor": 1e6}), t)
    for key in ("offsets", "perm_token", "inv_row"):
        assert np.array_equal(a[key], b[key])
    assert b["n_dropped"] == 0
    assert np.array_equal(a["y"], b["y"])


def test_drop_heavy_against_sorted_lists():
    """Flash-config shape at capacity factor 0.5 (C = 256): per-expert kept
    tokens are the C smallest token indices routed to it."""
    cfg = get_config("c2", capacity_factor=0.5)
    t = make_inputs(cfg, accept=lambda x, w, b, n: oracle.router_gap_ok(x, w, b, cfg.k, cfg.dtype, noise=n))
    xd = oracle.decode(t["x"], "bf16")
    wr = oracle.decode(t["w_router"], "bf16")
    p, _ = oracle.softmax_lse(oracle.router_logits(xd, wr))
    idx = oracle.topk_select(p, cfg.k)
    C = oracle.capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
    assert C == 256
    offsets, pt, ps, inv, nd = oracle.dispatch(idx, cfg.E, C)
    dropped = 0
    for e in range(cfg.E):
        toks = np.nonzero((idx == e).any(axis=1))[0]         # ascending
        kept = toks[:C]
        dropped += len(toks) - len(kept)
        assert pt[offsets[e]:offsets[e + 1]].tolist() == kept.tolist()
        for tt in toks[C:]:
            j = int(np.nonzero(idx[tt] == e)[0][0])
            assert inv[tt, j] == -1
    assert nd == dropped > 0


def test_all_dropped_token_outputs_shared_only():
    cfg = Cfg(T=6, d=4, E=4, k=2, f=3, S=1, capacity_factor=1 / 3)  # C = ceil(6*2/4/3) = 1
    bias = np.array([40.0, 30.0, 0.0, 0.0])   # every token picks experts 0 and 1
    t = rand_tensors(cfg, 14, router_bias=bias)
    o = oracle.forward(cfg, t)
    assert o["capacity"] == 1
    assert (o["inv_row"][1:] == -1).all()
    assert np.array_equal(o["y"][1:], o["shared_y"][1:])


def test_token_permutation_invariance():
    cfg = Cfg(T=30, d=6, E=5, k=2, f=4, S=1)
    t = rand_tensors(cfg, 15)
    o = oracle.forward(cfg, t)
    perm = np.random.default_rng(0).permutation(cfg.T)
    o2 = oracle.forward(cfg, dict(t, x=t["x"][perm]))
    assert np.allclose(o2["y"], o["y"][perm], rtol=1e-12, atol=1e-14)
    assert np.array_equal(o2["counts"], o["counts"])
    assert np.array_equal(o2["topk_idx"], o["topk_idx"][perm])
    assert abs(o2["lb"] - o["lb"]) < 1e-12 and abs(o2["z"] - o["z"]) < 1e-12


def test_sampled_rows_match_full():
    cfg = Cfg(T=25, d=6, E=5, k=2, f=4, S=2, capacity_factor=1.0)
    t = rand_tensors(cfg, 16)
    full = oracle.forward(cfg, t)
    rows = [0, 3, 24, 7]
    part = oracle.forward(cfg, t, rows=rows)
    assert np.array_equal(part["rows"], sorted(rows))
    assert np.allclose(part["y"], full["y"][sorted(rows)], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# input decoding and the parameter arithmetic printed by a page


def test_bf16_decode_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3E80, 0x7F7F], dtype=np.uint16)
    v = oracle.decode(bits, "bf16")
    assert v[:4].tolist() == [1.0, -2.0, 0.0, 0.25]
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
    with pytest.raises(TypeError):
        oracle.decode(np.zeros(2, np.float32), "bf16")


def test_param_arithmetic_fixture():
    """[P1 §3.3]: d_model 1024, 8 experts, top-2, d_ff 1024 -> 2M per expert,
    16M total, dense 4*d FFN 8M, 4M active; two-matrix experts as in
    [P3 §3.1] (num_experts * hidden * ffn * 2)."""
    with open(os.path.join(GOLDEN, "p1_param_arithmetic.json")) as fh:
        g = json.load(fh)
    d, E, k, dff = g["d_model"], g["n_expert"], g["top_k"], g["d_ff"]
    per_expert = 2 * d * dff
    assert round(per_expert / 2 ** 20) == g["per_expert_M"]
    assert round(E * per_expert / 2 ** 20) == g["total_M"]
    assert round(2 * d * 4 * d / 2 ** 20) == g["dense_M"]
    assert round(k * per_expert / 2 ** 20) == g["active_M"]


# ---------------------------------------------------------------------------
# 8-bit expert weights ([P3 §6]: compress each expert's weights to INT8;
# read as symmetric codes with one float32 scale per weight row)


def int8_tensors(cfg, seed):
    """Small INT8 codes with row scales (shared experts too), float32 x."""
    r = np.random.default_rng(seed)
    rows = 2 * cfg.f if cfg.act == "swiglu" else cfg.f

    def codes(*shape):
        return r.integers(-127, 128, size=shape).astype(np.int8)

    def scales(*shape):
        return f32(r.uniform(0.002, 0.004, size=shape))

    t = {
        "x": f32(r.standard_normal((cfg.T, cfg.d))),
        "w_router": f32(r.standard_normal((cfg.E, cfg.d)) * 0.5),
        "router_bias": None,
        "w1": codes(cfg.E, rows, cfg.d), "w1_scale": scales(cfg.E, rows),
        "w2": codes(cfg.E, cfg.d, cfg.f), "w2_scale": scales(cfg.E, cfg.d),
        "b1": None, "b2": None,
        "ws1": codes(cfg.S, rows, cfg.d) if cfg.S else None,
        "ws1_scale": scales(cfg.S, rows) if cfg.S else None,
        "ws2": codes(cfg.S, cfg.d, cfg.f) if cfg.S else None,
        "ws2_scale": scales(cfg.S, cfg.d) if cfg.S else None,
        "sb1": None, "sb2": None,
    }
    return t


@dataclass
class QCfg(Cfg):
    weights: str = "int8"


def test_dequantize_int8_worked_values():
    """Row n is scaled by scale[n]: hand-computed values (binary fractions,
    exact)."""
    q = np.array([[1, -2, 0], [127, -127, 64]], dtype=np.int8)
    s = f32([0.5, 2.0])
    w = oracle.dequantize_int8(q, s)
    assert np.array_equal(w, np.array([[0.5, -1.0, 0.0], [254.0, -254.0, 128.0]]))
    with pytest.raises(TypeError):
        oracle.dequantize_int8(q.astype(np.int16), s)
    with pytest.raises(ValueError):  # a scale per column is not the format
        oracle.dequantize_int8(q, f32([1.0, 1.0, 1.0]))


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_int8_unit_scales_equal_the_float_layer(act):
    """Scales of 1: the INT8 layer is the float layer on the codes."""
    cfg = QCfg(T=40, d=16, E=4, k=2, f=8, S=1, act=act)
    t = int8_tensors(cfg, 11)
    for key in ("w1_scale", "w2_scale", "ws1_scale", "ws2_scale"):
        t[key] = np.ones_like(t[key])
    for key in ("w1", "w2", "ws1", "ws2"):  # small codes keep the activations moderate
        t[key] = (t[key] // 43).astype(np.int8)
    fl = dict(t)
    for key in ("w1", "w2", "ws1", "ws2"):
        fl[key] = t[key].astype(np.float32)
    a = oracle.forward(cfg, t)
    b = oracle.forward(Cfg(T=40, d=16, E=4, k=2, f=8, S=1, act=act), fl)
    assert np.array_equal(a["y"], b["y"])


def test_int8_down_scale_is_per_output_row():
    """A zero scale on output row m of every W2 (routed and shared) zeroes
    column m of the layer output; a per-column reading would not."""
    cfg = QCfg(T=30, d=12, E=3, k=2, f=8, S=1)
    t = int8_tensors(cfg, 12)
    m = 5
    t["w2_scale"][:, m] = 0
    t["ws2_scale"][:, m] = 0
    y = oracle.forward(cfg, t)["y"]
    assert np.all(y[:, m] == 0.0)
    assert np.all(np.abs(np.delete(y, m, axis=1)).max(axis=0) > 0)


def test_int8_gate_scale_is_per_row_of_w1():
    """A zero scale on gate row n of every W1 (SwiGLU) silences hidden unit
    n: the same output as the float layer with column n of every W2 cleared."""
    cfg = QCfg(T=30, d=12, E=3, k=2, f=8, S=1)
    t = int8_tensors(cfg, 13)
    n = 3
    t["w1_scale"][:, n] = 0
    t["ws1_scale"][:, n] = 0
    a = oracle.forward(cfg, t)["y"]
    fl = dict(t)
    for key, sk in (("w1", "w1_scale"), ("w2", "w2_scale"), ("ws1", "ws1_scale"), ("ws2", "ws2_scale")):
        fl[key] = f32(t[key].astype(np.float64) * t[sk][..., None])
    fl["w2"][:, :, n] = 0
    fl["ws2"][:, :, n] = 0
    b = oracle.forward(Cfg(T=30, d=12, E=3, k=2, f=8, S=1), fl)["y"]
    # the float layer holds scale * code rounded to float32 (relative 6e-8
    # per weight); a scale on the wrong axis would differ at order one
    np.testing.assert_allclose(a, b, rtol=1e-4, atol=1e-7)


def test_int8_output_linear_in_down_scales():
    """Doubling every W2 scale doubles the output (no residual, no b2)."""
    cfg = QCfg(T=30, d=12, E=3, k=2, f=8, S=1)
    t = int8_tensors(cfg, 14)
    a = oracle.forward(cfg, t)["y"]
    t2 = dict(t)
    t2["w2_scale"] = t["w2_scale"] * np.float32(2)
    t2["ws2_scale"] = t["ws2_scale"] * np.float32(2)
    b = oracle.forward(cfg, t2)["y"]
    np.testing.assert_allclose(b, 2.0 * a, rtol=1e-12, atol=1e-15)


def test_int8_generator_codes_and_scales():
    """The INT8 workload's inputs: codes in [-127, 127], positive row scales,
    scale * code with about the 0.02 standard deviation of the bf16 layers."""
    cfg = get_config("c5q", T=8, d=256, E=4, f=64)
    t = make_inputs(cfg)
    for key in ("w1", "w2", "ws1", "ws2"):
        assert t[key].dtype == np.int8 and t[key].min() >= -127 and t[key].max() <= 127
        s = t[key + "_scale"]
        assert s.dtype == np.float32 and s.shape == t[key].shape[:2] and (s > 0).all()
    w = t["w1"].astype(np.float64) * t["w1_scale"][..., None]
    assert 0.018 < w.std() < 0.022


# ---------------------------------------------------------------------------
# router temperature and noise ([P2 §5.1], [P2 §2.2]); the other
# load-balance forms ([P3 §3.1], [P2 §4.2])


@dataclass
class TCfg(Cfg):
    router_temperature: float = 1.0


def test_temperature_divides_logits_and_bias():
    """Scores (x W^T + b) / tau: with tau = 2 the layer equals the tau = 1
    layer with W_r / 2 and b / 2 (exact halvings of float32 values)."""
    bias = 2.0 * np.log(1.0 / (np.arange(6) + 1.0))
    c2 = TCfg(T=24, d=8, E=6, k=2, f=4, router_temperature=2.0)
    t = rand_tensors(c2, 41, router_bias=bias)
    o2 = oracle.forward(c2, t)
    t1 = dict(t)
    t1["w_router"] = f32(t["w_router"] / 2)
    t1["router_bias"] = f32(t["router_bias"] / 2)
    o1 = oracle.forward(TCfg(T=24, d=8, E=6, k=2, f=4), t1)
    assert np.array_equal(o1["topk_idx"], o2["topk_idx"])
    for key in ("p", "lse", "topk_w", "y"):
        assert np.allclose(o1[key], o2[key], rtol=1e-13, atol=1e-15), key
    for key in ("lb", "z", "lb_squares", "kl_uniform", "freq_penalty"):
        assert abs(o1[key] - o2[key]) < 1e-12, key


def test_large_temperature_flattens_the_softmax():
    """tau -> infinity: p -> 1/E, lse -> ln E, lb_squares -> 1."""
    cfg = TCfg(T=16, d=4, E=5, k=2, f=2, router_temperature=1e9)
    o = oracle.forward(cfg, rand_tensors(cfg, 42))
    assert np.allclose(o["p"], 0.2, atol=1e-8)
    assert np.allclose(o["lse"], math.log(5), atol=1e-8)
    assert abs(o["lb_squares"] - 1.0) < 1e-8


def test_noise_is_added_after_the_temperature():
    """Noise n[t, e] = c_e for every token acts like a router bias of tau*c
    (the bias is divided by tau, the noise is not)."""
    c = np.array([0.5, -0.25, 1.0, 0.0, -1.5], dtype=np.float32)
    cfg = TCfg(T=20, d=6, E=5, k=2, f=3, router_temperature=2.0)
    t = rand_tensors(cfg, 43)
    tn = dict(t)
    tn["router_noise"] = np.tile(c, (cfg.T, 1))
    tb = dict(t)
    tb["router_bias"] = f32(2.0 * c)
    on, ob = oracle.forward(cfg, tn), oracle.forward(cfg, tb)
    assert np.array_equal(on["topk_idx"], ob["topk_idx"])
    for key in ("p", "lse", "topk_w", "y"):
        assert np.allclose(on[key], ob[key], rtol=1e-13, atol=1e-15), key


def test_noise_changes_the_selection_worked_example():
    """One token, logits [0, ln 2, ln 3] (the worked example above); noise
    [ln 4, 0, 0] lifts expert 0: scores [ln 4, ln 2, ln 3], p = [4, 2, 3]/9,
    top-2 = [0, 2], w = [4/7, 3/7], lse = ln 9."""
    cfg = TCfg(T=1, d=2, E=3, k=2, f=1)
    ln2, ln3 = math.log(2.0), math.log(3.0)
    t = {
        "x": f32([[1.0, 0.0]]),
        "w_router": f32([[0.0, 5.0], [ln2, -1.0], [ln3, 7.0]]),
        "router_bias": None,
        "router_noise": f32([[math.log(4.0), 0.0, 0.0]]),
        "w1": f32(np.ones((3, 2, 2))), "w2": f32(np.ones((3, 2, 1))),
        "b1": None, "b2": None, "ws1": None, "ws2": None,
    }
    o = oracle.forward(cfg, t)
    tol = 1e-6
    assert o["topk_idx"].tolist() == [[0, 2]]
    assert np.allclose(o["p"][0], [4 / 9, 2 / 9, 3 / 9], atol=tol)
    assert np.allclose(o["topk_w"][0], [4 / 7, 3 / 7], atol=tol)
    assert abs(o["lse"][0] - math.log(9.0)) < tol
    assert o["counts"].tolist() == [1, 0, 1]


def test_lb_squares_uniform_and_dominant():
    """E * sum P^2 is 1 for a zero router and tends to E when one expert
    takes all the probability."""
    cfg = TCfg(T=16, d=4, E=6, k=2, f=2)
    t = rand_tensors(cfg, 44)
    t["w_router"] = np.zeros_like(t["w_router"])
    assert abs(oracle.forward(cfg, t)["lb_squares"] - 1.0) < 1e-14
    t = rand_tensors(cfg, 44, router_bias=np.array([80.0, 0, 0, 0, 0, 0]))
    assert abs(oracle.forward(cfg, t)["lb_squares"] - 6.0) < 1e-9


def test_kl_and_frequency_penalty_closed_forms():
    """Two experts, k = 1, four tokens.  Router logits [ln 3, 0] for three
    tokens and [0, ln 3] for one: P = ((3 * 3/4 + 1/4) / 4, ...) = (5/8, 3/8);
    f = (3/4, 1/4).
      kl_uniform = 1/2 ln((1/2) / (5/8)) + 1/2 ln((1/2) / (3/8))
                 = 1/2 ln(16/15)                  (up to the 1e-8 in the log)
      freq_penalty = (1/4)^2 + (1/4)^2 = 1/8."""
    cfg = TCfg(T=4, d=2, E=2, k=1, f=1)
    ln3 = math.log(3.0)
    t = {
        "x": f32([[1.0, 0.0], [1.0, 0.0], [1.0, 0.0], [0.0, 1.0]]),
        "w_router": f32([[ln3, 0.0], [0.0, ln3]]),
        "router_bias": None,
        "w1": f32(np.ones((2, 2, 2))), "w2": f32(np.ones((2, 2, 1))),
        "b1": None, "b2": None, "ws1": None, "ws2": None,
    }
    o = oracle.forward(cfg, t)
    assert o["counts"].tolist() == [3, 1]
    assert abs(o["kl_uniform"] - 0.5 * math.log(16 / 15)) < 1e-7
    assert abs(o["freq_penalty"] - 0.125) < 1e-15
    assert abs(o["lb_squares"] - 2 * ((5 / 8) ** 2 + (3 / 8) ** 2)) < 1e-7


def test_kl_uniform_special_values_and_sign():
    """Uniform P: kl = -ln(1 + E * 1e-8) (only the page's 1e-8 remains);
    otherwise kl >= that value (Gibbs' inequality), and it grows as one
    expert takes more of the probability."""
    cfg = TCfg(T=16, d=4, E=8, k=2, f=2)
    t = rand_tensors(cfg, 45)
    t["w_router"] = np.zeros_like(t["w_router"])
    o = oracle.forward(cfg, t)
    assert abs(o["kl_uniform"] - (-math.log(1 + 8e-8))) < 1e-15
    prev = o["kl_uniform"]
    for b0 in (1.0, 3.0, 6.0):
        t = rand_tensors(cfg, 45, router_bias=np.array([b0] + [0.0] * 7))
        t["w_router"] = np.zeros_like(t["w_router"])
        kl = oracle.forward(cfg, t)["kl_uniform"]
        assert kl > prev
        prev = kl
    for seed in range(3):
        o = oracle.forward(cfg, rand_tensors(cfg, 46 + seed))
        assert o["kl_uniform"] >= -math.log(1 + 8e-8) - 1e-15
        assert o["freq_penalty"] >= 0.0


def test_noise_generator_draws():
    """Router noise: float32 [T, E], std as asked, fixed by the seed."""
    cfg = get_config("c2", T=512, router_noise_std=0.5)
    a = make_inputs(cfg)["router_noise"]
    b = make_inputs(cfg)["router_noise"]
    assert a.dtype == np.float32 and a.shape == (512, cfg.E)
    assert np.array_equal(a, b)
    assert abs(float(a.std()) - 0.5) < 0.02
    assert make_inputs(get_config("c2", T=64))["router_noise"] is None


def test_frequency_penalty_with_top2():
    """f is the share of all T*k selections: two tokens choosing {0, 1} and
    {0, 2} give f = (1/2, 1/4, 1/4, 0), so the penalty is
    (1/4)^2 + 0 + 0 + (1/4)^2 = 1/8."""
    cfg = TCfg(T=2, d=2, E=4, k=2, f=1)
    t = {
        "x": f32([[1.0, 0.0], [0.0, 1.0]]),
        "w_router": f32([[3.0, 3.0], [2.0, 0.0], [0.0, 2.0], [-5.0, -5.0]]),
        "router_bias": None,
        "w1": f32(np.ones((4, 2, 2))), "w2": f32(np.ones((4, 2, 1))),
        "b1": None, "b2": None, "ws1": None, "ws2": None,
    }
    o = oracle.forward(cfg, t)
    assert o["counts"].tolist() == [2, 1, 1, 0]
    assert abs(o["freq_penalty"] - 0.125) < 1e-15


# ---------------------------------------------------------------------------
# backward pass ([P3 §4.2] loss = task + aux; [P5 §2] coefficients)


@dataclass
class BCfg(TCfg):
    weights: str = "act"


def _loss(cfg, t, dy, aux_scale, lw=None):
    o = oracle.forward(cfg, t)
    if lw is None:
        aux = aux_scale * o["weighted"]
    else:
        aux = sum(c * o[key] for key, c in lw.items())
    return float(np.sum(dy * o["y"])) + aux, o["topk_idx"]


def _stable_tensors(cfg, seed, **kw):
    """Random tensors whose k-th / (k+1)-th probability gap is wide enough
    that a 2^-10 perturbation cannot change the selection."""
    for s in range(seed, seed + 200):
        t = rand_tensors(cfg, s, **kw)
        ok = oracle.router_gap_ok(t["x"], t["w_router"], t.get("router_bias"), cfg.k, "f32",
                                  gap=0.03, temperature=cfg.router_temperature,
                                  noise=t.get("router_noise"))
        if ok.all():
            return t
    raise RuntimeError("no stable draw")


# loss weights of the aux terms: None = 2.5 * (0.01 lb + 0.001 z); else the
# load-balance forms of [P3 §3.1] / [P2 §4.2] weighted into the loss
LW_ALL = {"lb": 0.3, "z": 0.05, "lb_squares": 0.7, "kl_uniform": 0.9}

FD_CASES = [
    # act, S, bias, residual, cf, tau, noise, loss weights
    ("swiglu", 1, False, True, 0.0, 1.0, False, None),
    ("gelu", 1, True, False, 0.0, 1.5, True, None),
    ("swiglu", 2, True, False, 0.75, 0.8, True, None),
    ("swiglu", 0, False, False, 0.0, 1.2, True, LW_ALL),
]


@pytest.mark.parametrize("case", FD_CASES, ids=["swiglu_shared_res", "gelu_bias_tau_noise",
                                                "swiglu_cap_shared2", "all_lb_forms"])
def test_backward_central_differences(case):
    """Every gradient entry against a central difference of the forward loss
    sum(dy * y) + 2.5 (0.01 lb + 0.001 z) (or the weighted load-balance
    forms), step 2^-10 (exact on float32)."""
    act, S, bias, res, cf, tau, noise, lw = case
    cfg = BCfg(T=6, d=4, E=4, k=2, f=3, S=S, act=act, capacity_factor=cf, add_residual=res,
               router_temperature=tau)
    t = _stable_tensors(cfg, 60, bias=bias, router_bias=np.array([0.25, 0, -0.5, 0]))
    if bias:
        r = np.random.default_rng(11)
        t["sb1"] = f32(r.standard_normal(t["ws1"].shape[:2]) * 0.1)
        t["sb2"] = f32(r.standard_normal((S, cfg.d)) * 0.1)
    if noise:
        t["router_noise"] = f32(np.random.default_rng(7).standard_normal((cfg.T, cfg.E)) * 0.5)
        t = dict(t)
    dy = np.random.default_rng(8).standard_normal((cfg.T, cfg.d))
    aux = 2.5
    g = oracle.backward(cfg, t, dy, aux, loss_weights=lw)
    _, idx0 = _loss(cfg, t, dy, aux, lw)
    h = 2.0 ** -10
    names = [("x", "dx"), ("w_router", "dw_router"), ("router_bias", "drouter_bias"),
             ("w1", "dw1"), ("w2", "dw2"), ("ws1", "dws1"), ("ws2", "dws2")]
    if bias:
        names += [("b1", "db1"), ("b2", "db2"), ("sb1", "dsb1"), ("sb2", "dsb2")]
    checked = 0
    for src, key in names:
        a = t.get(src)
        if a is None:
            continue
        ref = g[key]
        for i in np.ndindex(a.shape):
            orig = a[i]
            a[i] = orig + np.float32(h)
            lp, ip = _loss(cfg, t, dy, aux, lw)
            a[i] = orig - np.float32(h)
            lm, im = _loss(cfg, t, dy, aux, lw)
            a[i] = orig
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - ref[i]) <= 2e-5 * (1 + abs(ref[i])), (key, i, fd, ref[i])
            checked += 1
    assert checked > 100


def _torch_layer_loss(cfg, tt, dy, aux_scale):
    """The layer written with torch float64 ops, in the loop form of the pages
    (mask / gather / run / weight / add): router, softmax, torch.topk of the
    probabilities, renormalise, capacity by token order, experts, shared
    experts, residual, and the aux terms."""
    x, wr = tt["x"], tt["w_router"]
    T, E, k = x.shape[0], cfg.E, cfg.k
    logits = x @ wr.T
    if tt.get("router_bias") is not None:
        logits = logits + tt["router_bias"]
    s = logits / cfg.router_temperature
    if tt.get("router_noise") is not None:
        s = s + tt["router_noise"]
    p = torch.softmax(s, dim=-1)
    lse = torch.logsumexp(s, dim=-1)
    topv, topi = torch.topk(p, k, dim=-1)
    w = topv / topv.sum(-1, keepdim=True)

    def ffn(xr, w1, b1, w2, b2):
        a = xr @ w1.T + (0 if b1 is None else b1)
        if cfg.act == "gelu":
            h = F.gelu(a)
        else:
            f = w1.shape[0] // 2
            h = F.silu(a[:, :f]) * a[:, f:]
        return h @ w2.T + (0 if b2 is None else b2)

    cap = oracle.capacity(cfg.capacity_factor, T, k, E)
    seen = [0] * E
    y = torch.zeros_like(x)
    for t_ in range(T):
        for j in range(k):
            e = int(topi[t_, j])
            seen[e] += 1
            if cap is not None and seen[e] > cap:
                continue
            b1 = None if tt.get("b1") is None else tt["b1"][e]
            b2 = None if tt.get("b2") is None else tt["b2"][e]
            y[t_] = y[t_] + w[t_, j] * ffn(x[t_:t_ + 1], tt["w1"][e], b1, tt["w2"][e], b2)[0]
    for si in range(cfg.S):
        sb1 = None if tt.get("sb1") is None else tt["sb1"][si]
        sb2 = None if tt.get("sb2") is None else tt["sb2"][si]
        y = y + ffn(x, tt["ws1"][si], sb1, tt["ws2"][si], sb2)
    if cfg.add_residual:
        y = y + x
    counts = torch.zeros(E, dtype=torch.float64)
    for e in topi.reshape(-1).tolist():
        counts[e] += 1
    lb = E * torch.sum(counts / (T * k) * p.mean(0))
    z = torch.mean(lse * lse)
    return torch.sum(torch.as_tensor(dy) * y) + aux_scale * (0.01 * lb + 0.001 * z)


def test_backward_matches_torch_autograd():
    cfg = BCfg(T=40, d=8, E=6, k=2, f=5, S=2, act="swiglu", capacity_factor=1.0,
               add_residual=True, router_temperature=1.5)
    t = rand_tensors(cfg, 300, bias=True, router_bias=np.linspace(-1, 1, 6))
    t["router_noise"] = f32(np.random.default_rng(9).standard_normal((cfg.T, cfg.E)) * 0.3)
    r = np.random.default_rng(11)
    t["sb1"] = f32(r.standard_normal(t["ws1"].shape[:2]) * 0.1)
    t["sb2"] = f32(r.standard_normal((cfg.S, cfg.d)) * 0.1)
    dy = np.random.default_rng(10).standard_normal((cfg.T, cfg.d))
    g = oracle.backward(cfg, t, dy, 4.0)
    assert g["dw1"].shape == (6, 10, 8)
    keys = {"x": "dx", "w_router": "dw_router", "router_bias": "drouter_bias", "w1": "dw1",
            "b1": "db1", "w2": "dw2", "b2": "db2", "ws1": "dws1", "sb1": "dsb1", "ws2": "dws2",
            "sb2": "dsb2"}
    tt = {}
    for name in list(keys) + ["router_noise"]:
        if t.get(name) is not None:
            tt[name] = torch.tensor(np.asarray(t[name], np.float64), requires_grad=name in keys)
    loss = _torch_layer_loss(cfg, tt, dy, 4.0)
    loss.backward()
    for name, key in keys.items():
        ref = tt[name].grad.numpy()
        assert np.allclose(g[key], ref, rtol=1e-10, atol=1e-12), key


# ---------------------------------------------------------------------------
# the input acceptance rule (gap of at least 1e-4 between the k-th and the
# (k+1)-th router probability of every token), pinned by closed forms.
# [P3 §3.1] and [P4 §3.1] route by softmax and then take the k largest
# probabilities; the rule only keeps that choice away from near-ties.  Each
# token below has probabilities q chosen by hand: its logits are ln q (the
# router is the identity map, float32), so p = q to float32 rounding
# (absolute error < 1e-7, far inside the 2e-6 margins used here).

def _gap_token(q, k, temperature=1.0, noise=None, bias=None):
    """router_gap_ok on one token whose probabilities are q (identity router)."""
    q = np.asarray(q, dtype=np.float64)
    E = q.size
    x = f32(np.log(q))[None, :]
    w = f32(np.eye(E))
    n = None if noise is None else f32(noise)[None, :]
    b = None if bias is None else f32(bias)
    return bool(oracle.router_gap_ok(x, w, b, k, "f32", temperature=temperature, noise=n)[0])


def _q_k2(g):
    """Five experts; the 2nd and 3rd probabilities differ by g (the 1st/2nd
    and 3rd/4th gaps are about 0.1 and 0.15)."""
    return [0.35, 0.25 + g / 2, 0.25 - g / 2, 0.1, 0.05]


def _q_k1(g):
    """Five experts; the 1st and 2nd probabilities differ by g."""
    return [0.3 + g / 2, 0.3 - g / 2, 0.2, 0.15, 0.05]


@pytest.mark.parametrize("below", [True, False])
def test_gap_rule_threshold_k2(below):
    """k = 2: the gap that matters is p_(2) - p_(3).  Just below 1e-4 the
    token is rejected, just above it accepted.  A rule that compared the
    3rd and 4th probabilities (an index off by one) would accept both; one
    that took the gap on logits (ln(0.25 + g/2) - ln(0.25 - g/2) ~ 4 g)
    would accept the first."""
    g = 1e-4 - 2e-6 if below else 1e-4 + 2e-6
    assert _gap_token(_q_k2(g), 2) is (not below)


@pytest.mark.parametrize("below", [True, False])
def test_gap_rule_threshold_k1(below):
    """k = 1: the gap that matters is p_(1) - p_(2); the same token passes
    with k = 2, whose gap (about 0.1) is far above the threshold."""
    g = 1e-4 - 2e-6 if below else 1e-4 + 2e-6
    assert _gap_token(_q_k1(g), 1) is (not below)
    assert _gap_token(_q_k1(g), 2)


def test_gap_rule_other_gaps_do_not_count():
    """A near-tie away from the k-th / (k+1)-th pair does not reject: q with
    p_(1) = p_(2) exactly passes at k = 2 (gap p_(2) - p_(3) = 0.1), and
    fails at k = 1."""
    q = [0.3, 0.3, 0.2, 0.15, 0.05]
    assert _gap_token(q, 2)
    assert not _gap_token(q, 1)
    assert _gap_token(q, 3)          # p_(3) - p_(4) = 0.05


def test_gap_rule_k_equals_E_always_accepts():
    """k = E has no (k+1)-th expert: every token passes, a uniform one (all
    gaps zero) included; the same uniform token fails for every k < E."""
    E = 4
    q = [0.25] * E
    assert _gap_token(q, E)
    for k in range(1, E):
        assert not _gap_token(q, k)


def test_gap_rule_sorts_the_probabilities():
    """The rule ranks the probabilities, not the expert indices: the k = 2
    token of the threshold test with its experts listed in reverse order is
    judged the same way."""
    for g, ok in ((1e-4 - 2e-6, False), (1e-4 + 2e-6, True)):
        assert _gap_token(_q_k2(g)[::-1], 2) is ok


def test_gap_rule_temperature_moves_the_gap():
    """Temperature tau = 1/2 squares the unnormalised probabilities: with q
    of the k = 2 token, the new gap is ((0.25 + g/2)^2 - (0.25 - g/2)^2) /
    sum q^2 = 0.5 g / (0.26 + g^2 / 2), about 1.92 g.  g = 0.6e-4 fails at
    tau = 1 and passes at tau = 1/2 (1.15e-4); g = 1.2e-4 passes at tau = 1
    and fails at tau = 2, where the gap is (sqrt(q2) - sqrt(q3)) / sum sqrt(q),
    about 0.56e-4."""
    g = 0.6e-4
    q = np.array(_q_k2(g))
    sharp = 0.5 * g / float(np.sum(q ** 2))
    assert sharp > 1.1e-4
    assert not _gap_token(q, 2)
    assert _gap_token(q, 2, temperature=0.5)
    g = 1.2e-4
    q = np.array(_q_k2(g))
    flat = (math.sqrt(q[1]) - math.sqrt(q[2])) / float(np.sum(np.sqrt(q)))
    assert flat < 0.9e-4
    assert _gap_token(q, 2)
    assert not _gap_token(q, 2, temperature=2.0)


def test_gap_rule_noise_moves_the_gap():
    """Noise n added to an expert's score multiplies its unnormalised
    probability by e^n.  With q of the k = 2 token at g = 0.5e-4 (rejected)
    and e^n = 1 + delta on the 2nd expert, delta = (2e-4 - g) / ((0.25 +
    g/2)(1 - 2e-4)), the gap becomes exactly 2e-4 and the token passes.
    Lifting the 3rd expert instead by 1 + delta3, delta3 = (g + 0.5e-4) /
    (0.25 - g/2), makes it the 2nd largest, 0.5e-4 above the old 2nd before
    normalisation (Z = 1 + g + 0.5e-4): still a near-tie, rejected."""
    g = 0.5e-4
    q = _q_k2(g)
    delta = (2e-4 - g) / ((0.25 + g / 2) * (1 - 2e-4))
    assert not _gap_token(q, 2)
    assert _gap_token(q, 2, noise=[0.0, math.log1p(delta), 0.0, 0.0, 0.0])
    delta3 = (g + 0.5e-4) / (0.25 - g / 2)
    swapped = 0.5e-4 / (1 + g + 0.5e-4)
    assert 0.4e-4 < swapped < 0.6e-4
    assert not _gap_token(q, 2, noise=[0.0, 0.0, math.log1p(delta3), 0.0, 0.0])
    # the same lift on the 4th expert leaves the 2nd / 3rd pair alone
    assert not _gap_token(q, 2, noise=[0.0, 0.0, 0.0, math.log1p(delta3), 0.0])


def test_gap_rule_bias_enters_before_the_softmax():
    """A router bias is part of the logits: x = 0 with bias ln q gives the
    same probabilities as x = ln q, so the threshold token is judged the
    same way through the bias."""
    for g, ok in ((1e-4 - 2e-6, False), (1e-4 + 2e-6, True)):
        q = np.array(_q_k2(g))
        E = q.size
        x = f32(np.zeros((1, E)))
        w = f32(np.eye(E))
        got = bool(oracle.router_gap_ok(x, w, f32(np.log(q)), 2, "f32")[0])
        assert got is ok
