"""The seeded input generator: determinism, bf16 rounding, the tie-gap rule
and the skewed-routing workload's hot expert.  CPU only."""

import numpy as np
import pytest

import oracle
from moe_inputs import Bank, CONFIGS, f32_to_bf16_bits, get_config, make_inputs


def test_bf16_round_to_nearest_even():
    u = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0xBF80FFFF, 0x3F7FFFFF],
                 dtype=np.uint32)
    got = f32_to_bf16_bits(u.view(np.float32))
    # exact, tie->even(down), tie->even(up), above tie, carry into exponent, carry
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF81, 0x3F80]


def test_deterministic_and_streams_independent():
    cfg = get_config("c2", T=64)
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for key in ("x", "w_router", "w1", "w2"):
        assert np.array_equal(a[key], b[key])
    bank = Bank(cfg.seed, "w1", cfg.E, (2 * cfg.f, cfg.d), "bf16", 0.02)
    assert np.array_equal(bank[3], a["w1"][3])
    assert not np.array_equal(bank[3], bank[4])


def test_value_distribution():
    cfg = get_config("c2", T=512)
    t = make_inputs(cfg)
    x = oracle.decode(t["x"], "bf16")
    w = oracle.decode(t["w1"][0], "bf16")
    assert abs(x.std() - 1.0) < 0.02 and abs(x.mean()) < 0.02
    assert abs(w.std() - 0.02) < 0.001


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_gap_rule_holds_after_redraw(name):
    cfg = CONFIGS[name]
    if cfg.T > 4096:
        cfg = get_config(name, T=4096)
    acc = lambda x, w, b, n: oracle.router_gap_ok(x, w, b, cfg.k, cfg.dtype, noise=n)
    t = make_inputs(cfg, accept=acc)
    assert acc(t["x"], t["w_router"], t["router_bias"], t["router_noise"]).all()
    assert t["n_redrawn"] > 0          # the rule is active on these shapes


def test_skewed_bias_hot_expert():
    """Zipf-like bias b_i = 2 ln(1/(i+1)): the hottest expert is picked by more
    than 30 % of the tokens (top-6 picks distinct experts, so a share of the
    T*k assignments can never exceed 1/6; the tokens reading is used)."""
    cfg = get_config("c4", T=4096)
    t = make_inputs(cfg)
    assert t["router_bias"][0] == 0.0
    assert np.isclose(t["router_bias"][9], 2 * np.log(0.1), rtol=1e-6)
    xd, wr = oracle.decode(t["x"], "bf16"), oracle.decode(t["w_router"], "bf16")
    p, _ = oracle.softmax_lse(oracle.router_logits(xd, wr, t["router_bias"].astype(np.float64)))
    idx = oracle.topk_select(p, cfg.k)
    counts = oracle.expert_counts(idx, cfg.E)
    assert counts.max() / cfg.T > 0.30
