"""Seeded synthetic inputs for the MoE layer, shared by the GPU path's tests
and benchmark and by the CPU oracle.

This module holds no arithmetic of the layer itself: it draws numbers, rounds
them to the storage type and hands them out.  The one input rule that depends
on the layer (the top-k probability gap) is evaluated by a caller-supplied
`accept` callback; rejected token rows are redrawn from their own sub-stream.

Streams: every tensor (and, for expert weights, every expert) has its own
numpy PCG64 stream seeded with SeedSequence([seed, tag, index]), so any
expert's weights can be regenerated on demand without materialising the
whole stack (the decode-shaped layer holds 22.6 GB of expert weights).

Storage: "f32" tensors are float32 arrays; "bf16" tensors are uint16 arrays
holding bfloat16 bit patterns, rounded from float32 draws with
round-to-nearest-even.  Layers with 8-bit expert weights get int8 code
arrays (a standard normal draw times 127/4, rounded and clipped to
[-127, 127]) and one float32 scale per weight row (0.02 * 4 / 127 times a
factor drawn uniformly from [0.75, 1.25]), so that scale * code has about
the 0.02 standard deviation of the other layers' weights.  These are drawn
as given, already-quantized weights.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "get_config", "f32_to_bf16_bits", "Bank",
           "make_inputs", "TAGS"]

TAGS = {
    "x": 1, "w_router": 2, "w1": 3, "b1": 4, "w2": 5, "b2": 6,
    "ws1": 7, "sb1": 8, "ws2": 9, "sb2": 10, "x_redraw": 11,
    "w1_scale": 12, "w2_scale": 13, "ws1_scale": 14, "ws2_scale": 15, "router_noise": 16,
}
X_ROW_BLOCK = 4096          # rows of x per sub-stream
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerConfig:
    """Shape and options of one MoE layer workload."""
    name: str
    T: int                    # tokens (batch * seq)
    d: int                    # d_model
    E: int                    # routed experts
    k: int                    # top-k
    f: int                    # expert d_ffn
    S: int = 0                # shared experts (SwiGLU/GELU of width f, weight 1)
    dtype: str = "bf16"       # "bf16" or "f32"
    act: str = "swiglu"       # "swiglu" or "gelu"
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    router_bias: str = "none"      # "none" or "zipf": b_i = 2 ln(1/(i+1))
    expert_bias: str = "none"      # "none", "zero" or "random"
    add_residual: bool = False
    seed: int = 0
    weights: str = "act"      # expert weights: "act" (activation dtype) or "int8" (codes + row scales)
    router_temperature: float = 1.0   # tau of the router scores
    router_noise_std: float = 0.0     # > 0: Gaussian noise [T, E] of this std added to the scores

    @property
    def w1_rows(self) -> int:
        return 2 * self.f if self.act == "swiglu" else self.f


CONFIGS = {
    # tiny fp32 layer with GELU experts and (zero) biases
    "c1": LayerConfig("tiny_f32_gelu", T=512, d=64, E=8, k=2, f=256, dtype="f32",
                      act="gelu", expert_bias="zero", seed=1001),
    # small "Flash" layer, capacity factor 1.25
    "c2": LayerConfig("flash_bf16_T4096_d512_E16_k2_f1024_cf1.25", T=4096, d=512, E=16,
                      k=2, f=1024, capacity_factor=1.25, seed=1002),
    # FLAME-shaped layer: 64 routed top-6 + 2 shared
    "c3": LayerConfig("flame_bf16_T16384_d1024_E64_k6_S2_f512", T=16384, d=1024, E=64,
                      k=6, f=512, S=2, seed=1003),
    # skewed routing (fixed Zipf-like logit bias), no capacity limit
    "c4": LayerConfig("skew_bf16_T65536_d2048_E64_k6_S2_f1408", T=65536, d=2048, E=64,
                      k=6, f=1408, S=2, router_bias="zipf", seed=1004),
    # same, capacity factor 1.0
    "c4cap": LayerConfig("skew_bf16_T65536_d2048_E64_k6_S2_f1408_cf1.0", T=65536, d=2048,
                         E=64, k=6, f=1408, S=2, router_bias="zipf", capacity_factor=1.0,
                         seed=1004),
    # decode-shaped, weight-streaming layer
    "c5": LayerConfig("decode_bf16_T128_d7168_E256_k8_S1_f2048", T=128, d=7168, E=256,
                      k=8, f=2048, S=1, seed=1005),
    # the same layer with 8-bit expert weights (row-scaled INT8 codes)
    "c5q": LayerConfig("decode_int8w_T128_d7168_E256_k8_S1_f2048", T=128, d=7168, E=256,
                       k=8, f=2048, S=1, weights="int8", seed=1006),
    # the "Flash" layer with router temperature 1.5 and Gaussian router noise (std 1)
    "c2n": LayerConfig("flash_bf16_T4096_d512_E16_k2_f1024_cf1.25_tau1.5_noise1", T=4096, d=512,
                       E=16, k=2, f=1024, capacity_factor=1.25, router_temperature=1.5,
                       router_noise_std=1.0, seed=1007),
}


def get_config(name: str, **overrides) -> LayerConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, tag: str, *index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAGS[tag], *index])))


def _store(z32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(z32) if dtype == "bf16" else z32.astype(np.float32)


class Bank:
    """Lazily generated stack of per-expert tensors, [n, *shape].

    bank[e] draws expert e's tensor from its own stream; array() builds the
    whole stack.  Values: N(0, std^2) rounded to the storage dtype, or zeros;
    dtype "int8": codes rint(N(0, 1) * 127 / 4) clipped to [-127, 127];
    dtype "scale": float32 std * 4 / 127 * U(0.75, 1.25) (one per row).
    """

    def __init__(self, seed: int, tag: str, n: int, shape, dtype: str, std: float, zero=False):
        self.seed, self.tag, self.n = seed, tag, n
        self.shape = tuple(shape)
        self.dtype, self.std, self.zero = dtype, std, zero

    @property
    def np_dtype(self):
        return {"bf16": np.uint16, "int8": np.int8}.get(self.dtype, np.float32)

    @property
    def full_shape(self):
        return (self.n,) + self.shape

    @property
    def nbytes(self) -> int:
        return self.n * int(np.prod(self.shape)) * np.dtype(self.np_dtype).itemsize

    def __len__(self) -> int:
        return self.n

    def __getitem__(self, e: int) -> np.ndarray:
        if not 0 <= e < self.n:
            raise IndexError(e)
        if self.zero:
            return np.zeros(self.shape, dtype=self.np_dtype)
        if self.dtype == "scale":
            u = _rng(self.seed, self.tag, e).uniform(0.75, 1.25, self.shape).astype(np.float32)
            return u * np.float32(self.std * 4.0 / 127.0)
        z = _rng(self.seed, self.tag, e).standard_normal(self.shape, dtype=np.float32)
        if self.dtype == "int8":
            return np.clip(np.rint(z * np.float32(127.0 / 4.0)), -127, 127).astype(np.int8)
        z *= np.float32(self.std)
        return _store(z, self.dtype)

    def array(self, threads: int | None = None) -> np.ndarray:
        out = np.empty(self.full_shape, dtype=self.np_dtype)

        def fill(e):
            out[e] = self[e]

        _parallel(fill, range(self.n), threads)
        return out


def _parallel(fn, items, threads=None):
    items = list(items)
    n = threads or min(16, len(os.sched_getaffinity(0)))
    if n <= 1 or len(items) <= 1:
        for i in items:
            fn(i)
        return
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fn, items))


def _draw_x_rows(cfg: LayerConfig) -> np.ndarray:
    T, d = cfg.T, cfg.d
    x = np.empty((T, d), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    nblk = (T + X_ROW_BLOCK - 1) // X_ROW_BLOCK

    def fill(b):
        r0, r1 = b * X_ROW_BLOCK, min(T, (b + 1) * X_ROW_BLOCK)
        z = _rng(cfg.seed, "x", b).standard_normal((r1 - r0, d), dtype=np.float32)
        x[r0:r1] = _store(z, cfg.dtype)

    _parallel(fill, range(nblk))
    return x


def router_bias_values(cfg: LayerConfig):
    """Fixed per-expert router logit bias (float32) or None.

    "zipf": b_i = 2 ln(1/(i+1)), a fixed input of the skewed-routing workload.
    """
    if cfg.router_bias == "none":
        return None
    if cfg.router_bias == "zipf":
        return np.array([2.0 * math.log(1.0 / (i + 1)) for i in range(cfg.E)], dtype=np.float32)
    raise ValueError(cfg.router_bias)


def make_inputs(cfg: LayerConfig, accept=None, max_redraws: int = 64, materialize: bool = True):
    """All inputs of one layer workload.

    accept(x, w_router, router_bias, noise) -> bool[T] marks acceptable token
    rows (noise: the router noise rows of the same tokens, or None); each
    rejected row t is redrawn from stream (seed, "x_redraw", t, attempt)
    until accepted (its noise row stays).  Returns a dict; expert weight
    stacks are numpy arrays if `materialize`, else lazy `Bank`s.

    Router noise (router_noise_std > 0): float32 std * N(0, 1) [T, E] from
    stream (seed, "router_noise", 0).
    """
    dt = cfg.dtype
    x = _draw_x_rows(cfg)
    w_router = Bank(cfg.seed, "w_router", 1, (cfg.E, cfg.d), dt, WEIGHT_STD)[0]
    rbias = router_bias_values(cfg)
    noise = None
    if cfg.router_noise_std > 0:
        z = _rng(cfg.seed, "router_noise", 0).standard_normal((cfg.T, cfg.E), dtype=np.float32)
        noise = (z * np.float32(cfg.router_noise_std)).astype(np.float32)
    redrawn = set()
    if accept is not None:
        ok = np.asarray(accept(x, w_router, rbias, noise), dtype=bool)
        attempt = 0
        while not ok.all():
            if attempt >= max_redraws:
                raise RuntimeError(f"{cfg.name}: {int((~ok).sum())} rows still rejected "
                                   f"after {max_redraws} redraws")
            bad = np.nonzero(~ok)[0]
            for t in bad:
                z = _rng(cfg.seed, "x_redraw", int(t), attempt).standard_normal(cfg.d, dtype=np.float32)
                x[t] = _store(z, dt)
            redrawn.update(int(t) for t in bad)
            ok[bad] = np.asarray(accept(x[bad], w_router, rbias, None if noise is None else noise[bad]),
                                 dtype=bool)
            attempt += 1

    bias_zero = cfg.expert_bias == "zero"
    has_bias = cfg.expert_bias in ("zero", "random")
    E, S, d, f = cfg.E, cfg.S, cfg.d, cfg.f
    q8 = cfg.weights == "int8"
    wdt = "int8" if q8 else dt
    banks = {
        "w1": Bank(cfg.seed, "w1", E, (cfg.w1_rows, d), wdt, WEIGHT_STD),
        "w2": Bank(cfg.seed, "w2", E, (d, f), wdt, WEIGHT_STD),
        "b1": Bank(cfg.seed, "b1", E, (cfg.w1_rows,), dt, WEIGHT_STD, zero=bias_zero) if has_bias else None,
        "b2": Bank(cfg.seed, "b2", E, (d,), dt, WEIGHT_STD, zero=bias_zero) if has_bias else None,
        "ws1": Bank(cfg.seed, "ws1", S, (cfg.w1_rows, d), wdt, WEIGHT_STD) if S else None,
        "ws2": Bank(cfg.seed, "ws2", S, (d, f), wdt, WEIGHT_STD) if S else None,
        "sb1": Bank(cfg.seed, "sb1", S, (cfg.w1_rows,), dt, WEIGHT_STD, zero=bias_zero) if (S and has_bias) else None,
        "sb2": Bank(cfg.seed, "sb2", S, (d,), dt, WEIGHT_STD, zero=bias_zero) if (S and has_bias) else None,
    }
    if cfg.weights not in ("act", "int8"):
        raise ValueError(cfg.weights)
    if q8:  # one float32 scale per weight row
        banks["w1_scale"] = Bank(cfg.seed, "w1_scale", E, (cfg.w1_rows,), "scale", WEIGHT_STD)
        banks["w2_scale"] = Bank(cfg.seed, "w2_scale", E, (d,), "scale", WEIGHT_STD)
        banks["ws1_scale"] = Bank(cfg.seed, "ws1_scale", S, (cfg.w1_rows,), "scale", WEIGHT_STD) if S else None
        banks["ws2_scale"] = Bank(cfg.seed, "ws2_scale", S, (d,), "scale", WEIGHT_STD) if S else None
    out = {"x": x, "w_router": w_router, "router_bias": rbias, "router_noise": noise,
           "n_redrawn": len(redrawn)}
    for key, bank in banks.items():
        out[key] = None if bank is None else (bank.array() if materialize else bank)
    return out
