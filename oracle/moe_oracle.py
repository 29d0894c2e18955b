"""Plain CPU oracle of the forward pass of a top-k routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the test-suite, the package smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (own
bf16 decoding, own loops, own reductions) and imports nothing from it.

Everything is computed in float64 from the stored input values (float32, or
bfloat16 bit patterns decoded exactly), with no intermediate rounding.  The
structure deliberately follows the pages' reference loops (one expert at a
time, gather, run the FFN, weight, add back) rather than anything fast.

Sources (web pages; sections as printed on each page):
  [P1] "Naive-N0.5-Flash" open-source MoE blog, wzjinhao.cn/news/74695
  [P2] "The quietly activated expert group" MoE explainer, mqxn.cn/news/15586
  [P3] "Small MoE language model from scratch" tutorial, lshu.cn/news/325687
  [P4] "OpenMythos" re-implementation blog, lpnh.cn/news/1735864
  [P5] FLAME-MoE research-platform summary,
       lsdiaocha.cn/2025/0530/3166997.shtml

Readings taken where the pages are silent or disagree (each is also listed in
the design notes):
  * top-k ties: lower expert index first; outputs sorted by descending
    probability (torch.topk order in [P2 §4.1], [P3 §3.1]).
  * capacity C = ceil(cf * T * k / E) evaluated exactly on the binary64 value
    of cf ([P4 §3.1] gives cf * tokens / E, i.e. the k = 1 case).
  * overflow: within an expert, assignments are kept first-come in ascending
    token order; a dropped assignment contributes exactly zero and the kept
    weights are not renormalised ([P1 §2.2], [P4 §3.1]).
  * f_i of the load-balance loss is the pre-capacity share of the T*k
    assignments; P_i is the mean over all tokens of the full softmax
    ([P4 §3.1]).  z-loss = mean over tokens of logsumexp(logits)^2 ([P5 §2]
    names the loss; the squared-lse form is the standard router z-loss).
  * SwiGLU: h = silu(x W_gate^T) * (x W_up^T), then W_down; GELU is the exact
    erf form; dropout is the identity at inference ([P2 §3.1], [P3 §3.1]).
  * shared experts have weight 1 and sit outside the router ([P4 §2.1],
    [P5 §2]).  The residual x is added only when asked ([P2 §4.1] adds it
    inside the layer, [P3 §3.2] outside).
  * 8-bit expert weights ([P3 §6] suggests compressing each expert's
    weights to INT8 for deployment, with no scheme given): symmetric INT8
    codes q with one float32 scale per weight row, W[n, :] = scale[n] *
    q[n, :] (the row is an output channel of W1 and of W2).
  * router temperature and noise ([P2 §5.1], [P2 §2.2]): the scores are
    logits / tau + noise, tau dividing the router output with its bias and
    the caller's noise added after; everything downstream uses the scores.
  * backward ([P3 §4.2] trains on loss = task + aux; [P5 §2] coefficients
    0.01 / 0.001): the gradient of sum(dy * y) + aux_scale * (0.01 lb +
    0.001 z); top-k selection, capacity drops and the shares f_e carry no
    gradient (they are piecewise constant).
  * the other load-balance forms ([P3 §3.1] E * sum P^2; [P2 §4.2] KL of
    the uniform distribution from P, with 1e-8 in the logarithm, plus the
    squared distance of the hard frequencies from 1/E) use the same P and f
    as the main one and are reported unweighted.

Parity pins: every function below is exercised by the CPU tests against
closed forms, brute force or an independently written dense computation; the
one convention with no external pin (the f_i normalisation) is marked
"parity unpinned beyond the convention" at `aux_losses`.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "decode",
    "dequantize_int8",
    "expert_weight",
    "router_logits",
    "router_scores",
    "softmax_lse",
    "topk_select",
    "renormalise",
    "expert_counts",
    "capacity",
    "dispatch",
    "expert_ffn",
    "shared_ffn",
    "combine",
    "aux_losses",
    "router_gap_ok",
    "forward",
    "expert_ffn_backward",
    "backward",
]


# ---------------------------------------------------------------------------
# input decoding


def decode(a, dtype: str) -> np.ndarray:
    """Stored tensor -> float64.

    dtype "bf16": `a` holds bfloat16 bit patterns as uint16; the value is the
    float32 whose upper 16 bits are those bits (exact).  dtype "f32": `a` is
    float32.  Either way the result is exact in float64.
    """
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 tensors are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 tensors are passed as float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def dequantize_int8(q, scale) -> np.ndarray:
    """INT8 weight codes with one scale per row -> float64 ([P3 §6]: expert
    weights compressed to INT8).

    q: int8 [rows, cols]; scale: float32 [rows].  W[n, c] = scale[n] * q[n, c],
    exact in float64 (an 8-bit integer times a float32).
    """
    q = np.asarray(q)
    scale = np.asarray(scale)
    if q.dtype != np.int8:
        raise TypeError("INT8 weight codes are passed as int8")
    if scale.dtype != np.float32:
        raise TypeError("INT8 weight scales are passed as float32")
    if q.ndim != 2 or scale.shape != (q.shape[0],):
        raise ValueError("one scale per row of the code matrix")
    return scale.astype(np.float64)[:, None] * q.astype(np.float64)


def expert_weight(t, name: str, i: int, dtype: str, weights: str = "act") -> np.ndarray:
    """Weight matrix `name` ("w1", "w2", "ws1", "ws2") of expert i as float64:
    decoded from the activation dtype, or dequantized from INT8 codes with
    the row scales t[name + "_scale"][i]."""
    if weights == "int8":
        return dequantize_int8(t[name][i], t[name + "_scale"][i])
    if weights != "act":
        raise ValueError(f"unknown weight format {weights!r}")
    return decode(t[name][i], dtype)


# ---------------------------------------------------------------------------
# routing: [P2 §3.2] (router is one linear layer), [P3 §3.1] steps 1-2,
# [P4 §3.1] "routing and top-k selection"


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] * W_r[e, c] (+ b[e]).

    W_r uses the nn.Linear [out, in] layout, [E, d] ([P3 §3.1], bias-free
    router).  The optional per-expert bias is added to the logits before the
    softmax.
    """
    logits = x @ w_router.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def router_scores(logits: np.ndarray, temperature: float = 1.0, noise=None) -> np.ndarray:
    """The scores the softmax and the top-k see: s[t, e] = l[t, e] / tau + n[t, e].

    [P2 §5.1] (troubleshooting table) scales the router logits by a
    temperature, l / tau with tau = 1 by default, to soften a router whose
    top-1 share is too high; [P2 §2.2] (and the routing noise of [P3 §6])
    adds a controllable random perturbation to the scores before the top-k.
    Reading: tau divides the router's output, bias included, the noise is
    added after it, and the probabilities, weights, lse and the statistics
    all use s.  The noise n [T, E] is an input drawn by the caller.
    """
    s = np.asarray(logits, dtype=np.float64)
    if temperature != 1.0:
        s = s / float(temperature)
    if noise is not None:
        s = s + np.asarray(noise, dtype=np.float32).astype(np.float64)
    return s


def softmax_lse(logits: np.ndarray):
    """Softmax over experts and the per-token log-sum-exp.

    m = max_e l, Z = sum_e exp(l - m), p = exp(l - m) / Z, lse = m + ln Z.
    """
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    z = ex.sum(axis=1, keepdims=True)
    p = ex / z
    lse = (m + np.log(z))[:, 0]
    return p, lse


def topk_select(p: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest probabilities per token.

    Ordered by descending probability; equal probabilities keep ascending
    expert index (stable sort of -p).  [P3 §3.1] / [P4 §3.1] take torch.topk
    of the softmax output.
    """
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalise(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] ([P3 §3.1] step 2)."""
    sel = np.take_along_axis(p, idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def router_gap_ok(x, w_router, bias, k: int, dtype: str, gap: float = 1e-4,
                  temperature: float = 1.0, noise=None) -> np.ndarray:
    """Input acceptance rule: p_(k) - p_(k+1) >= gap for every token.

    [P3 §3.1] and [P4 §3.1] route by a softmax over the router's scores and
    keep the k largest probabilities; this rule keeps generated tokens away
    from near-ties of the k-th and (k+1)-th probability, so that the chosen
    set is unambiguous.  Evaluated in float64 on the stored (rounded)
    values, with the router's bias, temperature and noise rows (of the same
    tokens) applied.  With k == E there is no (k+1)-th expert and every
    token is accepted.  Used by the input generator through a callback.
    Pinned by closed-form tokens on both sides of the threshold (k = 1, 2,
    E; temperature, noise and bias moving the gap).
    """
    xd = decode(x, dtype)
    wr = decode(w_router, dtype)
    p, _ = softmax_lse(router_scores(router_logits(xd, wr, bias), temperature, noise))
    E = p.shape[1]
    if k >= E:
        return np.ones(p.shape[0], dtype=bool)
    srt = -np.sort(-p, axis=1)
    return (srt[:, k - 1] - srt[:, k]) >= gap


# ---------------------------------------------------------------------------
# counts, capacity, dispatch: [P2 §4.1] (expert_counts buffer),
# [P4 §3.1] "capacity factor and overflow handling" and the flatten/reorder
# description that follows its pseudo-code, [P1 §2.2] (expert capacity)


def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """counts[e] = number of (t, j) with idx[t, j] == e (before capacity)."""
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[e] += 1
    return counts


def capacity(capacity_factor: float, n_tokens: int, top_k: int, n_experts: int):
    """C = ceil(cf * T * k / E) in exact rational arithmetic, None = no limit.

    cf <= 0 means no limit.  cf is taken at its exact binary64 value.
    """
    if capacity_factor is None or not (capacity_factor > 0):
        if capacity_factor is not None and math.isnan(capacity_factor):
            raise ValueError("capacity factor is NaN")
        return None
    c = Fraction(float(capacity_factor)) * n_tokens * top_k / n_experts
    return int(math.ceil(c))


def dispatch(idx: np.ndarray, n_experts: int, cap):
    """Stable expert-contiguous permutation with capacity drops.

    For each expert e, the tokens routed to it in ascending token order; the
    first min(count, C) are kept.  Kept rows are ordered by (e, t).
    Returns (offsets[E+1], perm_token[R], perm_slot[R], inv_row[T, k] with -1
    for dropped assignments, n_dropped).
    """
    T, k = idx.shape
    lists = [[] for _ in range(n_experts)]
    for t in range(T):
        for j in range(k):
            lists[int(idx[t, j])].append((t, j))
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    perm_token, perm_slot = [], []
    inv_row = np.full((T, k), -1, dtype=np.int64)
    n_dropped = 0
    row = 0
    for e in range(n_experts):
        assigned = lists[e]  # already in ascending t (outer loop over t)
        kept = assigned if cap is None else assigned[:cap]
        n_dropped += len(assigned) - len(kept)
        for (t, j) in kept:
            perm_token.append(t)
            perm_slot.append(j)
            inv_row[t, j] = row
            row += 1
        offsets[e + 1] = row
    return (offsets, np.array(perm_token, dtype=np.int64),
            np.array(perm_slot, dtype=np.int64), inv_row, n_dropped)


# ---------------------------------------------------------------------------
# expert FFNs: [P2 §3.1] (two linear maps and a SwiGLU-type non-linearity),
# [P3 §3.1] (Linear + GELU + Dropout + Linear with biases)


def _gelu(z):
    """Exact GELU: z/2 * (1 + erf(z / sqrt 2)), elementwise via math.erf."""
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def _silu(z):
    """SiLU: z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows: np.ndarray, w1: np.ndarray, b1, w2: np.ndarray, b2, act: str) -> np.ndarray:
    """One expert on a block of rows (all float64).

    GELU:   h = gelu(x W1^T + b1);          out = h W2^T + b2
            W1 [f, d], W2 [d, f].
    SwiGLU: g = x W1[:f]^T, u = x W1[f:]^T;  h = silu(g) * u;  out = h W2^T
            W1 [2f, d] holds the gate rows then the up rows; optional biases
            b1 [2f] and b2 [d] are added the same way.
    """
    if act == "gelu":
        z = x_rows @ w1.T
        if b1 is not None:
            z = z + b1[None, :]
        h = _gelu(z)
    elif act == "swiglu":
        f = w1.shape[0] // 2
        g = x_rows @ w1[:f].T
        u = x_rows @ w1[f:].T
        if b1 is not None:
            g = g + b1[None, :f]
            u = u + b1[None, f:]
        h = _silu(g) * u
    else:
        raise ValueError(f"unknown activation {act!r}")
    out = h @ w2.T
    if b2 is not None:
        out = out + b2[None, :]
    return out


def shared_ffn(x: np.ndarray, ws1, sb1, ws2, sb2, n_shared: int, act: str, dtype: str,
               weights: str = "act", ws1_scale=None, ws2_scale=None) -> np.ndarray:
    """Sum of the always-active shared experts, each with weight 1 ([P4 §2.1],
    [P5 §2]).  weights "int8": ws1 / ws2 hold INT8 codes with row scales."""
    t = {"ws1": ws1, "ws2": ws2, "ws1_scale": ws1_scale, "ws2_scale": ws2_scale}
    out = np.zeros_like(x)
    for s in range(n_shared):
        out += expert_ffn(
            x, expert_weight(t, "ws1", s, dtype, weights), None if sb1 is None else decode(sb1[s], dtype),
            expert_weight(t, "ws2", s, dtype, weights), None if sb2 is None else decode(sb2[s], dtype), act)
    return out


def combine(routed: np.ndarray, shared, residual) -> np.ndarray:
    """y = shared + sum of weighted routed outputs (+ x when asked).

    `routed` already holds sum_j w[t, j] * o(t, idx[t, j]) over kept
    assignments ([P1 §2.1] weighted sum; [P5 §2] weights are the normalised
    routing scores; [P2 §4.1] optional residual).
    """
    y = routed.copy()
    if shared is not None:
        y = y + shared
    if residual is not None:
        y = y + residual
    return y


# ---------------------------------------------------------------------------
# auxiliary statistics: [P4 §3.1] load-balance loss alpha * E * sum f_i P_i,
# [P5 §2] router z-loss and the 0.01 / 0.001 coefficients; the two other
# load-balance forms the pages give: [P3 §3.1] E * sum P_i^2 and [P2 §4.2]
# KL(uniform || P) plus a penalty on the hard frequencies


def aux_losses(p: np.ndarray, lse: np.ndarray, counts: np.ndarray, top_k: int):
    """lb = E * sum_e f_e P_e, z = mean_t lse_t^2, weighted = 0.01 lb + 0.001 z.

    f_e = counts_e / (T k) with pre-capacity counts, so sum f = 1 and lb = 1
    under uniform routing; P_e = mean_t p[t, e] over the full softmax.
    The f_e normalisation is a convention: parity unpinned beyond the
    convention.

    Also, unweighted (the pages' coefficients are the caller's):
      lb_squares   = E * sum_e P_e^2                          ([P3 §3.1] code)
      kl_uniform   = sum_e (1/E) (ln(1/E) - ln(P_e + 1e-8))   ([P2 §4.2]: the KL
                     divergence of the uniform distribution from P, with the
                     page's 1e-8 inside the logarithm)
      freq_penalty = sum_e (f_e - 1/E)^2                      ([P2 §4.2]: f_e is
                     the expert's share of all top-k selections)
    """
    T, E = p.shape
    f = counts.astype(np.float64) / float(T * top_k)
    P = p.mean(axis=0)
    lb = float(E * np.sum(f * P))
    z = float(np.mean(lse * lse))
    u = 1.0 / E
    return {"lb": lb, "z": z, "weighted": 0.01 * lb + 0.001 * z, "f": f, "P": P,
            "lb_squares": float(E * np.sum(P * P)),
            "kl_uniform": float(np.sum(u * (np.log(u) - np.log(P + 1e-8)))),
            "freq_penalty": float(np.sum((f - u) ** 2))}


# ---------------------------------------------------------------------------
# the whole layer


def forward(cfg, t, rows=None, want_routed_rows=False):
    """Full forward of the layer on CPU.

    cfg: object with T, d, E, k, f, S, dtype ("bf16"/"f32"), act
         ("swiglu"/"gelu"), capacity_factor (<= 0: none), add_residual, and
         optionally weights ("act", or "int8": expert weights are INT8
         codes with float32 row scales w1_scale / w2_scale / ws1_scale /
         ws2_scale in t) and router_temperature (tau, default 1).
    t:   dict with x [T, d], w_router [E, d], router_bias [E] float32 or None,
         optionally router_noise [T, E] float32 (added to the scores),
         w1 / b1 / w2 / b2 (indexable by expert), ws1 / sb1 / ws2 / sb2
         (indexable by shared expert, may be None when S == 0).
    rows: optional iterable of token indices; the expert FFNs and y are then
         evaluated for those tokens only (routing, dispatch and aux always
         cover all T tokens).
    want_routed_rows: also return the raw (unweighted) expert output for
         every kept row in permuted order (needs rows is None).

    Returns a dict of float64 / int64 arrays and scalars.
    """
    dt = cfg.dtype
    wf = getattr(cfg, "weights", "act")
    x = decode(t["x"], dt)
    T, d = x.shape
    E, k = cfg.E, cfg.k
    wr = decode(t["w_router"], dt)
    rb = t.get("router_bias")
    rb = None if rb is None else np.asarray(rb, dtype=np.float32).astype(np.float64)

    tau = float(getattr(cfg, "router_temperature", 1.0))
    logits = router_scores(router_logits(x, wr, rb), tau, t.get("router_noise"))
    p, lse = softmax_lse(logits)
    idx = topk_select(p, k)
    w = renormalise(p, idx)
    counts = expert_counts(idx, E)
    cap = capacity(cfg.capacity_factor, T, k, E)
    offsets, perm_token, perm_slot, inv_row, n_dropped = dispatch(idx, E, cap)
    aux = aux_losses(p, lse, counts, k)

    tok = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    pos = {int(tt): i for i, tt in enumerate(tok)}
    routed = np.zeros((len(tok), d))
    routed_rows = np.zeros((len(perm_token), d)) if (want_routed_rows and rows is None) else None

    b1s, b2s = t.get("b1"), t.get("b2")
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        sel = [r for r in range(r0, r1) if int(perm_token[r]) in pos]
        if not sel:
            continue
        toks = perm_token[sel]
        out = expert_ffn(
            x[toks], expert_weight(t, "w1", e, dt, wf), None if b1s is None else decode(b1s[e], dt),
            expert_weight(t, "w2", e, dt, wf), None if b2s is None else decode(b2s[e], dt), cfg.act)
        for i, r in enumerate(sel):
            tt, j = int(perm_token[r]), int(perm_slot[r])
            routed[pos[tt]] += w[tt, j] * out[i]
            if routed_rows is not None:
                routed_rows[r] = out[i]

    shared = None
    if cfg.S > 0:
        shared = shared_ffn(x[tok], t["ws1"], t.get("sb1"), t["ws2"], t.get("sb2"), cfg.S, cfg.act, dt,
                            wf, t.get("ws1_scale"), t.get("ws2_scale"))
    y = combine(routed, shared, x[tok] if cfg.add_residual else None)

    return {
        "logits": logits, "p": p, "lse": lse,
        "topk_idx": idx, "topk_w": w,
        "counts": counts, "capacity": cap, "offsets": offsets,
        "perm_token": perm_token, "perm_slot": perm_slot,
        "perm_w": w[perm_token, perm_slot] if len(perm_token) else np.zeros(0),
        "inv_row": inv_row, "n_dropped": int(n_dropped),
        "lb": aux["lb"], "z": aux["z"], "weighted": aux["weighted"],
        "lb_squares": aux["lb_squares"], "kl_uniform": aux["kl_uniform"],
        "freq_penalty": aux["freq_penalty"],
        "rows": tok, "y": y, "shared_y": shared, "routed_rows": routed_rows,
    }


# ---------------------------------------------------------------------------
# backward pass: the gradient of the training loss the pages use,
# loss = task + aux ([P3 §4.2] adds the auxiliary loss to the main loss and
# back-propagates both; [P5 §2] weights load balance 0.01 and z-loss 0.001).
# The task loss enters through dy = dLoss/dy; the aux part is
# aux_scale * (0.01 lb + 0.001 z).  Top-k selection, capacity drops and the
# selection shares f_e are piecewise constant: no gradient flows through them.


def _gelu_grad(z):
    """d/dz gelu(z) = Phi(z) + z phi(z) (exact GELU)."""
    erf = np.vectorize(math.erf, otypes=[np.float64])
    Phi = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    phi = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return Phi + z * phi


def _silu_grad(z):
    """d/dz silu(z) = s (1 + z (1 - s)), s = 1 / (1 + exp(-z))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(x_rows, w1, b1, w2, b2, act: str, d_out):
    """Gradients of one expert on a block of rows, given d_out = dL/d out.

    Recomputes the pre-activations a = x W1^T (+ b1) and h = act(a), then
      dW2 = d_out^T h, db2 = sum_rows d_out, dh = d_out W2,
      da = dh * act'(a)   (SwiGLU: dg = dh u silu'(g), du = dh silu(g)),
      dW1 = da^T x, db1 = sum_rows da, dx = da W1.
    Returns (dx, dW1, db1, dW2, db2) in float64.
    """
    a = x_rows @ w1.T
    if b1 is not None:
        a = a + b1[None, :]
    if act == "gelu":
        h = _gelu(a)
    elif act == "swiglu":
        f = w1.shape[0] // 2
        g, u = a[:, :f], a[:, f:]
        h = _silu(g) * u
    else:
        raise ValueError(f"unknown activation {act!r}")
    dW2 = d_out.T @ h
    db2 = d_out.sum(axis=0)
    dh = d_out @ w2
    if act == "gelu":
        da = dh * _gelu_grad(a)
    else:
        da = np.concatenate([dh * u * _silu_grad(g), dh * _silu(g)], axis=1)
    dW1 = da.T @ x_rows
    db1 = da.sum(axis=0)
    dx = da @ w1
    return dx, dW1, db1, dW2, db2


def backward(cfg, t, dy, aux_scale: float = 1.0, loss_weights=None):
    """Gradients of  sum(dy * y) + aux_scale * (0.01 lb + 0.001 z)  with
    respect to x and every parameter (float64), for activation-dtype
    expert weights.  loss_weights, if given, replaces the aux part with
    c_lb lb + c_z z + c_sq lb_squares + c_kl kl_uniform for the dict
    {"lb": c_lb, "z": c_z, "lb_squares": c_sq, "kl_uniform": c_kl}
    (aux_scale is then ignored): the load-balance forms of [P3 §3.1] and
    [P2 §4.2] used as the training loss instead of, or beside, the main one.
    The frequency penalty of [P2 §4.2] depends on the selection only and has
    no gradient.

    dy: [T, d] upstream gradient of the layer output.
    Returns a dict: dx [T, d], dw_router [E, d], drouter_bias [E],
    dw1 [E, w1_rows, d], db1 [E, w1_rows], dw2 [E, d, f], db2 [E, d], and for
    S > 0 dws1 / dsb1 / dws2 / dsb2 of the same shapes per shared expert; plus
    dtopk_w [T, k] (the gradient reaching the routing weights) and
    dscores [T, E] (the gradient of the router scores).

    Steps, in the forward's reverse order:
      combine    y_t = sum_j w_tj o_tj + sum_s FFN_s(x_t) (+ x_t):
                 d o_tj = w_tj dy_t for kept slots, dw_tj = dy_t . o_tj;
      experts    expert_ffn_backward on each expert's kept rows, dx of the
                 rows added back to their tokens; shared experts on all
                 tokens with d out = dy; the residual passes dy to dx;
      renorm     w_j = p_j / P with P the sum of the k selected p:
                 dp_m = (dw_m - sum_j dw_j w_j) / P for selected m, else 0;
      aux        d lb / d p_te = E f_e / T;  d z / d s_te = 2 lse_t p_te / T;
                 d lb_squares / d p_te = 2 E P_e / T;
                 d kl_uniform / d p_te = -1 / (E (P_e + 1e-8) T);
      softmax    ds_te = p_te (dp_te - sum_e' p_te' dp_te');
      scores     s = (x W_r^T + b) / tau + noise:  dl = ds / tau,
                 dW_r = dl^T x, db = sum_t dl, dx += dl W_r.
    """
    dt = cfg.dtype
    if getattr(cfg, "weights", "act") != "act":
        raise ValueError("the backward takes activation-dtype expert weights")
    x = decode(t["x"], dt)
    T, d = x.shape
    E, k = cfg.E, cfg.k
    dy = np.asarray(dy, dtype=np.float64)
    wr = decode(t["w_router"], dt)
    rb = t.get("router_bias")
    rb = None if rb is None else np.asarray(rb, dtype=np.float32).astype(np.float64)
    tau = float(getattr(cfg, "router_temperature", 1.0))
    s = router_scores(router_logits(x, wr, rb), tau, t.get("router_noise"))
    p, lse = softmax_lse(s)
    idx = topk_select(p, k)
    w = renormalise(p, idx)
    counts = expert_counts(idx, E)
    cap = capacity(cfg.capacity_factor, T, k, E)
    offsets, perm_token, perm_slot, inv_row, _ = dispatch(idx, E, cap)

    dx = np.zeros((T, d))
    dw = np.zeros((T, k))
    g = {}
    b1s, b2s = t.get("b1"), t.get("b2")
    w1_0 = decode(t["w1"][0], dt)
    g["dw1"] = np.zeros((E,) + w1_0.shape)
    g["db1"] = np.zeros((E, w1_0.shape[0]))
    g["dw2"] = np.zeros((E, d, cfg.f))
    g["db2"] = np.zeros((E, d))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        toks, slots = perm_token[r0:r1], perm_slot[r0:r1]
        w1 = decode(t["w1"][e], dt)
        w2 = decode(t["w2"][e], dt)
        b1 = None if b1s is None else decode(b1s[e], dt)
        b2 = None if b2s is None else decode(b2s[e], dt)
        out = expert_ffn(x[toks], w1, b1, w2, b2, cfg.act)
        dw[toks, slots] = np.sum(dy[toks] * out, axis=1)
        d_out = w[toks, slots][:, None] * dy[toks]
        dxe, g["dw1"][e], g["db1"][e], g["dw2"][e], g["db2"][e] = expert_ffn_backward(
            x[toks], w1, b1, w2, b2, cfg.act, d_out)
        np.add.at(dx, toks, dxe)

    if cfg.S > 0:
        sb1s, sb2s = t.get("sb1"), t.get("sb2")
        ws1_0 = decode(t["ws1"][0], dt)
        g["dws1"] = np.zeros((cfg.S,) + ws1_0.shape)
        g["dsb1"] = np.zeros((cfg.S, ws1_0.shape[0]))
        g["dws2"] = np.zeros((cfg.S, d, cfg.f))
        g["dsb2"] = np.zeros((cfg.S, d))
        for si in range(cfg.S):
            dxs, g["dws1"][si], g["dsb1"][si], g["dws2"][si], g["dsb2"][si] = expert_ffn_backward(
                x, decode(t["ws1"][si], dt), None if sb1s is None else decode(sb1s[si], dt),
                decode(t["ws2"][si], dt), None if sb2s is None else decode(sb2s[si], dt), cfg.act, dy)
            dx += dxs
    if cfg.add_residual:
        dx += dy

    # routing weights -> probabilities (renormalisation), aux, softmax
    sel = np.take_along_axis(p, idx, axis=1)
    P = sel.sum(axis=1, keepdims=True)
    dp = np.zeros((T, E))
    dsel = (dw - np.sum(dw * w, axis=1, keepdims=True)) / P
    np.put_along_axis(dp, idx, dsel, axis=1)
    if loss_weights is None:
        c_lb, c_z, c_sq, c_kl = 0.01 * aux_scale, 0.001 * aux_scale, 0.0, 0.0
    else:
        c_lb, c_z = loss_weights.get("lb", 0.0), loss_weights.get("z", 0.0)
        c_sq, c_kl = loss_weights.get("lb_squares", 0.0), loss_weights.get("kl_uniform", 0.0)
    f_share = counts.astype(np.float64) / float(T * k)
    P_mean = p.mean(axis=0)
    dp += c_lb * E * f_share[None, :] / T
    dp += c_sq * 2.0 * E * P_mean[None, :] / T
    dp += c_kl * (-1.0 / (E * (P_mean + 1e-8)))[None, :] / T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    ds += c_z * 2.0 * lse[:, None] * p / T
    dl = ds / tau
    g["dw_router"] = dl.T @ x
    g["drouter_bias"] = dl.sum(axis=0)
    dx += dl @ wr
    g["dx"] = dx
    g["dtopk_w"] = dw
    g["dscores"] = ds
    return g
