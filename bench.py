"""Throughput of the MoE layer forward on one MI355X.

One step = one moe_forward call (router, permutation, routed and shared
expert FFNs, combine, aux statistics) over one batch of synthetic tokens
already resident in HBM, bf16 with float32 accumulation.

Headline workload (default): the skewed-routing layer, the largest named
layer that fits one GPU: T = 65536 tokens, d_model 2048, 64 routed experts
top-6 plus 2 shared experts, SwiGLU d_ffn 1408, Zipf-like router bias
b_i = 2 ln(1/(i+1)), no capacity limit.  The other named layers are timed as
extra legs of the same run (Flash T = 4096, FLAME-shaped T = 16384, decode
T = 128 with 22.5 GB of expert weights).

Prints ONE JSON line (rank 0).  Per leg:
  roofline      the grouped expert GEMMs (routed experts: gate/up GEMM with
                the SwiGLU epilogue + down GEMM; shared experts: the same
                pair over all tokens) timed with HIP events on the stream
                they run on, against the bf16 dense MFMA peak, or, for the
                weight-streaming decode layer, against the HBM peak;
  flush         the forward timed once per iteration with a 512 MB device
                write between iterations (cold L2 / Infinity Cache);
  backward      moe_forward_train + moe_backward (headline and Flash legs).
  cpu_baseline  the float64 CPU oracle timed on the host on a bounded
                sample of the leg's workload (the first tokens as a batch of
                their own; for the decode layer a few tokens of the full
                batch, with only their experts' weights), and the GPU output
                of the same tokens against it (parity).
Headline only:
  clock         the GPU clock amd-smi reports while the GEMM leg runs.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
HEADLINE = "c4"
EXTRA_LEGS = "c2,c3,c5"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_traffic.json")
# sources of the grouped GEMM kernels: the committed counter figures hold only
# while these are unchanged
GEMM_SRCS = [os.path.join(ROOT, "mixture_experts_layer_41_amd", "csrc", n)
             for n in ("gemm.hip", "gemm_mfma.hip", "gemm_pipe.hip", "gemm_common.h", "gemm_wide.hip")]
FLUSH_BYTES = 512 << 20
# Timed work per measurement of an extra leg (and of every grouped-GEMM
# leg), at least: a short layer timed over 20 steps (1.5 ms on the Flash
# layer) reads several percent slow against its steady state.
MIN_TIMED_SECONDS = 0.05
MAX_TIMED_ITERS = 2000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="headline layer config (default: c4)")
    ap.add_argument("--legs", default=EXTRA_LEGS,
                    help="comma-separated extra layer configs, or 'none' (default: c2,c3,c5)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time the oracle is run for on the headline workload")
    ap.add_argument("--cpu-leg-seconds", type=float, default=4.0,
                    help="CPU time the oracle is run for on each extra leg")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of a batch the CPU oracle leg runs on (a whole batch if smaller)")
    ap.add_argument("--cpu-decode-tokens", type=int, default=2,
                    help="tokens of the decode layer's batch the CPU oracle evaluates")
    ap.add_argument("--no-backward", action="store_true", help="skip the training (backward) legs")
    ap.add_argument("--no-flush", action="store_true", help="skip the cold-cache variant")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the amd-smi clock reading (and the GEMM launches it runs under)")
    ap.add_argument("--top-k", type=int, default=None,
                    help="override the headline workload's k (e.g. top-1 against top-2 inference)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def gemm_source_hash():
    h = hashlib.sha256()
    for p in GEMM_SRCS:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration(n_bytes=1 << 30, reps=5):
    """A plain device-to-device copy of n_bytes, run reps times: the reference
    workload against which the HBM byte counters are scaled."""
    import torch
    torch.cuda.set_device(0)
    src = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "reps": reps,
                      "GB_per_s": round(2 * n_bytes / dt / 1e9, 1),
                      "gemm_source_sha256_16": gemm_source_hash()}), flush=True)


def traffic_entry(workload):
    """HBM bytes of one grouped-GEMM launch (routed + shared) from the
    committed counter runs, if they were taken on this workload and the
    current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        if rec.get("kernel_sha256_16") != gemm_source_hash():
            return None
        return rec["bytes_per_launch"].get(workload)
    except (OSError, KeyError, ValueError, AttributeError):
        return None


def cpu_info():
    model = platform.processor() or None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')})"
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    return model, blas, int(threads)


def gpu_clock_sample():
    """One reading of amd-smi's graphics clocks of GPU 0 (one per XCD), or an
    error string; never raises."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                           text=True, timeout=20)
        if r.returncode != 0:
            return {"error": (r.stderr or r.stdout).strip()[-200:]}
        data = json.loads(r.stdout)
        gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
        clk = gpu["clock"]
        cur = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_")]
        mx = [clk[k]["max_clk"]["value"] for k in sorted(clk) if k.startswith("gfx_")]
        cur = [float(v) for v in cur if isinstance(v, (int, float))]
        return {"source": "amd-smi metric -g 0 -c", "gfx_clk_mhz": cur,
                "mean_mhz": round(sum(cur) / len(cur), 1) if cur else None,
                "max_clk_mhz": max(mx) if mx else None}
    except Exception as e:  # amd-smi missing or its output unexpected: report, never fail
        return {"error": str(e)[-200:]}


# ---------------------------------------------------------------------------


def dev_tensor(a):
    import numpy as np
    import torch
    from moe_inputs import Bank
    if a is None:
        return None
    if isinstance(a, Bank):
        from concurrent.futures import ThreadPoolExecutor
        tdt = {np.uint16: torch.bfloat16, np.int8: torch.int8}.get(a.np_dtype, torch.float32)
        out = torch.empty(a.full_shape, dtype=tdt, device="cuda")
        with ThreadPoolExecutor(max_workers=16) as ex:
            for e, arr in ex.map(lambda e: (e, a[e]), range(a.n)):
                out[e].copy_(dev_tensor(arr))
        return out
    a = np.ascontiguousarray(a)
    if a.dtype == np.int8:          # 8-bit weight codes
        return torch.from_numpy(a).cuda()
    if a.dtype == np.uint16:        # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def layer_weights(t):
    import torch
    from mixture_experts_layer_41_amd import binding as B
    rb = t["router_bias"]
    return B.LayerWeights(
        w_router=dev_tensor(t["w_router"]), w1=dev_tensor(t["w1"]), w2=dev_tensor(t["w2"]),
        b1=dev_tensor(t["b1"]), b2=dev_tensor(t["b2"]), shared_w1=dev_tensor(t["ws1"]),
        shared_w2=dev_tensor(t["ws2"]), shared_b1=dev_tensor(t["sb1"]),
        shared_b2=dev_tensor(t["sb2"]), w1_scale=dev_tensor(t.get("w1_scale")),
        w2_scale=dev_tensor(t.get("w2_scale")), shared_w1_scale=dev_tensor(t.get("ws1_scale")),
        shared_w2_scale=dev_tensor(t.get("ws2_scale")),
        router_bias=None if rb is None else torch.from_numpy(rb).cuda())


def oracle_lazy(cfg):
    """Whether the CPU oracle leg keeps the expert weights lazy (generated
    one expert at a time) and evaluates a few tokens of the full batch: the
    weight stacks of the decode layer (22.5 GB) are too large to hold."""
    return cfg.E * cfg.w1_rows * cfg.d * 3 > (1 << 32)


def cpu_sample_tokens(cfg, args):
    """Tokens the CPU oracle leg evaluates: a few of the decode batch; the
    whole batch when a capacity limit makes the drops depend on it (if it
    is not much larger than the sample); else the first --cpu-tokens."""
    if oracle_lazy(cfg):
        return args.cpu_decode_tokens
    if cfg.capacity_factor > 0 and cfg.T <= 4 * args.cpu_tokens:
        return cfg.T
    return args.cpu_tokens


def run_leg(cfg, args, headline, want_backward, want_host_inputs):
    """Times one layer config; returns (leg dict, host inputs or None,
    device handles for the parity check)."""
    import torch
    from moe_inputs import make_inputs
    from mixture_experts_layer_41_amd import binding as B

    stream = torch.cuda.current_stream()
    q8 = cfg.weights == "int8"
    log(f"[bench] leg {cfg.name}: generating inputs")
    t0 = time.perf_counter()
    # raw seeded draws (no tie rejection: timing only); expert weight stacks
    # stay lazy (generated one expert at a time) unless the CPU leg needs them
    t = make_inputs(cfg, materialize=want_host_inputs and not oracle_lazy(cfg))
    W = layer_weights(t)
    x = dev_tensor(t["x"])
    noise = dev_tensor(t.get("router_noise"))
    torch.cuda.synchronize()
    log(f"[bench] leg {cfg.name}: inputs on the GPU in {time.perf_counter() - t0:.1f} s")
    c = B.config_of(cfg)
    fwd = B.Forward(c, W)

    # ---- eager warm-up, then eager and (optionally) graph timing
    for _ in range(max(args.warmup, 1)):
        fwd(x, noise)
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fwd(x, noise)
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            graph = g
        except Exception as e:  # capture not possible: time eager launches
            log(f"[bench] graph capture failed ({e}); timing eager launches")

    def iters_for(fn, base):
        """At least `base` iterations, and enough for MIN_TIMED_SECONDS of
        work (estimated from 3 untimed calls)."""
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        est = (time.perf_counter() - s0) / 3
        return int(min(MAX_TIMED_ITERS, max(base, -(-MIN_TIMED_SECONDS // max(est, 1e-6)))))

    def timed(step_fn, steps):
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(steps):
            step_fn()
        torch.cuda.synchronize()
        return time.perf_counter() - s0

    # the headline leg times exactly --steps steps; an extra leg at least that
    # many and at least MIN_TIMED_SECONDS of them
    n_steps = args.steps if headline else iters_for(lambda: fwd(x, noise), args.steps)
    eager_s = timed(lambda: fwd(x, noise), n_steps)
    graph_s = timed(graph.replay, n_steps) if graph is not None else None
    best_s = min(s for s in (eager_s, graph_s) if s is not None)
    mode = "hip_graph" if (graph_s is not None and graph_s <= eager_s) else "eager"
    del graph
    step_us = best_s / n_steps * 1e6
    log(f"[bench] leg {cfg.name}: eager {eager_s / n_steps * 1e6:.1f} us/step"
        + (f", graph {graph_s / n_steps * 1e6:.1f} us/step" if graph_s else "")
        + f" ({n_steps} steps)")

    # ---- routing statistics of this batch (for the algorithmic work counts)
    torch.cuda.synchronize()
    aux = B.aux_to_dict(fwd.aux)
    R = int(aux["n_kept"])
    T, d, f, S, k, E = cfg.T, cfg.d, cfg.f, cfg.S, cfg.k, cfg.E
    per_row = (6 if cfg.act == "swiglu" else 4) * d * f        # flops per kept row (one expert)
    routed_flops = R * per_row
    shared_flops = T * S * per_row
    router_flops = 2 * T * d * E
    layer_flops = routed_flops + shared_flops + router_flops

    # ---- cold-cache variant: a 512 MB write between iterations, each
    # forward bracketed by its own events
    flush = None
    if not args.no_flush:
        junk = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        n_fl = max(5, min(args.steps, 20))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_fl)]
        torch.cuda.synchronize()
        for a, b in evs:
            junk.fill_(1)
            a.record(stream)
            fwd(x, noise)
            b.record(stream)
        torch.cuda.synchronize()
        fl_us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        flush = {"us_per_step_median": round(fl_us[len(fl_us) // 2], 2),
                 "tokens_per_s": round(T / (fl_us[len(fl_us) // 2] / 1e6), 1),
                 "iterations": n_fl, "flush_bytes": FLUSH_BYTES}
        del junk

    # ---- roofline leg: the grouped expert GEMMs alone (routed + shared),
    # HIP events on this stream
    pr = B.moe_permute(c, fwd.topk_idx)
    torch.cuda.synchronize()
    calls = []
    if q8:
        calls.append(B.ExpertFFN(c, E, 1, T * k, x, pr["perm_token"], pr["expert_offsets"], W.w1,
                                 W.b1, W.w2, W.b2, w1_scale=W.w1_scale, w2_scale=W.w2_scale))
        if S:
            calls.append(B.ExpertFFN(c, 1, S, T, x, None, None, W.shared_w1, W.shared_b1,
                                     W.shared_w2, W.shared_b2, w1_scale=W.shared_w1_scale,
                                     w2_scale=W.shared_w2_scale))
    else:
        calls.append(B.ExpertFFN(c, E, 1, T * k, x, pr["perm_token"], pr["expert_offsets"], W.w1,
                                 W.b1, W.w2, W.b2))
        if S:
            calls.append(B.ExpertFFN(c, 1, S, T, x, None, None, W.shared_w1, W.shared_b1,
                                     W.shared_w2, W.shared_b2))

    def ffn_all():
        for cl in calls:
            cl()

    for _ in range(5):
        ffn_all()
    n_ffn = iters_for(ffn_all, max(20, args.steps))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(n_ffn):
        ffn_all()
    ev1.record(stream)
    ev1.synchronize()
    ffn_s = ev0.elapsed_time(ev1) / 1e3 / n_ffn
    gemm_flops = routed_flops + shared_flops
    gemm_tflops = gemm_flops / ffn_s / 1e12

    # sustained clock while the GEMMs run (headline only): enqueue about two
    # seconds of GEMM launches, read amd-smi from the host meanwhile
    clock = None
    if headline and not args.no_clock:
        n_busy = max(1, int(2.0 / max(ffn_s, 1e-6)))
        box = {}
        th = threading.Thread(target=lambda: (time.sleep(0.8), box.setdefault("c", gpu_clock_sample())))
        for _ in range(min(n_busy, 4000)):
            ffn_all()
        th.start()
        th.join()
        torch.cuda.synchronize()
        clock = box.get("c")

    # algorithmic bytes of the same launches: the weights of every expert
    # that keeps a row (W1 [w1_rows, d] and W2 [d, f]; with 8-bit weights one
    # byte per code plus a float32 scale per row), the shared experts'
    # weights, the input rows read, H written and read back, the output rows
    offs = pr["expert_offsets"].cpu().numpy()
    touched = int((offs[1:] - offs[:-1] > 0).sum())
    ab = 2 if cfg.dtype == "bf16" else 4
    n_w = touched + S
    if q8:
        weight_bytes = n_w * ((cfg.w1_rows + f) * d + 4 * (cfg.w1_rows + d))
    else:
        weight_bytes = ab * n_w * (cfg.w1_rows + f) * d
    act_rows = R + T * S if S else R
    gemm_bytes = weight_bytes + ab * (R * d + (T * d if S else 0) + 2 * act_rows * f + act_rows * d)
    ridge = MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3          # flop per byte
    common = {"launch_us": round(ffn_s * 1e6, 2), "calls_timed": n_ffn, "flops_per_launch": gemm_flops,
              "bytes_per_launch": gemm_bytes, "touched_experts": touched,
              "traffic": traffic_entry(cfg.name)}
    if gemm_flops / weight_bytes >= ridge:
        roofline = {
            "kernel": "grouped expert GEMMs: routed (gate/up + SwiGLU epilogue, down) and "
                      "shared (the same pair over all tokens)",
            "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4), **common}
    else:   # weight streaming: fewer flops per byte than the MFMA/HBM ridge
        gbs = gemm_bytes / ffn_s / 1e9
        roofline = {
            "kernel": "grouped expert GEMMs streaming the weights of the touched and shared experts",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), **common}
    log(f"[bench] leg {cfg.name}: grouped GEMMs {ffn_s * 1e6:.1f} us -> {gemm_tflops:.1f} TFLOP/s, "
        f"{gemm_bytes / ffn_s / 1e9:.0f} GB/s")
    del calls

    # ---- training leg: moe_forward_train + moe_backward on the same batch
    backward = None
    if want_backward and cfg.dtype == "bf16" and not q8:
        tr = B.TrainStep(c, W)
        gen = torch.Generator(device="cuda").manual_seed(5)
        g_dy = torch.randn(T, d, device="cuda", generator=gen).to(torch.bfloat16)
        for _ in range(3):
            tr.forward(x, noise)
            tr.backward(g_dy)
        n_tr = iters_for(lambda: (tr.forward(x, noise), tr.backward(g_dy)), max(10, args.steps))
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))

        def loop_ms(fn):
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n_tr):
                fn()
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1)

        f_ms = loop_ms(lambda: tr.forward(x, noise))
        b_ms = loop_ms(lambda: tr.backward(g_dy))
        s_ms = loop_ms(lambda: (tr.forward(x, noise), tr.backward(g_dy)))
        bwd_s = b_ms / 1e3 / n_tr
        w1r = 2 * f if cfg.act == "swiglu" else f
        bflops = 2 * (R + T * S) * (2 * d * w1r + 2 * d * f) + 2 * 2 * T * d * E
        bt = bflops / bwd_s / 1e12
        backward = {
            "what": "moe_backward (all gradients) after moe_forward_train, same batch; "
                    "each figure from back-to-back calls",
            "us_per_step": round(bwd_s * 1e6, 2), "calls_timed": n_tr,
            "train_forward_us": round(f_ms / n_tr * 1e3, 2),
            "train_step_us": round(s_ms / n_tr * 1e3, 2),
            "tokens_per_s_train": round(T / (s_ms / n_tr / 1e3), 1),
            "flops_per_step": bflops, "achieved_tflops": round(bt, 2),
            "frac_of_mfma_peak": round(bt / MFMA_BF16_PEAK_TFLOPS, 4),
        }
        log(f"[bench] leg {cfg.name}: training forward {f_ms / n_tr * 1e3:.1f} us + backward "
            f"{bwd_s * 1e6:.1f} us ({bt:.0f} TFLOP/s algorithmic); whole step "
            f"{s_ms / n_tr * 1e3:.1f} us")
        del tr

    leg = {
        "workload": cfg.name, "tokens": T, "d_model": d, "experts": E, "top_k": k, "d_ffn": f,
        "shared_experts": S, "capacity_factor": cfg.capacity_factor,
        "router_temperature": cfg.router_temperature, "router_noise_std": cfg.router_noise_std,
        "expert_weights": "int8 codes + f32 row scales" if q8 else
        ("bf16" if cfg.dtype == "bf16" else "f32"),
        "us_per_step": round(step_us, 2), "tokens_per_s": round(T / (step_us / 1e6), 1),
        "launch": mode, "timed_steps": n_steps, "eager_us_per_step": round(eager_s / n_steps * 1e6, 2),
        "graph_us_per_step": None if graph_s is None else round(graph_s / n_steps * 1e6, 2),
        "layer_tflops": round(layer_flops / (step_us / 1e6) / 1e12, 2),
        "kept_rows": R, "dropped": int(aux["n_dropped"]),
        "roofline": roofline, "flush": flush, "backward": backward,
    }
    handles = {"fwd": fwd, "x": x, "noise": noise, "W": W}
    return leg, t if want_host_inputs else None, handles, clock


class _ExpertCache(dict):
    """Weights of some experts of a lazy stack, generated before the timed
    region; an expert not in it is generated on first use."""

    def __init__(self, bank, experts):
        from concurrent.futures import ThreadPoolExecutor
        experts = [int(e) for e in experts]
        with ThreadPoolExecutor(max_workers=16) as ex:
            super().__init__(zip(experts, ex.map(lambda e: bank[e], experts)))
        self.bank = bank

    def __missing__(self, e):
        v = self[e] = self.bank[e]
        return v


def cpu_baseline_leg(cfg, t, handles, n_tokens, seconds):
    """The oracle (float64 numpy, as it stands) timed on the host, and the
    GPU output of the same tokens against it.

    Stacked weights: the first n tokens of the batch as a batch of their own
    (per-token results do not depend on the batch without a capacity limit;
    with one, n is the whole batch or parity is skipped).  Lazy weights (the
    decode layer): routing over the full batch and the expert FFNs of its
    first n tokens only, with those tokens' experts generated beforehand (the
    generation is not timed)."""
    import numpy as np
    import torch
    import oracle

    fwd = handles["fwd"]
    y = fwd(handles["x"], handles["noise"])
    torch.cuda.synchronize()
    model, blas, threads = cpu_info()
    lazy = oracle_lazy(cfg)
    if lazy:
        n = min(n_tokens, cfg.T)
        rows = list(range(n))
        touched = sorted(set(fwd.topk_idx[:n].cpu().numpy().reshape(-1).tolist()))
        cs, ts = cfg, dict(t)
        for name in ("w1", "w2", "w1_scale", "w2_scale"):
            if ts.get(name) is not None:
                ts[name] = _ExpertCache(ts[name], touched)
        for name in ("ws1", "ws2", "ws1_scale", "ws2_scale"):
            if ts.get(name) is not None:
                ts[name] = _ExpertCache(ts[name], range(cfg.S))
        what = (f"tokens 0..{n - 1} of the {cfg.T}-token batch: routing of all {cfg.T} tokens, the "
                f"routed ({len(touched)} experts) and shared expert FFNs and the combine of those {n}")
    else:
        n = min(n_tokens, cfg.T)
        rows = None
        cs = dataclasses.replace(cfg, T=n)
        ts = dict(t)
        ts["x"] = t["x"][:n]
        if t.get("router_noise") is not None:
            ts["router_noise"] = t["router_noise"][:n]
        what = (f"the first {n} of the {cfg.T} tokens of this workload as one batch "
                f"(routing, permutation, routed and shared expert FFNs, combine, aux)")
    runs, t_cpu, ref = 0, 0.0, None
    while t_cpu < seconds or runs == 0:
        s0 = time.perf_counter()
        ref = oracle.forward(cs, ts, rows=rows)
        t_cpu += time.perf_counter() - s0
        runs += 1
    cpu = {"value": round(n * runs / t_cpu, 2), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{what}, {runs} run(s) in {t_cpu:.1f} s, float64 numpy",
           "cpu_model": model, "blas": blas}
    log(f"[bench] {cfg.name}: oracle {t_cpu / runs:.2f} s per run of {n} tokens on {threads} threads "
        f"({model}; {blas})")
    parity = None
    if lazy or not (cfg.capacity_factor > 0 and n < cfg.T):
        yg = y[:n].float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(yg - ref["y"])) / np.max(np.abs(ref["y"])))
        other = int((fwd.topk_idx[:n].cpu().numpy() != ref["topk_idx"][:n]).any(1).sum())
        parity = {"tokens_compared": n, "y_normwise_err": err, "tokens_with_other_topk": other,
                  "note": "raw draws without the tie-gap rule: a token with a near-tie may pick "
                          "another expert"}
        log(f"[bench] {cfg.name}: parity on {n} tokens: {parity}")
    return cpu, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer runs on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    from moe_inputs import get_config

    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    if args.top_k is not None:
        cfg = dataclasses.replace(cfg, k=args.top_k, name=f"{cfg.name}_top{args.top_k}")
    extra = [] if args.legs.strip().lower() in ("", "none") else \
        [w.strip() for w in args.legs.split(",") if w.strip() and w.strip() != args.workload]

    # ---- headline
    want_cpu = not args.no_cpu
    head, t, handles, clock = run_leg(cfg, args, True, not args.no_backward, want_cpu)
    cpu = parity = None
    if want_cpu:
        cpu, parity = cpu_baseline_leg(cfg, t, handles, cpu_sample_tokens(cfg, args), args.cpu_seconds)
    del t, handles
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ---- extra legs (other named layers), each freed before the next
    legs = {}
    for name in extra:
        lc = get_config(name)
        leg, tl, h, _ = run_leg(lc, args, False, not args.no_backward and name == "c2", want_cpu)
        if want_cpu:
            leg["cpu_baseline"], leg["parity"] = cpu_baseline_leg(lc, tl, h, cpu_sample_tokens(lc, args),
                                                                  args.cpu_leg_seconds)
        legs[name] = leg
        del h, tl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    out = {
        "metric": "MoE-layer fwd tokens/s + grouped-GEMM % MFMA peak (1 MI355X)",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded draws of the layer's shapes and distributions)",
        "config": {k2: v for k2, v in head.items() if k2 not in ("roofline", "flush", "backward")},
        "roofline": head["roofline"],
        "flush": head["flush"],
        "backward": head["backward"],
        "cpu_baseline": cpu,
        "parity": parity,
        "clock": clock,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
