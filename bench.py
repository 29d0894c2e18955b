"""Throughput of the MoE layer forward on one MI355X.

One step = one moe_forward call (router, permutation, routed and shared
expert FFNs, combine, aux statistics) over one batch of synthetic tokens
already resident in HBM.  Workload: the small "Flash" layer (T = 4096 tokens
as 2 x 2048, d_model 512, 16 experts, top-2, SwiGLU d_ffn 1024, capacity
factor 1.25), bf16 with float32 accumulation.

Prints ONE JSON line (rank 0).  Extra legs:
  roofline      the grouped expert GEMMs (moe_expert_ffn on the routed rows:
                gate/up GEMM + down GEMM) timed with HIP events on the stream
                they run on, against the bf16 dense MFMA peak;
  cpu_baseline  the float64 CPU oracle on the same inputs, timed on the host.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
WORKLOAD = "c2"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_flash_T4096_traffic.json")
# sources of the grouped GEMM kernels: the committed counter figures hold only
# while these are unchanged
GEMM_SRCS = [os.path.join(ROOT, "mixture_experts_layer_41_amd", "csrc", n)
             for n in ("gemm.hip", "gemm_mfma.hip", "gemm_pipe.hip", "gemm_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=WORKLOAD, help="named layer config (default: c2)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-backward", action="store_true", help="skip the training (backward) leg")
    ap.add_argument("--top-k", type=int, default=None,
                    help="override the workload's k (e.g. top-1 against top-2 inference)")
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
    """HBM traffic of the grouped GEMMs from the committed counter runs, if
    they were taken on this workload and the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        if rec.get("kernel_sha256_16") != gemm_source_hash() or rec.get("workload") != workload:
            return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer runs on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from moe_inputs import Bank, get_config, make_inputs
    from mixture_experts_layer_41_amd import binding as B

    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    if args.top_k is not None:
        cfg = dataclasses.replace(cfg, k=args.top_k, name=f"{cfg.name}_top{args.top_k}")
    log(f"[bench] workload {cfg.name}")
    # raw seeded draws (no tie rejection: timing only); expert weight stacks
    # stay lazy (generated one expert at a time) unless the CPU leg needs them
    big = cfg.E * cfg.w1_rows * cfg.d * 3 > (1 << 31)
    t = make_inputs(cfg, materialize=not (args.no_cpu or big))
    if big and not args.no_cpu:
        log(f"[bench] {cfg.name}: weights too large for the CPU oracle leg; skipping it")
        args.no_cpu = True

    def dev(a):
        if a is None:
            return None
        if isinstance(a, Bank):
            from concurrent.futures import ThreadPoolExecutor
            tdt = {np.uint16: torch.bfloat16, np.int8: torch.int8}.get(a.np_dtype, torch.float32)
            out = torch.empty(a.full_shape, dtype=tdt, device="cuda")
            with ThreadPoolExecutor(max_workers=16) as ex:
                for e, arr in ex.map(lambda e: (e, a[e]), range(a.n)):
                    out[e].copy_(dev(arr))
            return out
        a = np.ascontiguousarray(a)
        if a.dtype == np.int8:          # 8-bit weight codes
            return torch.from_numpy(a).cuda()
        if a.dtype == np.uint16:        # bf16 bit patterns
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    rb = t["router_bias"]
    W = B.LayerWeights(
        w_router=dev(t["w_router"]), w1=dev(t["w1"]), w2=dev(t["w2"]), b1=dev(t["b1"]),
        b2=dev(t["b2"]), shared_w1=dev(t["ws1"]), shared_w2=dev(t["ws2"]),
        shared_b1=dev(t["sb1"]), shared_b2=dev(t["sb2"]),
        w1_scale=dev(t.get("w1_scale")), w2_scale=dev(t.get("w2_scale")),
        shared_w1_scale=dev(t.get("ws1_scale")), shared_w2_scale=dev(t.get("ws2_scale")),
        router_bias=None if rb is None else torch.from_numpy(rb).cuda())
    q8 = cfg.weights == "int8"
    x = dev(t["x"])
    noise = dev(t.get("router_noise"))   # [T, E] float32 or None
    c = B.config_of(cfg)
    fwd = B.Forward(c, W)
    stream = torch.cuda.current_stream()

    # ---- eager warm-up and (optionally) a captured graph of one step
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
            graph = None

    def timed(step_fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step_fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    eager_s = timed(lambda: fwd(x, noise), args.steps)
    graph_s = timed(graph.replay, args.steps) if graph is not None else None
    best_s = min(s for s in (eager_s, graph_s) if s is not None)
    mode = "hip_graph" if (graph_s is not None and graph_s <= eager_s) else "eager"
    log(f"[bench] eager {eager_s / args.steps * 1e6:.1f} us/step"
        + (f", graph {graph_s / args.steps * 1e6:.1f} us/step" if graph_s else ""))

    # ---- routing statistics of this batch (for the algorithmic work counts)
    torch.cuda.synchronize()
    aux = B.aux_to_dict(fwd.aux)
    R = int(aux["n_kept"])
    T, d, f, S, k = cfg.T, cfg.d, cfg.f, cfg.S, cfg.k
    per_row = (6 if cfg.act == "swiglu" else 4) * d * f        # flops per kept row (one expert)
    routed_flops = R * per_row
    shared_flops = T * S * per_row
    router_flops = 2 * T * d * cfg.E
    layer_flops = routed_flops + shared_flops + router_flops

    # ---- roofline leg: the routed grouped GEMMs alone, HIP events on this stream
    pr = B.moe_permute(c, fwd.topk_idx)
    torch.cuda.synchronize()
    y_perm = torch.empty(T * k, d, dtype=B.torch_dtype(c), device="cuda")
    if q8:
        ffn_call = B.moe_expert_ffn_int8
        ffn_args = (c, cfg.E, 1, T * k, x, pr["perm_token"], pr["expert_offsets"], W.w1,
                    W.w1_scale, W.b1, W.w2, W.w2_scale, W.b2, y_perm)
    else:
        ffn_call = B.moe_expert_ffn
        ffn_args = (c, cfg.E, 1, T * k, x, pr["perm_token"], pr["expert_offsets"], W.w1, W.b1,
                    W.w2, W.b2, y_perm)
    for _ in range(10):
        ffn_call(*ffn_args)
    n_ffn = max(50, args.steps // 2)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(n_ffn):
        ffn_call(*ffn_args)
    ev1.record(stream)
    ev1.synchronize()
    ffn_s = ev0.elapsed_time(ev1) / 1e3 / n_ffn
    gemm_tflops = routed_flops / ffn_s / 1e12
    # algorithmic bytes of the same call: the weights of every expert that
    # keeps a row (W1 [w1_rows, d] and W2 [d, f]; with 8-bit weights one byte
    # per code plus a float32 scale per row), the gathered input rows, H
    # written and read back, the output rows
    counts = pr["expert_offsets"].cpu().numpy()
    touched = int((counts[1:] - counts[:-1] > 0).sum())
    ab = 2 if cfg.dtype == "bf16" else 4
    if q8:
        weight_bytes = touched * ((cfg.w1_rows + f) * d + 4 * (cfg.w1_rows + d))
    else:
        weight_bytes = ab * touched * (cfg.w1_rows + f) * d
    routed_bytes = weight_bytes + ab * (R * d + 2 * R * f + R * d)
    # MFMA-bound unless the weights alone give fewer flops per byte than the
    # MFMA / HBM ridge (the weight-streaming decode shape)
    if routed_flops / weight_bytes >= MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        roofline = {
            "kernel": "grouped expert GEMMs (gate/up + activation epilogue, down) over the routed rows",
            "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_entry(cfg.name), "launch_us": round(ffn_s * 1e6, 2),
            "flops_per_launch": routed_flops, "bytes_per_launch": routed_bytes,
        }
    else:   # weight streaming: fewer flops per byte than the MFMA/HBM ridge
        gbs = routed_bytes / ffn_s / 1e9
        roofline = {
            "kernel": "grouped expert GEMMs streaming the weights of the touched experts",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_entry(cfg.name),
            "launch_us": round(ffn_s * 1e6, 2), "bytes_per_launch": routed_bytes,
            "flops_per_launch": routed_flops, "touched_experts": touched,
        }
    log(f"[bench] grouped GEMMs {ffn_s * 1e6:.1f} us -> {gemm_tflops:.1f} TFLOP/s, "
        f"{routed_bytes / ffn_s / 1e9:.0f} GB/s")

    # ---- training leg: moe_forward_train + moe_backward on the same batch
    # (bf16 activations with bf16 expert weights), HIP events on this stream
    backward = None
    if not args.no_backward and cfg.dtype == "bf16" and not q8:
        tr = B.TrainStep(c, W)
        g_dy = torch.randn(T, d, device="cuda", generator=torch.Generator(device="cuda").manual_seed(5))
        g_dy = g_dy.to(torch.bfloat16)
        for _ in range(5):
            tr.forward(x, noise)
            tr.backward(g_dy)
        n_tr = max(20, args.steps // 4)
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))

        def loop_ms(fn):
            """n_tr back-to-back calls (steady state, as the inference leg),
            bracketed by events on the stream."""
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n_tr):
                fn()
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1)

        f_ms = loop_ms(lambda: tr.forward(x, noise))
        # the backward repeated on the last forward's saved state
        b_ms = loop_ms(lambda: tr.backward(g_dy))
        s_ms = loop_ms(lambda: (tr.forward(x, noise), tr.backward(g_dy)))
        bwd_s = b_ms / 1e3 / n_tr
        # algorithmic backward flops: twice the forward's expert products
        # (d input and d weight of each), routed and shared, plus the router's
        w1r = 2 * f if cfg.act == "swiglu" else f
        bflops = 2 * (R + T * S) * (2 * d * w1r + 2 * d * f) + 2 * 2 * T * d * cfg.E
        bt = bflops / bwd_s / 1e12
        backward = {
            "what": "moe_backward (all gradients) after moe_forward_train, same batch; "
                    "each figure from back-to-back calls",
            "us_per_step": round(bwd_s * 1e6, 2),
            "train_forward_us": round(f_ms / n_tr * 1e3, 2),
            "train_step_us": round(s_ms / n_tr * 1e3, 2),
            "tokens_per_s_train": round(T / (s_ms / n_tr / 1e3), 1),
            "flops_per_step": bflops, "achieved_tflops": round(bt, 2),
            "frac_of_mfma_peak": round(bt / MFMA_BF16_PEAK_TFLOPS, 4),
        }
        log(f"[bench] training step: forward {f_ms / n_tr * 1e3:.1f} us + backward "
            f"{bwd_s * 1e6:.1f} us ({bt:.0f} TFLOP/s algorithmic); whole step "
            f"{s_ms / n_tr * 1e3:.1f} us")

    # ---- CPU oracle leg (rank 0, N = 1 only)
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:
            cores = os.cpu_count()
        runs, t_cpu = 0, 0.0
        ref = None
        while t_cpu < args.cpu_seconds or runs == 0:
            t0 = time.perf_counter()
            ref = oracle.forward(cfg, t)
            t_cpu += time.perf_counter() - t0
            runs += 1
        cpu = {"value": round(T * runs / t_cpu, 1), "unit": "tokens/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"full layer forward of this workload ({T} tokens), {runs} run(s), "
                         f"{t_cpu:.1f} s, float64 numpy"}
        y = fwd(x, noise)
        torch.cuda.synchronize()
        yg = y.float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(yg - ref["y"])) / np.max(np.abs(ref["y"])))
        idx_mismatch = int((fwd.topk_idx.cpu().numpy() != ref["topk_idx"]).any(1).sum())
        parity = {"y_normwise_err": err, "tokens_with_other_topk": idx_mismatch,
                  "lb_rel_err": abs(aux["load_balance"] - ref["lb"]) / abs(ref["lb"])}
        log(f"[bench] oracle {t_cpu / runs:.2f} s/forward on {cores} threads; parity {parity}")

    value = T * args.steps / best_s
    out = {
        "metric": "MoE-layer fwd tokens/s + grouped-GEMM % MFMA peak (1 MI355X)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(best_s / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "d_model": d, "experts": cfg.E,
                   "top_k": k, "d_ffn": f, "shared_experts": S,
                   "capacity_factor": cfg.capacity_factor,
                   "router_temperature": cfg.router_temperature,
                   "router_noise_std": cfg.router_noise_std, "expert_weights": "int8 codes + "
                   "f32 row scales" if q8 else ("bf16" if cfg.dtype == "bf16" else "f32"),
                   "launch": mode,
                   "eager_us_per_step": round(eager_s / args.steps * 1e6, 2),
                   "graph_us_per_step": None if graph_s is None else round(graph_s / args.steps * 1e6, 2),
                   "layer_tflops": round(layer_flops / (best_s / args.steps) / 1e12, 2),
                   "kept_rows": R, "dropped": int(aux["n_dropped"])},
        "roofline": roofline,
        "backward": backward,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
