#!/usr/bin/env python3
"""Throughput of the ternary MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole layer path (router logits, certified top-8,
grouping, gate/up + SiLU/clamp, down, combine) over one batch. The default
workload is one-token decode through one layer (hidden 2048, 256 experts,
top-8, moe_intermediate_size 512); successive steps rotate over 24 distinct
layers (3.9 GB of packed experts, far above the 256 MB last-level cache) and
fresh tokens, so expert weights stream from HBM. The K timed steps run as one
captured HIP graph, replayed once after the warm-up. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import os
import sys
import time

METRIC = "ternary MoE layer tokens/s (decode & prefill); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA
H, I, E, K_TOP = 2048, 512, 256, 8
PACKED_GU = I * ((H + 4) // 5)  # bytes of one gate or up matrix
PACKED_D = H * ((I + 4) // 5)
EXPERT_BYTES = 2 * PACKED_GU + PACKED_D + 4 * (2 * I + H)  # 643,072
ROUTER_BYTES = E * H * 4

WORKLOADS = {
    2: dict(name="moe_layer_decode_T1", tokens=1, bias=None, layers=24, steps=2400, warmup=48),
    3: dict(name="moe_layer_decode_T64_zipf1.1", tokens=64, bias="zipf", layers=24, steps=480, warmup=48),
    4: dict(name="moe_layer_prefill_T4096_uniform", tokens=4096, bias="uniform", layers=4, steps=40, warmup=4),
    5: dict(name="moe_stack24_T256_residual", tokens=256, bias=None, layers=24, steps=20, warmup=2),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="distinct layers to rotate over")
    ap.add_argument("--kernel", default="gateup", help="kernel whose roofline is reported")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of one HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the oracle's timed sample")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ensure_built():
    here = os.path.dirname(os.path.abspath(__file__))
    if not os.path.exists(os.path.join(here, "ternary_weight_moe_base_amd", "libtmoe.so")):
        from ternary_weight_moe_base_amd import build as b
        b.build(verbose=True)


# -------------------------------------------------------------- CPU baseline
def cpu_baseline(cfg: int, wl: dict, n_tok: int):
    """The CPU oracle, untuned, timed on this host on a bounded token sample."""
    import numpy as np

    import oracle as O
    import tmoe_inputs as ti

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    layer_of = (lambda i: i % wl["layers"]) if cfg in (2, 3, 4) else (lambda i: 0)
    if cfg == 2:
        batches = [(i, ti.activations(cfg, i + 1)[i:i + 1]) for i in range(n_tok)]
    else:
        x = ti.activations(cfg, wl["tokens"])
        batches = [(0, x[:n_tok])]
    cache = {}

    def raw(layer, e):
        if (layer, e) not in cache:
            cache[(layer, e)] = tuple(ti.expert_matrix(cfg, layer, e, m) for m in range(3))
        return cache[(layer, e)]

    # draw the inputs the oracle will read (untimed): router, then the routed experts
    prep = []
    for i, xb in batches:
        layer = layer_of(i)
        Wr, b = ti.router_matrix(cfg, layer), ti.router_bias(cfg, wl["bias"])
        idx, _, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, K_TOP)
        prep.append((layer, xb, Wr, b, sorted(set(idx.ravel().tolist()))))
    with concurrent.futures.ThreadPoolExecutor(min(16, threads)) as ex:
        keys = [(layer, e) for layer, _, _, _, es in prep for e in es]
        for k_, v in zip(keys, ex.map(lambda le: tuple(ti.expert_matrix(cfg, le[0], le[1], m) for m in range(3)),
                                      keys)):
            cache[k_] = v
    tokens = 0
    t0 = time.perf_counter()
    for layer, xb, Wr, b, _ in prep:
        O.moe_layer(xb, Wr, b, lambda e, layer=layer: raw(layer, e), k=K_TOP)
        tokens += xb.shape[0]
    dt = time.perf_counter() - t0
    per_layer_tokens = tokens
    sample = (f"{per_layer_tokens} token(s) of the {wl['name']} workload through the oracle's moe_layer "
              f"(raw fp32 experts drawn beforehand, untimed), {dt:.1f} s")
    return {"value": per_layer_tokens / dt, "unit": "tokens/s", "cores": blas if blas > 1 else 1,
            "host_cpus": threads, "kind": "oracle", "sample": sample}


# ------------------------------------------------------------------ workload
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU only: the layer is data-parallel and this build runs "
              "and reports one MI355X (--gpus 1). Multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    ensure_built()
    import ternary_weight_moe_base_amd as tm
    import tmoe_inputs as ti
    from ternary_weight_moe_base_amd import synthetic

    cfg = args.config
    wl = dict(WORKLOADS[cfg])
    K = args.steps if args.steps is not None else wl["steps"]
    W_ = args.warmup if args.warmup is not None else wl["warmup"]
    L = args.layers if args.layers is not None else wl["layers"]
    T = wl["tokens"]
    dev = torch.device("cuda")
    torch.cuda.init()

    t0 = time.perf_counter()
    layers = [synthetic.build_layer(cfg, l, wl["bias"]) for l in range(L)]
    torch.cuda.synchronize()
    log(f"built {L} layers in {time.perf_counter() - t0:.1f} s")

    ws = torch.zeros(tm.moe_workspace_bytes(T, layers[0]), dtype=torch.uint8, device=dev)
    Y = torch.empty((T, H), dtype=torch.float32, device=dev)
    n_steps = W_ + K
    if cfg == 5:
        X = synthetic.activations(cfg, T)
        idx_buf = torch.empty((n_steps * L, T, K_TOP), dtype=torch.int32, device=dev)
    else:
        n_batches = n_steps if cfg == 2 else min(n_steps, 64)
        X = synthetic.activations(cfg, n_batches * T).view(n_batches, T, H)
        idx_buf = torch.empty((n_steps, T, K_TOP), dtype=torch.int32, device=dev)

    def step(i):
        if cfg == 5:
            for l in range(L):
                tm.moe_forward(layers[l], X, None, ws, idx=idx_buf[i * L + l], resid_out=X)
        else:
            tm.moe_forward(layers[i % L], X[i % X.shape[0]], Y, ws, idx=idx_buf[i])

    for i in range(W_):
        step(i)
    torch.cuda.synchronize()

    use_graph = not args.no_graph
    prof_cap = K * (L if cfg == 5 else 1)
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            graph.capture_begin()
            for i in range(W_, W_ + K):
                step(i)
            graph.capture_end()
        torch.cuda.synchronize()
        graph.replay()  # first replay of a fresh graph: untimed
        torch.cuda.synchronize()
    else:
        tm.profile_begin(args.kernel, prof_cap)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W_, W_ + K):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if use_graph:
        # Kernel durations: the same K steps launched eagerly, the selected
        # kernel carrying start/stop events recorded by its own dispatch.
        tm.profile_begin(args.kernel, prof_cap)
        for i in range(W_, W_ + K):
            step(i)
    kern_ms = tm.profile_end(prof_cap)

    ms_per_step = 1e3 * elapsed / K
    layer_passes = K * (L if cfg == 5 else 1)
    tokens_per_layer_s = T * layer_passes / elapsed

    # algorithmic bytes: packed experts (+ scales) with >= 1 routed token, router, X, Y
    idx_h = idx_buf.cpu().numpy()
    if cfg == 5:
        sel = idx_h[W_ * L:(W_ + K) * L]
    else:
        sel = idx_h[W_:W_ + K]
    n_hit = np.array([len(np.unique(s)) for s in sel])
    step_bytes = ROUTER_BYTES + n_hit * EXPERT_BYTES + T * H * 2 + T * H * (2 if cfg == 5 else 4)
    hbm_gbs = float(step_bytes.sum()) / elapsed / 1e9

    # roofline of the selected kernel: algorithmic bytes (or flops) per launch / mean launch time
    P = T * K_TOP
    mean_ms = float(np.mean(kern_ms)) if len(kern_ms) else float("nan")
    if args.kernel == "gateup":
        kb = n_hit * 2 * (PACKED_GU + 4 * I) + T * H * 2 + P * I * 4
        kflops = 4.0 * P * I * H
    elif args.kernel == "down":
        kb = n_hit * (PACKED_D + 4 * H) + P * I * 4 + P * H * 4
        kflops = 2.0 * P * I * H
    elif args.kernel == "router_logits":
        kb = np.full(len(n_hit), ROUTER_BYTES + T * H * 2 + T * E * 4)
        kflops = 2.0 * T * E * H
    else:
        kb = np.full(len(n_hit), np.nan)
        kflops = float("nan")
    mean_kb = float(np.mean(kb))
    if cfg == 4:
        achieved = kflops / (mean_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None}
    else:
        achieved = mean_kb / (mean_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    roof.update({"kernel": args.kernel, "mean_launch_us": mean_ms * 1e3, "launches": int(len(kern_ms)),
                 "algorithmic_bytes_per_launch": mean_kb})

    out = {
        "metric": METRIC,
        "value": tokens_per_layer_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W_,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "tokens_per_step": T, "layers_per_step": L if cfg == 5 else 1,
                   "distinct_layers": L, "hidden": H, "experts": E, "top_k": K_TOP, "moe_intermediate": I,
                   "weights": "ternary, 5 trits/byte, fp32 row scales", "hip_graph": use_graph},
        "achieved_hbm_gbs": hbm_gbs,
        "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": float(np.mean(step_bytes)) * (L if cfg == 5 else 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens if args.cpu_tokens is not None else (6 if cfg == 2 else 8)
        log(f"timing the CPU oracle on {n_tok} token(s)")
        out["cpu_baseline"] = cpu_baseline(cfg, wl, n_tok)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
