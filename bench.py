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
Other workloads (--config): 1 the streamed 2048 -> 512 ternary linear, 3 a
64-token batch with Zipf routing, 4 4096-token prefill, 5 the 24-layer stack
at 256 tokens, 6 one token through the 24-layer stack, 7 the LM head top-16,
8 config 6 with experts in pinned host memory, 9/10/11 one token through the
attention halves / the whole model / the model and its LM head at context 4096.
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
PCIE_PEAK_GBS = 64.0  # host link, PCIe 5.0 x16, one direction
FP64_PEAK_TFLOPS = 78.6  # fp64 vector / matrix
H, I, E, K_TOP = 2048, 512, 256, 8
PACKED_GU = I * ((H + 4) // 5)  # bytes of one gate or up matrix
PACKED_D = H * ((I + 4) // 5)
EXPERT_BYTES = 2 * PACKED_GU + PACKED_D + 4 * (2 * I + H)  # 643,072
ROUTER_BYTES = E * H * 4

WORKLOADS = {
    # the 2048 -> 512 ternary linear, streamed: 2048 distinct 512 x 2048 matrices stacked into one
    # 1,048,576 x 2048 operand (436 MB packed, past the 256 MB last-level cache), 4 tokens per launch
    1: dict(name="ternary_linear_T4_streamed_2048x512x2048", tokens=4, bias=None, layers=1, steps=50, warmup=5,
            linear=True, mats=2048),
    2: dict(name="moe_layer_decode_T1", tokens=1, bias=None, layers=24, steps=2400, warmup=48),
    3: dict(name="moe_layer_decode_T64_zipf1.1", tokens=64, bias="zipf", layers=24, steps=480, warmup=48),
    4: dict(name="moe_layer_prefill_T4096_uniform", tokens=4096, bias="uniform", layers=4, steps=40, warmup=4,
            prof_steps=40, cpu_tokens=256),
    5: dict(name="moe_stack24_T256_residual", tokens=256, bias=None, layers=24, steps=20, warmup=2, stack=True),
    # one token at a time through the same 24-layer stack: per-token decode latency
    6: dict(name="moe_stack24_decode_T1_residual", tokens=1, bias=None, layers=24, steps=100, warmup=4, stack=True,
            model_cfg=5),
    # config 6 with every layer's experts in pinned host memory, read over PCIe on demand
    8: dict(name="moe_stack24_decode_T1_host_experts", tokens=1, bias=None, layers=24, steps=40, warmup=2, stack=True,
            model_cfg=5, host_experts=True),
    # one token through the 24 attention halves (18 sliding-window layers, 6 global) at context 4096
    9: dict(name="attention24_decode_T1_ctx4096", tokens=1, bias=None, layers=24, steps=100, warmup=4, model_cfg=5,
            attention=True, moe=False, context=4096),
    # one token through the whole 24-layer stack, attention then MoE per layer, at context 4096
    10: dict(name="model24_decode_T1_ctx4096", tokens=1, bias=None, layers=24, steps=100, warmup=4, model_cfg=5,
             attention=True, moe=True, context=4096),
    # config 10 plus the output head: the next token's top-16 over the 151,936-token vocabulary
    11: dict(name="model24_lmhead_decode_T1_ctx4096", tokens=1, bias=None, layers=24, steps=100, warmup=4, model_cfg=5,
             attention=True, moe=True, context=4096, head=True),
    # the model's untied bf16 output head (151,936 x 2048, 622 MB) and its top-16, one token per step
    7: dict(name="lm_head_topk16_T1", tokens=1, bias=None, layers=1, steps=400, warmup=10, model_cfg=5, lm_head=True),
}
LMH_K = 16
LMH_KERNELS = ("lmh_logits", "lmh_topk", "lmh_merge")


# kernels each path launches (names of the C ABI's timing hook)
DECODE_KERNELS = ("router_logits", "gateup", "down")  # T <= 3: gate/up routes, down also combines
BATCH_KERNELS = ("router_logits", "router_topk", "group", "gateup", "down", "combine")


def roofline(name, ms, n_hit, T, cfg, bias):
    """Achieved rate of one kernel: algorithmic bytes (or flops) per launch over
    its mean launch duration. Algorithmic bytes count what the step must move:
    packed weights + scales of the experts with a routed token, the fp32 router,
    the layer input X and output Y; intermediates (logits, h, expert outputs)
    are not counted."""
    import numpy as np

    P = T * K_TOP
    mean_s = float(np.mean(ms)) * 1e-3
    stack = WORKLOADS[cfg].get("stack", False)
    x_b, y_b = T * H * 2, T * H * (2 if stack else 4)
    flops = None
    if name == "router_logits":
        b = np.full(len(n_hit), ROUTER_BYTES + x_b + (E * 4 if bias else 0))
        flops, fpeak = 2.0 * T * E * H, FP64_PEAK_TFLOPS
    elif name == "gateup":
        b = n_hit * 2 * (PACKED_GU + 4 * I) + x_b
        flops, fpeak = 4.0 * P * I * H, BF16_PEAK_TFLOPS
    elif name == "down":
        b = n_hit * (PACKED_D + 4 * H)
        flops, fpeak = 2.0 * P * I * H, BF16_PEAK_TFLOPS
    elif name == "combine":
        b = np.full(len(n_hit), y_b + (x_b if stack else 0) + T * K_TOP * 8)
    else:  # top-k, grouping, tiles: index arrays only
        b = np.full(len(n_hit), T * K_TOP * 4 * 4)
    mean_b = float(np.mean(b))
    if WORKLOADS[cfg].get("host_experts") and name in ("gateup", "down"):
        achieved = mean_b / mean_s / 1e9  # the expert bytes cross the host link
        r = {"bound": "pcie", "achieved": achieved, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
             "frac": achieved / PCIE_PEAK_GBS, "traffic": None}
    elif cfg == 4 and flops is not None:
        achieved = flops / mean_s / 1e12
        r = {"bound": "alu" if name == "router_logits" else "mfma", "achieved": achieved, "peak": fpeak, "unit": "TFLOP/s", "frac": achieved / fpeak,
             "traffic": None, "algorithmic_flops_per_launch": flops}
    else:
        achieved = mean_b / mean_s / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    r.update({"kernel": name, "mean_launch_us": mean_s * 1e6, "launches": int(len(ms)),
              "algorithmic_bytes_per_launch": mean_b})
    return r


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="distinct layers to rotate over")
    ap.add_argument("--kernel", default=None, help="kernel whose roofline is reported (default: the dominant one)")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of one HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill record of the default workload")
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
def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(cfg: int, wl: dict, n_tok: int | None, budget_s: float = 12.0, one_core_budget_s: float = 8.0):
    """The CPU oracle, untuned, timed on this host on a bounded sample of the
    workload, twice: with every host core (the reported value) and with one
    core (BLAS limited to one thread; the oracle's other steps are
    single-threaded NumPy anyway). One-token decode: token i through layer
    i mod 24 until the time budget or n_tok tokens. Batched workloads: the
    first `cpu_tokens` tokens of the workload's batch (for the 4096-token
    prefill, 256 tokens, which route to nearly every expert) as one batch
    through layer 0. The inputs a call reads (router, raw fp32 experts it
    routes to) are drawn before the call; only the oracle's moe_layer (which
    ternarizes the routed experts itself) is timed."""
    import numpy as np

    import oracle as O
    import tmoe_inputs as ti

    threads = len(os.sched_getaffinity(0))
    blas = _blas_threads()
    mcfg = wl.get("model_cfg", cfg)
    one = wl["tokens"] == 1
    pool = concurrent.futures.ThreadPoolExecutor(min(16, threads))

    def prepare(layer, xb):
        Wr, b = ti.router_matrix(mcfg, layer), ti.router_bias(mcfg, wl["bias"])
        idx, _, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, K_TOP)
        es = sorted(set(idx.ravel().tolist()))
        mats = dict(zip(es, pool.map(lambda e: tuple(ti.expert_matrix(mcfg, layer, e, m) for m in range(3)), es)))
        return Wr, b, mats

    def timed_run(batches, budget):
        tokens, timed = 0, 0.0
        for layer, xb in batches:
            Wr, b, mats = prepare(layer, xb)
            t0 = time.perf_counter()
            O.moe_layer(xb, Wr, b, lambda e: mats[e], k=K_TOP)
            timed += time.perf_counter() - t0
            tokens += xb.shape[0]
            if timed >= budget:
                break
        return tokens, timed

    if one:
        def batches():
            return ((i % wl["layers"], ti.activations(mcfg, i + 1)[i:i + 1]) for i in range(n_tok or 1000))
        what = "token i through layer i mod 24"
    else:
        n = n_tok or wl.get("cpu_tokens", 8)
        xs = ti.activations(mcfg, wl["tokens"])[:n]

        def batches():
            return iter([(0, xs)])
        what = f"the first {n} tokens of the batch as one call through layer 0"
    tokens, timed = timed_run(batches(), budget_s)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            tokens1, timed1 = timed_run(batches(), one_core_budget_s)
        one_core = {"value": tokens1 / timed1, "unit": "tokens/s", "cores": 1,
                    "sample": f"{tokens1} token(s), {timed1:.1f} s of oracle time"}
    except ImportError:  # pragma: no cover
        one_core = None
    pool.shutdown()
    sample = (f"{tokens} token(s) of the {wl['name']} workload ({what}) through the oracle's moe_layer; "
              f"{timed:.1f} s of oracle time; router and raw fp32 experts drawn beforehand, untimed")
    return {"value": tokens / timed, "unit": "tokens/s", "cores": blas if blas > 1 else 1,
            "host_cpus": threads, "kind": "oracle", "sample": sample, "one_core": one_core}


# ------------------------------------------------------------------ LM head
def cpu_baseline_lm_head(wl: dict, budget_s: float = 12.0):
    """The oracle's lm_head_topk on this host for successive tokens until
    budget_s seconds of oracle time; the table is drawn once beforehand
    (untimed)."""
    import numpy as np

    import oracle as O
    import tmoe_inputs as ti

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    cfg, V = wl["model_cfg"], ti.VOCAB
    with concurrent.futures.ThreadPoolExecutor(min(16, threads)) as ex:
        parts = list(ex.map(lambda v0: ti.lm_head_rows(cfg, v0, min(v0 + 8192, V)), range(0, V, 8192)))
    Wh = np.concatenate(parts)
    x = ti.activations(cfg, 64)
    tokens, timed = 0, 0.0
    for i in range(64):
        t0 = time.perf_counter()
        O.lm_head_topk(x[i:i + 1], Wh, LMH_K)
        timed += time.perf_counter() - t0
        tokens += 1
        if timed >= budget_s:
            break
    sample = (f"{tokens} token(s) of the {wl['name']} workload through the oracle's lm_head_topk over the full "
              f"151,936-token table; {timed:.1f} s of oracle time; the table drawn beforehand, untimed")
    return {"value": tokens / timed, "unit": "tokens/s", "cores": blas if blas > 1 else 1, "host_cpus": threads,
            "kind": "oracle", "sample": sample}


def cpu_baseline_linear(wl: dict, budget_s: float = 12.0):
    """The oracle's ternary_linear on this host, matrix by matrix of the
    streamed operand, until budget_s seconds of oracle time; each matrix is
    drawn and ternarized before its timed call (untimed)."""
    import numpy as np

    import oracle as O
    import tmoe_inputs as ti

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    x = O.bf16_to_f64(ti.activations(1, wl["tokens"]))
    done, timed = 0, 0.0
    for q in range(wl["mats"]):
        t, sc = O.ternarize_absmean(ti.expert_matrix(1, q // 1024, q % 1024, ti.MAT_GATE))
        t0 = time.perf_counter()
        O.ternary_linear(t, sc, x)
        timed += time.perf_counter() - t0
        done += 1
        if timed >= budget_s:
            break
    per_operand = timed / done * wl["mats"]
    sample = (f"{done} of the {wl['mats']} matrices of the {wl['name']} operand through the oracle's ternary_linear "
              f"({wl['tokens']} tokens), {timed:.1f} s of oracle time, scaled to the whole operand; weights drawn "
              f"and ternarized beforehand, untimed")
    return {"value": wl["tokens"] / per_operand, "unit": "tokens/s", "cores": blas if blas > 1 else 1,
            "host_cpus": threads, "kind": "oracle", "sample": sample}


def main_linear(args, wl: dict):
    import numpy as np
    import torch

    ensure_built()
    import ternary_weight_moe_base_amd as tm
    from ternary_weight_moe_base_amd import synthetic

    K = args.steps if args.steps is not None else wl["steps"]
    W_ = args.warmup if args.warmup is not None else wl["warmup"]
    T, mats = wl["tokens"], wl["mats"]
    N = mats * 512
    dev = torch.device("cuda")
    torch.cuda.init()
    t0 = time.perf_counter()
    Pt, sc = synthetic.streamed_linear(1, mats)
    torch.cuda.synchronize()
    log(f"built {mats} matrices in {time.perf_counter() - t0:.1f} s")
    X = synthetic.activations(1, 64 * T).view(64, T, H)
    Y = torch.empty((T, N), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(tm.linear_workspace_bytes(T, H), 16), dtype=torch.uint8, device=dev)

    def step(i):
        tm.ternary_linear(Pt, sc, N, H, X[i % 64], Y, ws)

    for i in range(W_):
        step(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
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
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W_, W_ + K):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    tm.profile_begin("linear", K)
    for i in range(W_, W_ + K):
        step(i)
    ms = tm.profile_end(K)
    torch.cuda.synchronize()
    mean_s = float(np.mean(ms)) * 1e-3
    launch_bytes = Pt.numel() + 4 * N + T * H * 2 + T * N * 4  # packed weights, row scales, X, Y
    achieved = launch_bytes / mean_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": None, "kernel": "ternary_linear", "mean_launch_us": mean_s * 1e6, "launches": int(len(ms)),
            "algorithmic_bytes_per_launch": float(launch_bytes),
            "packed_weight_gbs": Pt.numel() / mean_s / 1e9}
    out = {
        "metric": METRIC, "value": T * K / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W_,
        "ms_per_step": 1e3 * elapsed / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "tokens_per_step": T, "rows": N, "cols": H, "matrices": mats,
                   "weights": "ternary, 5 trits/byte, fp32 row scales", "hip_graph": use_graph},
        "achieved_hbm_gbs": launch_bytes * K / elapsed / 1e9,
        "hbm_frac": launch_bytes * K / elapsed / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": float(launch_bytes),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline_linear(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


ATTN_KERNELS = ("linear", "attention")


def main_attention(args, wl: dict):
    """One-token decode through the 24 attention halves (config 9) or through
    the whole stack, attention then MoE per layer (config 10), with key/value
    caches prefilled to `context` positions by the library's own prefill
    (one 4096-token call per layer, untimed). Step i is the token at position
    context + i; the K timed steps are one captured graph."""
    import numpy as np
    import torch

    ensure_built()
    import ternary_weight_moe_base_amd as tm
    from ternary_weight_moe_base_amd import synthetic

    K = args.steps if args.steps is not None else wl["steps"]
    W_ = args.warmup if args.warmup is not None else wl["warmup"]
    L, ctx, mcfg = wl["layers"], wl["context"], wl["model_cfg"]
    dev = torch.device("cuda")
    torch.cuda.init()
    t0 = time.perf_counter()
    attn = [synthetic.build_attention(mcfg, l, synthetic.is_global_layer(l)) for l in range(L)]
    moe = [synthetic.build_layer(mcfg, l, None) for l in range(L)] if wl["moe"] else None
    caches = []
    xp = synthetic.activations(mcfg, ctx)
    wsp = torch.empty(tm.attention_workspace_bytes(ctx, attn[0]), dtype=torch.uint8, device=dev)
    scratch = torch.empty((ctx, H), dtype=torch.int16, device=dev)
    for l in range(L):
        cap = ctx + W_ + K + 1 if attn[l].window == 0 else attn[l].window + ctx - 1
        kc, vc = tm.kv_cache(attn[l], cap)
        tm.attention_forward(attn[l], xp, 0, kc, vc, wsp, X_out=scratch)  # prefill: fills the cache
        caches.append((kc, vc))
    del wsp, scratch
    torch.cuda.synchronize()
    log(f"built and prefilled {L} layers in {time.perf_counter() - t0:.1f} s")
    X = synthetic.activations(mcfg, W_ + K, layer=1).view(W_ + K, 1, H)
    xw = torch.empty((1, H), dtype=torch.int16, device=dev)
    wsa = torch.empty(tm.attention_workspace_bytes(1, attn[0]), dtype=torch.uint8, device=dev)
    wsm = torch.empty(tm.moe_workspace_bytes(1, moe[0]) if moe else 16, dtype=torch.uint8, device=dev)
    head = wl.get("head", False)
    if head:
        from tmoe_inputs import VOCAB
        table = synthetic.lm_head_table(mcfg)
        wsh = torch.empty(tm.lm_head_workspace_bytes(1, VOCAB, LMH_K), dtype=torch.uint8, device=dev)
        nxt = torch.empty((W_ + K, 1, LMH_K), dtype=torch.int32, device=dev)
        nval = torch.empty((1, LMH_K), dtype=torch.float32, device=dev)

    def step(i):
        for l in range(L):
            tm.attention_forward(attn[l], X[i] if l == 0 else xw, ctx + i, *caches[l], wsa, X_out=xw)
            if moe:
                tm.moe_forward(moe[l], xw, None, wsm, resid_out=xw)
        if head:
            tm.lm_head_topk(xw, table, LMH_K, nxt[i], nval, wsh)

    for i in range(W_):
        step(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
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
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W_, W_ + K):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel durations over the same steps launched again (eagerly, same positions)
    kern = {}
    names = ATTN_KERNELS + (DECODE_KERNELS if moe else ()) + (("lmh_logits",) if head else ())
    cap_n = K * L * 2
    for name in names:
        tm.profile_begin(name, cap_n)
        for i in range(W_, W_ + K):
            step(i)
        ms = tm.profile_end(cap_n)
        if len(ms):
            kern[name] = ms
    torch.cuda.synchronize()
    per_token_us = {n: float(np.sum(v)) * 1e3 / K for n, v in kern.items()}
    # algorithmic bytes per launch
    n_glob = sum(1 for a in attn if a.window == 0)
    keys_glob = ctx + W_ + (K - 1) / 2 + 1  # mean visible keys of a global layer over the timed steps
    kv_bytes = 2 * 4 * 128 * 4  # key + value of one position, all 4 heads, fp32
    att_b = (n_glob * keys_glob + (L - n_glob) * 512) / L * kv_bytes
    lin_b = (tm.tiled_bytes(3072, H) + 4 * 3072 + tm.tiled_bytes(H, H) + 4 * H) / 2 + H * 2
    dom = args.kernel if args.kernel else max(per_token_us, key=per_token_us.get)
    if dom == "attention":
        b = att_b
    elif dom == "linear":
        b = lin_b
    elif dom == "gateup":
        b = 8 * 2 * (PACKED_GU + 4 * I) + H * 2
    elif dom == "down":
        b = 8 * (PACKED_D + 4 * H)
    elif dom == "lmh_logits":
        b = 151936 * H * 2 + H * 2
    else:
        b = ROUTER_BYTES + H * 2
    mean_s = float(np.mean(kern[dom])) * 1e-3
    roof = {"bound": "hbm", "achieved": b / mean_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": b / mean_s / 1e9 / HBM_PEAK_GBS, "traffic": None, "kernel": dom, "mean_launch_us": mean_s * 1e6,
            "launches": int(len(kern[dom])), "algorithmic_bytes_per_launch": float(b),
            "kernels_us_per_token": {n: round(v, 3) for n, v in per_token_us.items()}}
    out = {
        "metric": METRIC, "value": K / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W_,
        "ms_per_step": 1e3 * elapsed / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "tokens_per_step": 1, "layers_per_step": L, "context": ctx,
                   "global_layers": n_glob, "sliding_window": 512, "heads": "16 query, 4 key/value, 128 wide",
                   "parts": ("attention + MoE" if moe else "attention") + (" + LM head top-16" if head else ""),
                   "hip_graph": use_graph},
        "token_latency_us": 1e6 * elapsed / K,
        "roofline": roof,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main_lm_head(args, wl: dict):
    import numpy as np
    import torch

    ensure_built()
    import ternary_weight_moe_base_amd as tm
    import tmoe_inputs as ti
    from ternary_weight_moe_base_amd import synthetic

    K = args.steps if args.steps is not None else wl["steps"]
    W_ = args.warmup if args.warmup is not None else wl["warmup"]
    T, V, k = wl["tokens"], ti.VOCAB, LMH_K
    dev = torch.device("cuda")
    torch.cuda.init()
    Wd = synthetic.lm_head_table(wl["model_cfg"])
    X = synthetic.activations(wl["model_cfg"], 64 * T).view(64, T, H)
    idx = torch.empty((K + W_, T, k), dtype=torch.int32, device=dev)
    val = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = torch.zeros(tm.lm_head_workspace_bytes(T, V, k), dtype=torch.uint8, device=dev)

    def step(i):
        tm.lm_head_topk(X[i % 64], Wd, k, idx[i], val, ws)

    for i in range(W_):
        step(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
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
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W_, W_ + K):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    kern = {}
    for name in LMH_KERNELS:
        tm.profile_begin(name, K)
        for i in range(W_, W_ + K):
            step(i)
        ms = tm.profile_end(K)
        if len(ms):
            kern[name] = ms
    torch.cuda.synchronize()
    per_step_us = {n: float(np.mean(v)) * 1e3 for n, v in kern.items()}
    table_bytes = V * H * 2
    step_bytes = table_bytes + T * H * 2 + T * k * 8
    mean_s = float(np.mean(kern["lmh_logits"])) * 1e-3
    achieved = (table_bytes + T * H * 2) / mean_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": None, "kernel": "lmh_logits", "mean_launch_us": mean_s * 1e6, "launches": int(len(kern["lmh_logits"])),
            "algorithmic_bytes_per_launch": float(table_bytes + T * H * 2),
            "kernels_us_per_step": {n: round(v, 3) for n, v in per_step_us.items()}}
    out = {
        "metric": METRIC, "value": T * K / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W_,
        "ms_per_step": 1e3 * elapsed / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "tokens_per_step": T, "vocab": V, "hidden": H, "top_k": k,
                   "table": "bf16 [151936][2048], untied output embedding", "hip_graph": use_graph},
        "achieved_hbm_gbs": step_bytes * K / elapsed / 1e9,
        "hbm_frac": step_bytes * K / elapsed / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": float(step_bytes),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline_lm_head(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ workload
EVICT_BYTES = 1 << 30  # streamed between the untimed and the timed replay (4x the 256 MB last-level cache)


def evict_caches(buf) -> None:
    """Reads and writes `buf` (EVICT_BYTES) so that nothing the timed steps read
    is still in the L2 or last-level caches when they start."""
    import torch

    buf.add_(1)
    torch.cuda.synchronize()


def run_layer(args, cfg: int, K: int, W_: int, L: int, evict) -> dict:
    """One MoE-layer workload (configs 2-6, 8): builds its layers, runs W_
    warm-up steps, captures the K timed steps in one HIP graph, replays it
    once untimed, evicts the caches, replays it timed; then times each kernel
    over the same steps launched eagerly (at most `prof_steps` of them).
    Returns the JSON record of the run (no CPU baseline)."""
    import numpy as np
    import torch

    import ternary_weight_moe_base_amd as tm
    from ternary_weight_moe_base_amd import synthetic

    wl = dict(WORKLOADS[cfg])
    T = wl["tokens"]
    stack = wl.get("stack", False)
    mcfg = wl.get("model_cfg", cfg)  # seeds of the model's weights and activations
    dev = torch.device("cuda")

    t0 = time.perf_counter()
    layers = [synthetic.build_layer(mcfg, l, wl["bias"]) for l in range(L)]
    torch.cuda.synchronize()
    if wl.get("host_experts"):  # move each layer's experts to pinned host memory, free the device copies
        for l in range(L):
            layers[l] = tm.experts_on_host(layers[l])
        torch.cuda.empty_cache()
    log(f"{wl['name']}: built {L} layers in {time.perf_counter() - t0:.1f} s")

    ws = torch.zeros(tm.moe_workspace_bytes(T, layers[0]), dtype=torch.uint8, device=dev)
    Y = torch.empty((T, H), dtype=torch.float32, device=dev)
    n_steps = W_ + K
    if cfg == 5:
        X = synthetic.activations(mcfg, T)
        idx_buf = torch.empty((n_steps * L, T, K_TOP), dtype=torch.int32, device=dev)
    elif cfg in (6, 8):
        X = synthetic.activations(mcfg, n_steps).view(n_steps, 1, H)  # token i = row i of the stack batch
        Xw = torch.empty((1, H), dtype=X.dtype, device=dev)  # the token's residual stream
        idx_buf = torch.empty((n_steps * L, T, K_TOP), dtype=torch.int32, device=dev)
    else:
        n_batches = n_steps if cfg == 2 else min(n_steps, 64 if T < 4096 else 16)
        X = synthetic.activations(cfg, n_batches * T).view(n_batches, T, H)
        idx_buf = torch.empty((n_steps, T, K_TOP), dtype=torch.int32, device=dev)

    def step(i):
        if cfg == 5:
            for l in range(L):
                tm.moe_forward(layers[l], X, None, ws, idx=idx_buf[i * L + l], resid_out=X)
        elif cfg in (6, 8):
            for l in range(L):
                tm.moe_forward(layers[l], X[i] if l == 0 else Xw, None, ws, idx=idx_buf[i * L + l], resid_out=Xw)
        else:
            tm.moe_forward(layers[i % L], X[i % X.shape[0]], Y, ws, idx=idx_buf[i])

    for i in range(W_):
        step(i)
    torch.cuda.synchronize()

    use_graph = not args.no_graph
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
    evict()  # the timed steps start with cold caches, whatever K is

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W_, W_ + K):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-kernel durations: the same steps launched again (eagerly), one kernel
    # at a time carrying start/stop events recorded by its own dispatch on the
    # stream it runs on.
    prof_steps = min(K, wl.get("prof_steps", K))
    prof_cap = prof_steps * (L if stack else 1)
    kern = {}
    for name in (DECODE_KERNELS if T <= 3 else BATCH_KERNELS):
        evict()
        tm.profile_begin(name, prof_cap)
        for i in range(W_, W_ + prof_steps):
            step(i)
        ms = tm.profile_end(prof_cap)
        if len(ms):
            kern[name] = ms
    torch.cuda.synchronize()

    ms_per_step = 1e3 * elapsed / K
    layer_passes = K * (L if stack else 1)
    tokens_per_layer_s = T * layer_passes / elapsed

    # algorithmic bytes: packed experts (+ scales) with >= 1 routed token, router, X, Y
    idx_h = idx_buf.cpu().numpy()
    sel = idx_h[W_ * L:(W_ + K) * L] if stack else idx_h[W_:W_ + K]
    n_hit = np.array([len(np.unique(s)) for s in sel])
    step_bytes = ROUTER_BYTES + n_hit * EXPERT_BYTES + T * H * 2 + T * H * (2 if stack else 4)
    hbm_gbs = float(step_bytes.sum()) / elapsed / 1e9

    # roofline of the dominant kernel (largest total time per step)
    prof_passes = prof_steps * (L if stack else 1)
    per_step_us = {n: float(np.sum(v)) * 1e3 / prof_passes for n, v in kern.items()}
    dom = args.kernel if args.kernel else max(per_step_us, key=per_step_us.get)
    sel_prof = sel[:prof_passes]
    n_hit_prof = np.array([len(np.unique(s)) for s in sel_prof])
    roof = roofline(dom, kern[dom], n_hit_prof, T, cfg, bias=wl["bias"] is not None)
    roof["kernels_us_per_layer"] = {n: round(v, 3) for n, v in per_step_us.items()}

    extra = {}
    if stack and T == 1:  # one token through the whole stack per step: its latency
        extra = {"token_latency_us": 1e6 * elapsed / K, "stack_tokens_per_s": K / elapsed}
    return {
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
        "config": {"workload": wl["name"], "tokens_per_step": T, "layers_per_step": L if stack else 1,
                   "distinct_layers": L, "hidden": H, "experts": E, "top_k": K_TOP, "moe_intermediate": I,
                   "weights": "ternary, 5 trits/byte, fp32 row scales", "hip_graph": use_graph,
                   "expert_memory": "pinned host, read over PCIe" if wl.get("host_experts") else "hbm",
                   "timed_replay": f"cold: {EVICT_BYTES >> 20} MiB streamed after the untimed replay",
                   "kernel_timing_steps": prof_steps},
        "achieved_hbm_gbs": hbm_gbs,
        "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": float(np.mean(step_bytes)) * (L if stack else 1),
        "roofline": roof,
        **extra,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU only: the layer is data-parallel, and this benchmark "
              "runs and reports one MI355X (--gpus 1). Multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    ensure_built()

    cfg = args.config
    wl = dict(WORKLOADS[cfg])
    if wl.get("lm_head"):
        return main_lm_head(args, wl)
    if wl.get("linear"):
        return main_linear(args, wl)
    if wl.get("attention"):
        return main_attention(args, wl)
    K = args.steps if args.steps is not None else wl["steps"]
    W_ = args.warmup if args.warmup is not None else wl["warmup"]
    L = args.layers if args.layers is not None else wl["layers"]
    torch.cuda.init()
    evict_buf = torch.zeros(EVICT_BYTES // 4, dtype=torch.float32, device="cuda")
    out = run_layer(args, cfg, K, W_, L, lambda: evict_caches(evict_buf))
    # the metric's other half: the 4096-token prefill, with the same step counts
    prefill = None
    if cfg == 2 and not args.no_prefill:
        torch.cuda.empty_cache()
        wp = WORKLOADS[4]
        Kp = args.steps if args.steps is not None else wp["steps"]
        Wp = args.warmup if args.warmup is not None else wp["warmup"]
        pf = run_layer(args, 4, Kp, Wp, wp["layers"], lambda: evict_caches(evict_buf))
        prefill = {key: pf[key] for key in ("value", "unit", "steps", "warmup", "ms_per_step", "config", "roofline",
                                            "achieved_hbm_gbs", "hbm_frac", "algorithmic_bytes_per_step")}
        prefill["workload"] = pf["config"]["workload"]
    del evict_buf
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_tokens)
        if prefill is not None:
            prefill["cpu_baseline"] = cpu_baseline(4, WORKLOADS[4], None)
    else:
        out["cpu_baseline"] = None
        if prefill is not None:
            prefill["cpu_baseline"] = None
    if prefill is not None:
        out["prefill"] = prefill
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
