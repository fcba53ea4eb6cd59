"""Benchmark of the INT4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode1|decode4|decode64|prefill512|prefill8192]

A step is one forward of the whole layer (router, top-k, permutation, gate/up
projection with SiLU-gate, down projection with the weighted combine) over one
batch of synthetic tokens.  Decode configs rotate over 48 resident layers
(hidden 2560, 512 experts, top-10, intermediate 640, INT4 group 128; 62 GB),
each with its own seeded weights and activations, so every step streams its
weights from HBM rather than from the 256 MB last-level cache.  Inputs are
resident in HBM before timing starts.

Prints one JSON line (rank 0).  `roofline` describes the dominant kernel,
timed live with HIP events recorded around it on the stream it runs on;
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s vs MI355X peak"

CONFIGS = {
    "decode1": dict(tokens=1, layers=48, zipf=None, shared=False),
    "decode4": dict(tokens=4, layers=48, zipf=None, shared=False),
    "decode64": dict(tokens=64, layers=48, zipf=None, shared=False),
    "prefill512": dict(tokens=512, layers=16, zipf=1.1, shared=False),
    "prefill8192": dict(tokens=8192, layers=4, zipf=None, shared=True),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="decode1", choices=sorted(CONFIGS))
    p.add_argument("--layers", type=int, default=0, help="resident layers (0: config default)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_moe_router_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer would shard by experts across GPUs, which is not implemented here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_moe_router_amd import _binding as B
    from quantized_moe_router_amd import accounting as acc
    from quantized_moe_router_amd import synth
    from quantized_moe_router_amd.layer import MoeInt4Layer

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    B.lib()
    cfg = dict(CONFIGS[args.config])
    if args.layers:
        cfg["layers"] = args.layers
    T, L = cfg["tokens"], cfg["layers"]
    shape = synth.LayerShape(tokens=T)
    H, E, I, k = shape.hidden, shape.experts, shape.inter, shape.top_k
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- resident layers and activations (generated on the device) ----
    layers, xs = [], []
    shared = None
    if cfg["shared"]:
        sh = synth.make_shared(H, seed=104729)
        shared = {kk: (torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
                       if isinstance(v, np.ndarray) else v) for kk, v in sh.items()}
    for l in range(L):
        w = synth.device_weights(shape, seed=l, device=dev)
        x = synth.device_activations(shape, seed=1000 + l, device=dev)
        if cfg["zipf"] is not None:
            # bias feature: x[:, H-1] = 1, router[e, H-1] = -s*ln(rank_e)
            g = torch.Generator(device="cpu").manual_seed(7919 + l)
            rank = torch.randperm(E, generator=g).double() + 1.0
            w["router_w"][:, H - 1] = (-cfg["zipf"] * torch.log(rank)).to(torch.bfloat16).view(torch.int16).to(dev)
            x[:, H - 1] = torch.tensor(1.0, dtype=torch.bfloat16).view(torch.int16)
        layers.append(MoeInt4Layer(w, k, shared=shared))
        xs.append(x)
    ws = layers[0].workspace(T)
    for lay in layers:
        lay._ws[(T, None)] = ws
    out = torch.empty(T, H, dtype=torch.int16, device=dev)

    def step(i, events=None):
        lay = layers[i % L]
        w = lay.w
        if events is None:
            B.moe_int4_forward(xs[i % L], w["router_w"], w["w13_packed"], w["w13_scales"], w["w2_packed"],
                               w["w2_scales"], k, out, lay.shape(T), lay._shared_c, ws)
        else:
            B.moe_int4_forward_traced(xs[i % L], w["router_w"], w["w13_packed"], w["w13_scales"],
                                      w["w2_packed"], w["w2_scales"], k, out, lay.shape(T), lay._shared_c,
                                      ws, events)

    # ---- exact algorithmic work: distinct experts touched per layer ----
    distinct = []
    for l in range(L):
        r = layers[l].route(xs[l])
        distinct.append(int((r["counts"] > 0).sum().item()))
    torch.cuda.synchronize()

    # ---- warmup (eager), then the timed region: replays of captured HIP graphs ----
    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    G = min(L, K)
    graphs = []
    for start, n in [(W, G), (W + (K // G) * G, K % G)]:
        if n == 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(start + i)
        graphs.append((g, n))
    torch.cuda.synchronize()
    # the full graph holds G consecutive steps (all L layers once when K >= L); the
    # optional second graph holds the K mod G remaining steps
    plan = [graphs[0]] * (K // G) + ([graphs[1]] if K % G else [])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for g, _ in plan:
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    assert sum(n for _, n in plan) == K
    ms_per_step = wall / K * 1e3
    tokens_per_s = T * K / wall

    # ---- stage breakdown: eager traced forwards (events around each stage) ----
    NS = max(L, 2 * L if T <= 64 else L)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(NS)]
    for e4 in evs:                  # torch creates the underlying hipEvent on first record
        for e in e4:
            e.record()
    torch.cuda.synchronize()
    for i in range(NS):
        step(i, evs[i])
    torch.cuda.synchronize()
    st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(NS)]) * 1e3
    route_us, w13_us, w2_us = st.mean(axis=0)
    layer_us = gpu_ms * 1e3 / K      # device time per step inside the graph replays

    # bytes / flops per step (averaged over the layers the timed steps visited)
    visited = [(W + i % G) % L for i in range(K)]
    dist = np.array([distinct[l] for l in visited], dtype=np.float64)
    sh_bytes = acc.shared_int6_bytes() if cfg["shared"] else 0
    layer_bytes = np.mean([acc.layer_bytes(T, d, shared_bytes=sh_bytes) for d in dist])
    expert_w13 = 2 * I * H // 2 + 2 * I * (H // 128) * 2
    w13_bytes = float(np.mean(dist)) * expert_w13 + T * H * 2 + T * k * I * 2
    flops = acc.layer_flops(T, shared_inter=640 if cfg["shared"] else 0)
    w13_flops = 2 * T * k * 2 * I * H

    decode = T <= 64
    if decode:
        achieved = w13_bytes / (w13_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "w13_slot_kernel (top-k + gate/up INT4 dequant GEMV + SiLU-gate)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": round(w13_bytes)}
    else:
        achieved = w13_flops / (w13_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": "gate/up projection stage",
                "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": w13_flops}
    trf = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(trf):
        with open(trf) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash():
            roof["traffic"] = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "w4a16 (int4 weights, bf16 activations, fp32 accumulation)",
        "data": "synthetic (seeded, device-generated weights and activations)",
        "config": {"workload": f"{args.config}: one MoE layer forward per step, T={T} tokens, "
                               f"hidden {H}, {E} experts, top-{k}, intermediate {I}, INT4 group 128"
                               + (", Zipf(1.1) routing skew" if cfg["zipf"] else "")
                               + (", INT6 shared expert" if cfg["shared"] else "")
                               + f"; {L} resident layers rotated",
                   "tokens": T, "layers_resident": L},
        "layer": {"device_us": round(layer_us, 3), "timing": "HIP-graph replay, events around the replays",
                  "stages_us_eager": {"route": round(route_us, 2),
                  "gate_up": round(w13_us, 2), "down_combine": round(w2_us, 2)},
                  "distinct_experts": round(float(dist.mean()), 2),
                  "algorithmic_bytes": round(layer_bytes), "hbm_gbs": round(layer_bytes / (layer_us * 1e-6) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "flops": flops, "tflops": round(flops / (layer_us * 1e-6) / 1e12, 3)},
        "roofline": roof,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers[0], xs, T, k, args.cpu_seconds, synth)
    print(json.dumps(result), flush=True)


def cpu_baseline(layer, xs, T, k, budget_s, synth):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    first layer's weights with the benchmark's activations, whole tokens."""
    import numpy as np

    import oracle
    w = layer.w
    host = {"router_w": synth.to_host(w["router_w"]), "w13_packed": synth.to_host(w["w13_packed"]),
            "w13_scales": synth.to_host(w["w13_scales"]), "w2_packed": synth.to_host(w["w2_packed"]),
            "w2_scales": synth.to_host(w["w2_scales"]), "top_k": k, "group": 128}
    if layer.shared is not None:
        host["shared"] = {kk: (synth.to_host(v) if hasattr(v, "cpu") else v) for kk, v in layer.shared.items()}
    n_tok = 0
    t0 = time.perf_counter()
    i = 0
    while True:
        n = min(T, 8)                   # whole tokens, a few per call at most
        host["x"] = synth.to_host(xs[i % len(xs)][:n])
        oracle.forward(host)
        n_tok += n
        i += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(n_tok / el, 3), "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{n_tok} whole tokens (the first min(T, 8) of each of the benchmark's T={T} "
                      f"activation sets; routing, experts, combine), layer 0 weights, {el:.1f} s"}


if __name__ == "__main__":
    main()
