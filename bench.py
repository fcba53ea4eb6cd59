"""Benchmark of the INT4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config prefill8192|prefill512|decode1|decode4|decode64|quantize64|lmhead1|hc1|hc512]

A step is one forward of the whole layer (router, top-k, permutation, gate/up
projection with SiLU-gate, down projection with the weighted combine, and the
INT6 shared expert where the workload has one) over one batch of synthetic
tokens.  The default workload is the largest single-GPU one: 8192 tokens
through the real-shape layer (hidden 2560, 512 experts, top-10, intermediate
640, INT4 group 128) plus the always-on INT6 shared expert, rotating over 4
resident layers.  Decode configs rotate over 48 resident layers (62 GB), each
with its own seeded weights and activations, so every step streams its
weights from HBM rather than from the 256 MB last-level cache.  Inputs are
resident in HBM before timing starts.

The default run also measures, as the extra key `decode48x4`, one decode step
of the whole 48-layer stack: 4 tokens through all 48 resident layers in
sequence, fresh activations per layer, reported as sustained HBM GB/s over
the bytes the method must read (router rows, every touched expert once,
activations, outputs).

Timed region: exactly K steps replayed from captured HIP graphs, bracketed by
events.  Per-stage times come from a second pass over the same K steps, run
eagerly behind a short spin kernel (so the host's enqueue never starves the
GPU) with timing-only events between the stages on the launch stream.

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
    # the load-time quantizer (not the layer): 64 experts' bf16 gate/up and
    # down weights at the real shape per step
    "quantize64": dict(experts=64),
    # INT8 W8A16 linear layers (not the MoE layer): lm_head [248320, 2560]
    # group 128 at decode, two resident copies used alternately; the
    # hyper-connection mixers down [320, 10240] + up [10240, 320] group 64,
    # rotating over `pairs` resident pairs (96 per token in the model: two
    # per decoder layer, 48 layers)
    "lmhead1": dict(kind="int8", tokens=1, n=248320, k=2560, group=128, copies=2),
    "hc1": dict(kind="int8hc", tokens=1, pairs=96),
    "hc512": dict(kind="int8hc", tokens=512, pairs=16),
}
VALU_PEAK_TOPS = 39.3        # MI355X vector ALU, non-packed fp32 lane operations per second (T)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="prefill8192", choices=sorted(CONFIGS))
    p.add_argument("--no-decode48", action="store_true",
                   help="skip the 48-layer decode step measured beside the default workload")
    p.add_argument("--decode48-steps", type=int, default=20)
    p.add_argument("--layers", type=int, default=0, help="resident layers (0: config default)")
    p.add_argument("--tokens", type=int, default=0,
                   help="tokens per step (0: config default); for sweeps over the batch size")
    p.add_argument("--group", type=int, default=128, choices=(64, 128),
                   help="INT4 group of the routed experts (MoE configs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="also run 4 plain device copies of MIB MiB (reference for memory counters)")
    return p.parse_args()


class TimingEvents:
    """hipEvents created with hipEventDisableSystemFence, on the HIP runtime this
    process already uses (torch's).  A default event performs a system-scope
    fence when it is recorded, which costs microseconds per record on this
    part; a timing-only event does not."""

    FLAG = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self.ct = ctypes
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        self.hip = ctypes.CDLL(path)

    def create(self) -> int:
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.FLAG)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev.value

    def record(self, ev: int, stream: int) -> None:
        rc = self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a: int, b: int) -> float:
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value


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
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
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
    if args.config == "quantize64":
        return bench_quantize(args)
    if CONFIGS[args.config].get("kind", "").startswith("int8"):
        return bench_int8(args)
    cfg = dict(CONFIGS[args.config])
    if args.layers:
        cfg["layers"] = args.layers
    if args.tokens:
        cfg["tokens"] = args.tokens
    T, L = cfg["tokens"], cfg["layers"]
    shape = synth.LayerShape(tokens=T, group=args.group)
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
        layers.append(MoeInt4Layer(w, k, group=args.group, shared=shared))
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

    if args.copy_calibration:
        # a plain copy of known size: each launch reads and writes exactly n bytes
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- exact algorithmic work: distinct experts touched per layer ----
    distinct = []
    for l in range(L):
        r = layers[l].route(xs[l])
        distinct.append(int((r["counts"] > 0).sum().item()))
    torch.cuda.synchronize()

    # ---- warmup (eager) ----
    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps replayed from captured HIP graphs ----
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
    assert sum(n for _, n in plan) == K
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ga.record()
    for g, _ in plan:
        g.replay()
    gb.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ga.elapsed_time(gb)
    ms_per_step = gpu_ms / K
    tokens_per_s = T * K / (gpu_ms * 1e-3)

    # ---- stage timing: K traced forwards queued behind a spin kernel ----
    # The spin keeps the GPU busy while the host enqueues all K steps, so they
    # run back to back; timing-only events on the launch stream mark every
    # stage of every step (each event adds a little time between stages, not
    # inside them).
    TE = TimingEvents()
    stream = torch.cuda.current_stream().cuda_stream
    evs = [[TE.create() for _ in range(4)] for _ in range(K)]
    ev0, ev1 = TE.create(), TE.create()
    torch.cuda.synchronize()
    t_enq = time.perf_counter()
    for i in range(min(W, 8)):
        step(i, evs[i])
    t_enq = (time.perf_counter() - t_enq) / max(1, min(W, 8))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sa.record(); torch.cuda._sleep(1_000_000); sb.record(); torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(sa.elapsed_time(sb), 1e-3)
    spin = int(cycles_per_ms * (K * t_enq * 1e3 * 1.5 + 2.0))
    torch.cuda.synchronize()
    torch.cuda._sleep(spin)
    TE.record(ev0, stream)
    for i in range(K):
        step(W + i, evs[i])
    TE.record(ev1, stream)
    torch.cuda.synchronize()
    traced_us = TE.ms(ev0, ev1) * 1e3 / K
    st = np.array([[TE.ms(evs[i][j], evs[i][j + 1]) for j in range(3)] for i in range(K)]) * 1e3
    route_us, w13_us, w2_us = st.mean(axis=0)

    # bytes / flops per step (averaged over the layers the timed steps visited)
    visited = [(W + i) % L for i in range(K)]
    dist = np.array([distinct[l] for l in visited], dtype=np.float64)
    d_mean = float(np.mean(dist))
    sh_bytes = acc.shared_int6_bytes() if cfg["shared"] else 0
    layer_bytes = np.mean([acc.layer_bytes(T, d, group=args.group, shared_bytes=sh_bytes) for d in dist])
    S = T * k
    expert_w13 = 2 * I * H // 2 + 2 * I * (H // args.group) * 2
    expert_w2 = H * I // 2 + H * (I // args.group) * 2
    stage_bytes = {"route": acc.router_bytes() + T * H * 2,
                   "gate_up": d_mean * expert_w13 + T * H * 2 + S * I * 2,
                   "down_combine": d_mean * expert_w2 + S * I * 2 + T * H * 2 + sh_bytes}
    flops = acc.layer_flops(T, shared_inter=640 if cfg["shared"] else 0)
    w13_flops = 2 * S * 2 * I * H
    stage_us = {"route": route_us, "gate_up": w13_us, "down_combine": w2_us}
    layer_us = ms_per_step * 1e3

    decode = T <= 16
    kernels = {"route": "router_kernel (router GEMV; top-k in one extra routing workgroup)",
               "gate_up": "w13_slot_kernel (INT4 gate/up dequant GEMV + SiLU-gate)",
               "down_combine": ("w2_rows_kernel (INT4 down dequant GEMV + weighted combine)" if T == 1 else
                                "w2_slot_kernel + w2_combine_kernel (INT4 down dequant GEMV per slot, then the "
                                "weighted combine)")}
    if decode:
        dom = max(stage_us, key=stage_us.get)
        achieved = stage_bytes[dom] / (stage_us[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kernels[dom],
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": round(stage_bytes[dom]),
                "launch_us": round(stage_us[dom], 3)}
        trf_key = dom
    else:
        achieved = w13_flops / (w13_us * 1e-6) / 1e12
        # the whole-expert GEMM runs from 64 slots per expert on average at group 128
        big = S >= 64 * E
        kname = ("moe_gemm_big_kernel<kRoutedW13> (whole-expert gate/up grouped GEMM: one workgroup per "
                 "chunk of up to 192 rows of one expert and 256 weight rows, fp16 MFMA 32x32x16 on INT4 "
                 "weights dequantised exactly in registers, SiLU-gate epilogue)" if big else
                 "moe_gemm_kernel<kRoutedW13> (gate/up grouped GEMM over 128- or 64-row tiles of sorted "
                 "rows, fp16 MFMA 32x32x16, INT4 weight groups staged through LDS, SiLU-gate epilogue)")
        roof = {"bound": "mfma", "kernel": kname,
                "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": w13_flops,
                "algorithmic_bytes_per_launch": round(stage_bytes["gate_up"]),
                "launch_us": round(w13_us, 3)}
        trf_key = "gate_up"
    trf = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(trf):
        with open(trf) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash() and trf_key in tr.get("stages", {}):
            roof["traffic"] = tr["stages"][trf_key]

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
        "dtype": ("w4a16: int4 weights, bf16 router and activations, fp32 accumulation (GEMV path)"
                  if decode else
                  "w4a16 on fp16 MFMA: int4 weights dequantised exactly to fp16, activations converted "
                  "to fp16, bf16 router MFMA, fp32 accumulation"),
        "data": "synthetic (seeded, device-generated weights and activations)",
        "config": {"workload": f"{args.config}: one MoE layer forward per step, T={T} tokens, "
                               f"hidden {H}, {E} experts, top-{k}, intermediate {I}, INT4 group {args.group}"
                               + (", Zipf(1.1) routing skew" if cfg["zipf"] else "")
                               + (", INT6 shared expert" if cfg["shared"] else "")
                               + f"; {L} resident layers rotated",
                   "tokens": T, "layers_resident": L},
        "layer": {"device_us": round(layer_us, 3),
                  "timing": "HIP-graph replay of the K steps, events around the replays",
                  "stage_timing": "K traced forwards queued behind a spin kernel, timing-only events "
                                  "between the stages on the launch stream",
                  "traced_us_per_step": round(traced_us, 3),
                  "stages_us": {kk: round(v, 2) for kk, v in stage_us.items()},
                  "stages_gbs": {kk: round(stage_bytes[kk] / (stage_us[kk] * 1e-6) / 1e9, 1) for kk in stage_us},
                  "distinct_experts": round(d_mean, 2),
                  "algorithmic_bytes": round(layer_bytes), "hbm_gbs": round(layer_bytes / (layer_us * 1e-6) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "flops": flops, "tflops": round(flops / (layer_us * 1e-6) / 1e12, 3),
                  "wall_s": round(wall, 4)},
        "roofline": roof,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers[0], xs, T, k, args.cpu_seconds, synth)
    if args.config == "prefill8192" and not args.no_decode48 and not args.layers and not args.tokens:
        del layers, xs, ws, out
        torch.cuda.empty_cache()
        result["decode48x4"] = bench_decode48(args)
    print(json.dumps(result), flush=True)


def bench_decode48(args, T=4, L=48):
    """One decode step of a 48-layer stack: T tokens through all L resident
    layers in sequence (each layer its own seeded weights and fresh
    activations), replayed from one captured HIP graph per step.  Returns
    the time per step and the sustained HBM rate over the algorithmic bytes
    (router rows, each touched expert once, activations in and out)."""
    import numpy as np
    import torch

    from quantized_moe_router_amd import _binding as B
    from quantized_moe_router_amd import accounting as acc
    from quantized_moe_router_amd import synth
    from quantized_moe_router_amd.layer import MoeInt4Layer

    dev = torch.device("cuda:0")
    shape = synth.LayerShape(tokens=T)
    k = shape.top_k
    layers, xs = [], []
    for l in range(L):
        layers.append(MoeInt4Layer(synth.device_weights(shape, seed=l, device=dev), k))
        xs.append(synth.device_activations(shape, seed=1000 + l, device=dev))
    ws = layers[0].workspace(T)
    out = torch.empty(T, shape.hidden, dtype=torch.int16, device=dev)
    distinct = []
    for l in range(L):
        r = layers[l].route(xs[l])
        distinct.append(int((r["counts"] > 0).sum().item()))
    step_bytes = sum(acc.layer_bytes(T, d) for d in distinct)

    def step():
        for l in range(L):
            lay = layers[l]
            w = lay.w
            B.moe_int4_forward(xs[l], w["router_w"], w["w13_packed"], w["w13_scales"], w["w2_packed"],
                               w["w2_scales"], k, out, lay.shape(T), None, ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    K = max(1, args.decode48_steps)
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    for _ in range(K):
        g.replay()
    gb.record()
    torch.cuda.synchronize()
    ms = ga.elapsed_time(gb) / K
    gbs = step_bytes / (ms * 1e-3) / 1e9
    status = B.workspace_status(ws)
    del g, layers, xs, ws
    torch.cuda.empty_cache()
    return {"workload": f"decode step over {L} resident layers in sequence, T={T} tokens per layer, "
                        "hidden 2560, 512 experts, top-10, intermediate 640, INT4 group 128, "
                        "fresh activations per layer",
            "steps": K, "us_per_step": round(ms * 1e3, 2), "us_per_layer": round(ms * 1e3 / L, 3),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algorithmic_bytes_per_step": int(step_bytes),
            "distinct_experts_per_layer": round(float(np.mean(distinct)), 2),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "timing": "HIP-graph replay of the 48-layer step, events around the replays",
            "workspace_status": status}


def bench_quantize(args):
    """The load-time INT4 quantizer on 64 experts' weights per step: gate/up
    [64 * 2I, H] and down [64 * H, I] bf16, N(0, 0.02) with 0.1 % outliers x15
    (generated on the device).  Work per weight: 20 candidate clips, each
    costing at least a multiply, a rounding, a residual FMA and a squared-error
    FMA (4 vector operations), so 80 operations per weight against the
    non-packed fp32 vector rate."""
    import numpy as np
    import torch

    from quantized_moe_router_amd import _binding as B
    from quantized_moe_router_amd import synth

    E, H, I = CONFIGS["quantize64"]["experts"], 2560, 640
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(4242)
    mats = []
    for rows, cols in ((E * 2 * I, H), (E * H, I)):
        w = torch.randn(rows, cols, generator=g, device=dev) * 0.02
        mask = torch.rand(rows, cols, generator=g, device=dev) < 1e-3
        w = torch.where(mask, w * 15.0, w)
        wb = w.to(torch.bfloat16).view(torch.int16).contiguous()
        del w, mask
        packed = torch.empty(rows, cols // 8, dtype=torch.int32, device=dev)
        scales = torch.empty(rows, cols // 128, dtype=torch.int16, device=dev)
        mats.append((wb, rows, cols, packed, scales))
    nweights = sum(r * c for _, r, c, _, _ in mats)

    def step():
        for wb, rows, cols, packed, scales in mats:
            B.moe_int4_quantize(wb, rows, cols, packed, scales)

    K, W = max(1, min(args.steps, 50)), max(1, min(args.warmup, 5))
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    TE = TimingEvents()
    stream = torch.cuda.current_stream().cuda_stream
    ev = [TE.create() for _ in range(3 * K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        TE.record(ev[3 * i], stream)
        B.moe_int4_quantize(*mats[0][:3], mats[0][3], mats[0][4])
        TE.record(ev[3 * i + 1], stream)
        B.moe_int4_quantize(*mats[1][:3], mats[1][3], mats[1][4])
        TE.record(ev[3 * i + 2], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    l0 = np.mean([TE.ms(ev[3 * i], ev[3 * i + 1]) for i in range(K)])
    l1 = np.mean([TE.ms(ev[3 * i + 1], ev[3 * i + 2]) for i in range(K)])
    ms = float(l0 + l1)
    per_s = nweights / (ms * 1e-3)
    n0 = mats[0][1] * mats[0][2]
    achieved = 80 * n0 / (l0 * 1e-3) / 1e12
    result = {
        "metric": "INT4 load-time quantizer: weights quantized per second",
        "value": round(per_s / 1e9, 3), "unit": "Gweights/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, int4 codes + bf16 scales out, fp32 search",
        "data": "synthetic (seeded, device-generated bf16 weights)",
        "config": {"workload": f"quantize64: {E} experts' gate/up [{E * 2 * I}x{H}] and down "
                               f"[{E * H}x{I}] bf16 weights per step, group 128, 20 clip ratios",
                   "weights": nweights},
        "roofline": {"bound": "alu", "kernel": "quantize_int4_kernel (gate/up launch)",
                     "achieved": round(achieved, 3), "peak": VALU_PEAK_TOPS, "unit": "Top/s",
                     "frac": round(achieved / VALU_PEAK_TOPS, 4), "traffic": None,
                     "algorithmic_ops_per_launch": 80 * n0, "launch_us": round(float(l0) * 1e3, 2)},
        "wall_s": round(wall, 4),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = 64
        wh = synth.make_dense_weights(rows, H, 4242)
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle.quantize_int4(wh)
            n += rows * H
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(n / el / 1e9, 6), "unit": "Gweights/s",
                                  "cores": oracle.max_threads(), "kind": "oracle",
                                  "sample": f"{n // (rows * H)} calls on {rows}x{H} weights of the same "
                                            f"distribution (host-generated), {el:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_int8(args):
    """INT8 W8A16 linear layers.  A step is one lm_head projection (lmhead1)
    or one hyper-connection mixer pair, down then up, the down output being
    the up input (hc1, hc512), over T tokens.  Weights are generated on the
    device (uniform random words: uniform codes; bf16 scales |N(0,1)|*0.0004),
    activations bf16 N(0, 1).  Timed region: K steps replayed from a captured
    HIP graph; per-launch times from a second, eager pass with timing-only
    events between the launches.  The roofline is the larger launch's:
    algorithmic bytes (codes + scales + activations in + outputs) against
    HBM, and for many tokens also its flops against the bf16 MFMA peak."""
    import numpy as np
    import torch

    from quantized_moe_router_amd import _binding as B

    cfg = dict(CONFIGS[args.config])
    if args.tokens:
        cfg["tokens"] = args.tokens
    T = cfg["tokens"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev).manual_seed(90001)

    def make(n, k, group):
        w = torch.randint(-2**31, 2**31 - 1, (n, k // 4), dtype=torch.int32, device=dev, generator=gen)
        s = (torch.randn(n, k // group, device=dev, generator=gen).abs() * 4e-4).to(torch.bfloat16)
        return w, s.view(torch.int16)

    if cfg["kind"] == "int8":
        N, Kd, G = cfg["n"], cfg["k"], cfg["group"]
        mats = [make(N, Kd, G) for _ in range(cfg["copies"])]
        launches = [("lm_head", N, Kd, G)]
        x0 = torch.randn(T, Kd, device=dev, generator=gen).to(torch.bfloat16).view(torch.int16)
    else:
        mats = []
        for _ in range(cfg["pairs"]):
            mats.append(make(320, 10240, 64) + make(10240, 320, 64))
        launches = [("down", 320, 10240, 64), ("up", 10240, 320, 64)]
        x0 = torch.randn(T, 10240, device=dev, generator=gen).to(torch.bfloat16).view(torch.int16)
    outs = [torch.empty(T, n, dtype=torch.int16, device=dev) for _, n, _, _ in launches]
    wss = []
    for _, n, kk, g in launches:
        need = B.moe_int8_linear_workspace_bytes(T, n, kk, g)
        wss.append(torch.empty(need, dtype=torch.uint8, device=dev) if need else None)
    nrot = len(mats)
    if args.copy_calibration:
        # a plain copy of known size: each launch reads and writes exactly n bytes
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def launch(i, j):
        m = mats[i % nrot]
        _, n, kk, g = launches[j]
        xin = x0 if j == 0 else outs[0]
        B.moe_int8_linear(xin, m[2 * j], m[2 * j + 1], T, n, kk, g, outs[j], wss[j])

    def step(i):
        for j in range(len(launches)):
            launch(i, j)

    K, W = args.steps, min(args.warmup, 20)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    Gn = min(nrot, K)
    graphs = []
    for start, n in [(W, Gn), (W + (K // Gn) * Gn, K % Gn)]:
        if n == 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(start + i)
        graphs.append((g, n))
    torch.cuda.synchronize()
    plan = [graphs[0]] * (K // Gn) + ([graphs[1]] if K % Gn else [])
    assert sum(n for _, n in plan) == K
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ga.record()
    for g, _ in plan:
        g.replay()
    gb.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ga.elapsed_time(gb)
    ms_per_step = gpu_ms / K

    # per-launch times: eager pass behind a spin kernel, events on the stream
    TE = TimingEvents()
    stream = torch.cuda.current_stream().cuda_stream
    nl = len(launches)
    evs = [[TE.create() for _ in range(nl + 1)] for _ in range(K)]
    sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sa.record(); torch.cuda._sleep(1_000_000); sb.record(); torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(sa.elapsed_time(sb), 1e-3)
    torch.cuda._sleep(int(cycles_per_ms * (K * nl * 0.03 + 5.0)))
    for i in range(K):
        TE.record(evs[i][0], stream)
        for j in range(nl):
            launch(W + i, j)
            TE.record(evs[i][j + 1], stream)
    torch.cuda.synchronize()
    per = np.array([[TE.ms(evs[i][j], evs[i][j + 1]) for j in range(nl)] for i in range(K)]) * 1e3
    launch_us = per.mean(axis=0)

    def alg_bytes(n, kk, g):
        return n * kk + n * (kk // g) * 2 + T * kk * 2 + T * n * 2

    dom = int(np.argmax(launch_us))
    name, n, kk, g = launches[dom]
    kname, uses_mfma = int8_kernel_label(T, n, kk, g)
    byt = alg_bytes(n, kk, g)
    fl = 2.0 * T * n * kk
    hbm = byt / (launch_us[dom] * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": f"{name}: {kname}", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": byt, "launch_us": round(float(launch_us[dom]), 3)}
    if uses_mfma:
        tf = fl / (launch_us[dom] * 1e-6) / 1e12
        roof["mfma_tflops"] = round(tf, 2)
        roof["mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
    trf = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(trf):
        with open(trf) as f:
            t = json.load(f)
        if t.get("source_hash") == kernel_source_hash() and t.get("tokens", T) == T:
            roof["traffic"] = t.get("bytes_per_launch")
    step_bytes = sum(alg_bytes(n_, k_, g_) for _, n_, k_, g_ in launches)
    if cfg["kind"] == "int8":
        metric = "INT8 W8A16 lm_head tokens/s"
        workload = (f"{args.config}: lm_head [{N}x{Kd}] INT8 group {G}, T={T} tokens per step, "
                    f"{nrot} resident copies used alternately")
    else:
        metric = "INT8 W8A16 hyper-connection mixer (down+up) tokens/s"
        workload = (f"{args.config}: hyper-connection down [320x10240] then up [10240x320], INT8 group 64, "
                    f"T={T} tokens per step, rotating over {nrot} resident pairs")
    result = {
        "metric": metric, "value": round(T * K / (gpu_ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8 codes x fp16 activations, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded, device-generated)",
        "config": {"workload": workload, "tokens": T,
                   "launch_us": {nm: round(float(u), 3) for (nm, _, _, _), u in zip(launches, launch_us)},
                   "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof, "wall_s": round(wall, 4), "source_hash": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from quantized_moe_router_amd import synth
        if cfg["kind"] == "int8":
            rows = 2048
            lay = synth.make_int8_linear(T, rows, Kd, G, seed=11)
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.int8_linear(lay["x"], lay["packed"], lay["scales"], G)
                done += rows
                if time.perf_counter() - t0 >= args.cpu_seconds:
                    break
            el = time.perf_counter() - t0
            sample = (f"{done // rows} oracle calls on {rows} of the {N} rows (same shape and "
                      f"distribution, host-generated), {el:.1f} s; scaled by rows")
            tok_s = T * (done / N) / el
        else:
            ntok = min(T, 8)
            dn = synth.make_int8_linear(ntok, 320, 10240, 64, seed=11)
            up = synth.make_int8_linear(ntok, 10240, 320, 64, seed=12)
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.int8_linear(dn["x"], dn["packed"], dn["scales"], 64)
                oracle.int8_linear(up["x"], up["packed"], up["scales"], 64)
                done += ntok
                if time.perf_counter() - t0 >= args.cpu_seconds:
                    break
            el = time.perf_counter() - t0
            sample = f"{done // ntok} oracle down+up pairs on {ntok} tokens, {el:.1f} s"
            tok_s = done / el
        result["cpu_baseline"] = {"value": round(tok_s, 3), "unit": "tokens/s", "cores": oracle.max_threads(),
                                  "kind": "oracle", "sample": sample}
    print(json.dumps(result), flush=True)


def int8_kernel_label(T, N, K, G):
    """(name, uses matrix cores) of what moe_int8_linear runs for a shape: the
    library's plan rules (few tokens: a GEMV, the row-split one on narrow
    matrices; 5-16 tokens on wide matrices: the matrix-core GEMV; otherwise
    the GEMM, loading its whole K range at once up to K = 320, else split
    over K while the output tiles alone would leave the chip idle)."""
    narrow = (N + 3) // 4 < 2048 and K >= 1024
    if 1 <= T <= 4 and narrow:
        return f"int8_gemv_rowsplit_kernel<{T}> (one weight row per workgroup, K split over its waves)", False
    if 1 <= T <= 4 and T * K * 2 + T * (K // 16) * 4 <= 65536:
        return f"int8_gemv_kernel<{T}> (x in LDS, fp16 dot2 on byte-permuted codes)", False
    if 4 < T <= 16 and not narrow and T * (K // 8 + 1) * 16 <= 65536:
        return "int8_gemv_mfma_kernel (matrix-core GEMV, codes as the B operand)", True
    if K <= 320:
        return (f"int8_gemm_short_kernel<{K // 64}, {G // 64}> (fp16 MFMA, exact per-group scaling, "
                "every load of the tile at once)"), True
    tiles = -(-T // 128) * -(-N // 128)
    unit = max(G, 64)
    units = K // unit
    ks = 1
    if tiles < 256:
        ks = min(-(-256 // tiles), units // max(256 // unit, 1), 16)
        ks = max(ks, 1)
    kslice = -(-units // ks) * unit
    split = -(-K // kslice) > 1
    return ("int8_gemm_kernel (fp16 MFMA, exact per-group scaling)" + (" + split-K sum" if split else "")), True


def cpu_baseline(layer, xs, T, k, budget_s, synth):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    first layer's weights with the benchmark's activations, whole tokens."""
    import numpy as np

    import oracle
    w = layer.w
    host = {"router_w": synth.to_host(w["router_w"]), "w13_packed": synth.to_host(w["w13_packed"]),
            "w13_scales": synth.to_host(w["w13_scales"]), "w2_packed": synth.to_host(w["w2_packed"]),
            "w2_scales": synth.to_host(w["w2_scales"]), "top_k": k, "group": layer.group}
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
    # the same calls on one thread, for a quarter of the budget (at least one call)
    n1, t1 = 0, time.perf_counter()
    while True:
        n = min(T, 8)
        host["x"] = synth.to_host(xs[i % len(xs)][:n])
        oracle.forward(host, nthreads=1)
        n1 += n
        i += 1
        if time.perf_counter() - t1 >= budget_s / 4:
            break
    el1 = time.perf_counter() - t1
    return {"value": round(n_tok / el, 3), "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{n_tok} whole tokens (the first min(T, 8) of each of the benchmark's T={T} "
                      f"activation sets; routing, experts, combine), layer 0 weights, {el:.1f} s",
            "one_thread": {"value": round(n1 / el1, 3), "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} whole tokens the same way, {el1:.1f} s"}}


if __name__ == "__main__":
    main()
