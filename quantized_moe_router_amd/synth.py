"""Seeded synthetic inputs for the INT4 routed-expert MoE layer.

This module only draws random numbers and lays them out in the documented byte
format; it holds none of the layer's arithmetic.  Both the CPU oracle (in the
tests) and the HIP path consume the very same bytes it returns.

Byte format (the library's input contract):
  * x          bf16 bits, uint16 [T, H], row-major.
  * router_w   bf16 bits, uint16 [E, H].
  * w13_packed int32 [E, 2I, H/8]: fused gate (rows 0..I-1) and up (rows I..2I-1)
               projections, 8 INT4 codes per word along the input dimension,
               least significant nibble first, each stored as code + 8.
  * w13_scales bf16 bits [E, 2I, H/128]: one per (row, 128 inputs).
  * w2_packed  int32 [E, H, I/8]; w2_scales bf16 bits [E, H, I/128].
  * shared expert (optional): INT6 codes, 32 per six int32 words, stored
    code + 32, group 64, with a bf16 gate row [H].

Because every nibble of a uniformly random 32-bit word is uniform on 0..15,
uniformly random words *are* uniformly random INT4 codes in [-8, 7] stored
with the +8 bias; likewise six random words are 32 uniform INT6 codes in
[-32, 31] stored +32.  So the generator never packs anything itself.

Distributions (per layer): router N(0, 0.02), activations N(0, 1), INT4
scales |N(0,1)| * 0.02, INT6 scales |N(0,1)| * 0.005, all rounded to bf16
(round to nearest even).  A Zipf(s) routing skew is planted through a bias
feature: x[:, H-1] = 1 and router_w[e, H-1] = bf16(-s * ln(rank_e)) for a seeded
permutation rank of 1..E, which adds s * ln(1/rank) to expert e's logit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class LayerShape:
    tokens: int
    hidden: int = 2560
    experts: int = 512
    top_k: int = 10
    inter: int = 640
    group: int = 128


TINY = LayerShape(tokens=8, hidden=256, experts=16, top_k=2, inter=128)
DECODE = LayerShape(tokens=1)
DECODE4 = LayerShape(tokens=4)
PREFILL512 = LayerShape(tokens=512)
PREFILL8192 = LayerShape(tokens=8192)

SHARED_INTER = 640
SHARED_GROUP = 64


def bf16_bits(a) -> np.ndarray:
    """float array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _words(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 2**32, size=shape, dtype=np.uint32).view(np.int32)


def make_dense_weights(rows: int, cols: int, seed: int, std: float = 0.02,
                       outlier_frac: float = 1e-3, outlier_scale: float = 15.0) -> np.ndarray:
    """Dense bf16 weights before quantization, uint16 bits [rows, cols]:
    N(0, std), with a seeded fraction of entries multiplied by outlier_scale
    (the heavy tail a clip search exists for)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(std)
    mask = rng.random((rows, cols)) < outlier_frac
    w[mask] *= np.float32(outlier_scale)
    return bf16_bits(w)


# INT8 W8A16 linear layers: the hyper-connection low-rank mixers (down
# [320, 10240] and up [10240, 320], group 64) and lm_head ([248320, 2560],
# group 128).  Packed int32 [N, K/4], four codes per word, least significant
# byte first, each stored as code + 128: random words are uniform codes in
# [-128, 127].  Scales bf16(|N(0,1)| * 0.0004), about amax / 127 of an
# N(0, 0.02) weight group; activations bf16(N(0, 1)).
INT8_SCALE_STD = 0.0004


def make_int8_linear(tokens: int, n: int, k: int, group: int, seed: int = 0,
                     x_seed: int | None = None) -> dict:
    """Host INT8 linear layer {x, packed, scales, group}; the weights come from
    `seed`, the activations from `x_seed` (default seed + 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    packed = _words(rng, (n, k // 4))
    scales = bf16_bits(np.abs(rng.standard_normal((n, k // group), dtype=np.float32))
                       * np.float32(INT8_SCALE_STD))
    xrng = np.random.Generator(np.random.PCG64(seed + 1 if x_seed is None else x_seed))
    x = bf16_bits(xrng.standard_normal((tokens, k), dtype=np.float32))
    return {"x": x, "packed": packed, "scales": scales, "group": group}


def make_weights(shape: LayerShape, seed: int = 0) -> dict:
    """Router and expert weights of one layer (independent of the token count)."""
    H, E, I, G = shape.hidden, shape.experts, shape.inter, shape.group
    rng = np.random.Generator(np.random.PCG64(seed))
    router = rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02)
    return {
        "router_f32": router,
        "w13_packed": _words(rng, (E, 2 * I, H // 8)),
        "w13_scales": bf16_bits(np.abs(rng.standard_normal((E, 2 * I, H // G), dtype=np.float32)) * np.float32(0.02)),
        "w2_packed": _words(rng, (E, H, I // 8)),
        "w2_scales": bf16_bits(np.abs(rng.standard_normal((E, H, I // G), dtype=np.float32)) * np.float32(0.02)),
    }


def make_shared(hidden: int, seed: int) -> dict:
    """INT6 group-64 shared expert (intermediate 640) and its gate row."""
    srng = np.random.Generator(np.random.PCG64(seed))
    SI, SG = SHARED_INTER, SHARED_GROUP
    H = hidden
    return {
        "gate_w": bf16_bits(srng.standard_normal(H, dtype=np.float32) * np.float32(0.02)),
        "w13_packed": _words(srng, (2 * SI, H // 32 * 6)),
        "w13_scales": bf16_bits(np.abs(srng.standard_normal((2 * SI, H // SG), dtype=np.float32)) * np.float32(0.005)),
        "w2_packed": _words(srng, (H, SI // 32 * 6)),
        "w2_scales": bf16_bits(np.abs(srng.standard_normal((H, SI // SG), dtype=np.float32)) * np.float32(0.005)),
        "group": SG,
    }


def make_layer(shape: LayerShape, seed: int = 0, x_seed: int | None = None,
               zipf_s: float | None = None, shared: bool = False, weights: dict | None = None) -> dict:
    """Host (numpy) layer.  Weights come from `seed` (or are passed in, as made
    by make_weights); activations from `x_seed` (default seed + 1)."""
    T, H, E = shape.tokens, shape.hidden, shape.experts
    w = make_weights(shape, seed) if weights is None else weights
    xrng = np.random.Generator(np.random.PCG64(seed + 1 if x_seed is None else x_seed))
    x = xrng.standard_normal((T, H), dtype=np.float32)
    router = w["router_f32"]
    if zipf_s is not None:
        router = router.copy()
        prng = np.random.Generator(np.random.PCG64(seed + 7919))
        rank = prng.permutation(E).astype(np.float64) + 1.0
        router[:, H - 1] = (-zipf_s * np.log(rank)).astype(np.float32)
        x[:, H - 1] = 1.0
    layer = {
        "shape": shape,
        "top_k": shape.top_k,
        "group": shape.group,
        "router_w": bf16_bits(router),
        "x": bf16_bits(x),
        "w13_packed": w["w13_packed"],
        "w13_scales": w["w13_scales"],
        "w2_packed": w["w2_packed"],
        "w2_scales": w["w2_scales"],
    }
    if shared:
        layer["shared"] = make_shared(H, seed + 104729)
    return layer


def to_device(layer: dict, device="cuda") -> dict:
    """Copy a host layer's arrays to torch tensors on `device` (bit-identical)."""
    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = {}
    for key, v in layer.items():
        if isinstance(v, np.ndarray):
            out[key] = dev(v)
        elif isinstance(v, dict):
            out[key] = {kk: (dev(vv) if isinstance(vv, np.ndarray) else vv) for kk, vv in v.items()}
        else:
            out[key] = v
    return out


def device_weights(shape: LayerShape, seed: int, device="cuda") -> dict:
    """Expert and router weights drawn directly on the GPU with torch's seeded
    device generator (used for the many-layer resident sets, where host
    generation would take minutes).  Same formats and distributions as
    make_layer; int16 tensors hold bf16 bits."""
    H, E, I, G = shape.hidden, shape.experts, shape.inter, shape.group
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def words(*s):
        n = math.prod(s)
        return torch.randint(0, 256, (n * 4,), dtype=torch.uint8, device=device, generator=g).view(torch.int32).view(*s)

    def scales(*s):
        return (torch.randn(*s, device=device, generator=g).abs() * 0.02).to(torch.bfloat16).view(torch.int16)

    return {
        "router_w": (torch.randn(E, H, device=device, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16),
        "w13_packed": words(E, 2 * I, H // 8),
        "w13_scales": scales(E, 2 * I, H // G),
        "w2_packed": words(E, H, I // 8),
        "w2_scales": scales(E, H, I // G),
    }


def device_activations(shape: LayerShape, seed: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape.tokens, shape.hidden, device=device, generator=g).to(torch.bfloat16).view(torch.int16)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy with the library's dtypes (int16 -> uint16 bits)."""
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a
