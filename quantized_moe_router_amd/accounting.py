"""Algorithmic bytes and flops of the INT4 routed-expert MoE layer.

These are the roofline numerators: what the method must move or compute,
independent of how a kernel does it.  The per-expert byte count reproduces the
totals printed on the pages (model card "What is quantized": 58.0 GiB of INT4
gs128 experts over 48 layers of 512; "vLLM Edition" section 2: 120.8B routed
parameters; "vLLM Optimization Edition" section 3.3 "MoE block (decode-05)":
about 25 MB of expert weights per token per layer).
"""
from __future__ import annotations


def expert_params(hidden: int = 2560, inter: int = 640) -> int:
    """Weights of one SwiGLU expert: fused gate/up [2I, H] plus down [H, I]."""
    return 2 * inter * hidden + hidden * inter


def expert_bytes(hidden: int = 2560, inter: int = 640, group: int = 128, bits: int = 4) -> int:
    """Packed codes plus bf16 scales of one expert."""
    packed = expert_params(hidden, inter) * bits // 8
    scales = (2 * inter * (hidden // group) + hidden * (inter // group)) * 2
    return packed + scales


def router_bytes(hidden: int = 2560, experts: int = 512) -> int:
    return experts * hidden * 2


def layer_bytes(tokens: int, distinct_experts: int, hidden: int = 2560, experts: int = 512,
                inter: int = 640, group: int = 128, shared_bytes: int = 0) -> int:
    """Bytes one layer call must move: router weights, each touched expert once,
    activations in (bf16) and the output (bf16)."""
    return (router_bytes(hidden, experts) + distinct_experts * expert_bytes(hidden, inter, group)
            + shared_bytes + 2 * tokens * hidden * 2)


def shared_int6_bytes(hidden: int = 2560, inter: int = 640, group: int = 64) -> int:
    """INT6 shared expert plus its bf16 gate row."""
    return expert_bytes(hidden, inter, group, bits=6) + hidden * 2


def layer_flops(tokens: int, top_k: int = 10, hidden: int = 2560, experts: int = 512,
                inter: int = 640, shared_inter: int = 0) -> int:
    """Multiply-adds x 2 of router, routed experts and (optional) shared expert."""
    router = 2 * tokens * experts * hidden
    routed = 2 * tokens * top_k * expert_params(hidden, inter)
    shared = 2 * tokens * expert_params(hidden, shared_inter) + 2 * tokens * hidden if shared_inter else 0
    return router + routed + shared
