"""Convenience wrapper: a resident MoE INT4 layer on the GPU.

Allocates outputs and a zero-filled workspace with torch and calls the C ABI;
no arithmetic of the layer happens here.
"""
from __future__ import annotations

import torch

from . import _binding as B


class MoeInt4Layer:
    """Holds device tensors of one layer (keys as produced by synth.to_device /
    synth.device_weights) and runs the library's entry points on them."""

    def __init__(self, weights: dict, top_k: int, group: int = 128, shared: dict | None = None):
        self.w = weights
        self.top_k = int(top_k)
        self.group = int(group)
        E, H = weights["router_w"].shape
        self.E, self.H = int(E), int(H)
        self.I = int(weights["w2_packed"].shape[2] * 8)
        self.shared = shared
        self._shared_c = B.make_shared(shared)
        self._ws = {}

    def shape(self, tokens: int) -> B.MoeShape:
        return B.make_shape(tokens, self.H, self.E, self.I, self.top_k, self.group)

    def workspace(self, tokens: int, device=None) -> torch.Tensor:
        key = (tokens, device)
        if key not in self._ws:
            self._ws[key] = B.new_workspace(self.shape(tokens), self._shared_c,
                                            device=device or self.w["router_w"].device)
        return self._ws[key]

    def workspaces(self) -> list:
        return list(self._ws.values())

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=torch.int16, device=x.device)
        w = self.w
        B.moe_int4_forward(x, w["router_w"], w["w13_packed"], w["w13_scales"], w["w2_packed"],
                           w["w2_scales"], self.top_k, out, self.shape(T), self._shared_c,
                           self.workspace(T), stream)
        return out

    def route(self, x: torch.Tensor, stream=None) -> dict:
        T, dev = x.shape[0], x.device
        r = {
            "ids": torch.empty(T, self.top_k, dtype=torch.int32, device=dev),
            "weights": torch.empty(T, self.top_k, dtype=torch.float32, device=dev),
            "counts": torch.empty(self.E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(self.E + 1, dtype=torch.int32, device=dev),
            "sorted_slots": torch.empty(max(T * self.top_k, 1), dtype=torch.int32, device=dev),
        }
        B.moe_int4_route(x, self.w["router_w"], self.shape(T), r["ids"], r["weights"], r["counts"],
                         r["offsets"], r["sorted_slots"], self.workspace(T), stream)
        return r

    def experts(self, x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=torch.int16, device=x.device)
        w = self.w
        B.moe_int4_experts(x, ids, weights, w["w13_packed"], w["w13_scales"], w["w2_packed"],
                           w["w2_scales"], self.shape(T), self._shared_c, out, self.workspace(T), stream)
        return out
