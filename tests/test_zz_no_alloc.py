"""moe_int4_forward_noalloc (static per-device scratch, no allocation) against
moe_int4_forward (caller workspace) through the C ABI: the same kernels, so
the outputs must be bit-identical, on consecutive calls whose second input is
smaller than the first (the scratch keeps the previous call's contents)."""
import sys

import numpy as np
import pytest
import torch

from quantized_moe_router_amd import _binding as B
from quantized_moe_router_amd import synth
from quantized_moe_router_amd.layer import MoeInt4Layer

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(L, x, status):
    w = L.w
    T = x.shape[0]
    out = torch.empty(T, L.H, dtype=torch.int16, device=x.device)
    B.moe_int4_forward_noalloc(x, w["router_w"], w["w13_packed"], w["w13_scales"], w["w2_packed"],
                               w["w2_scales"], L.top_k, out, L.shape(T), L._shared_c, status)
    return out


@pytest.mark.parametrize("shared,token_seq", [
    (False, (64, 7)),      # many-token (matrix-core) path, then the few-token path
    (False, (16, 5)),      # few-token path twice
    (True, (40, 3)),       # with the INT6 shared expert
])
def test_noalloc_matches_forward(shared, token_seq):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    shape0 = synth.LayerShape(tokens=max(token_seq), hidden=512, experts=32, top_k=4, inter=256)
    host = synth.make_layer(shape0, seed=11, shared=shared)
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, shape0.top_k, group=shape0.group, shared=dev.get("shared"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, T in enumerate(token_seq):
        say(f"noalloc call {i}: T={T} shared={shared}")
        x = dev["x"][:T].contiguous()
        ref = L.forward(x)
        got = _noalloc(L, x, status)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), f"call {i} (T={T}): noalloc output differs from forward"
        assert int(status.item()) == 0
        assert B.workspace_status(L.workspace(T)) == 0


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    s = B.make_shape(8192, 2560, 512, 640, 10, 128)
    assert B.workspace_bytes(s) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_int4_forward_noalloc(x, x, x, x, x, x, 10, x[8:], s, None)
    assert e.value.code == B.EWORKSPACE and "static scratch" in str(e.value)
