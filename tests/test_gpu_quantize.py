"""GPU parity of the load-time INT4 quantizer ("Running 125B MoE on Three
3090s - vLLM Optimization Edition", section 7: round to nearest, group 128,
symmetric, per-group clip search for the smallest squared error): the HIP
kernel, through the C ABI, against the CPU oracle on the same bf16 inputs.

The codes and the scale of a group are integers decided by floating point;
both sides take the decision in fp32 with the same operations in the same
order, so packed words and scales must match bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_router_amd import _binding as B
from quantized_moe_router_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


def gpu_quantize(w: np.ndarray, group: int = 128):
    rows, cols = w.shape
    wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).cuda()
    packed = torch.empty((rows, cols // 8), dtype=torch.int32, device="cuda")
    scales = torch.empty((rows, cols // group), dtype=torch.int16, device="cuda")
    B.moe_int4_quantize(wd, rows, cols, packed, scales, group=group)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


def check(w: np.ndarray, label: str, group: int = 128):
    say(f"quantize case {label}: {w.shape} group {group}")
    gp, gs = gpu_quantize(w, group)
    op, os_, _, _ = oracle.quantize_int4(w, group)
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"{label}: {len(bad_s)} scales differ, first {bad_s[:3].tolist()}"
    bad_w = np.argwhere(gp != op)
    assert bad_w.size == 0, f"{label}: {len(bad_w)} packed words differ, first {bad_w[:3].tolist()}"


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("rows,cols,seed", [(7, 128, 1), (300, 2560, 2), (64, 640, 3), (1, 4096, 4)])
def test_quantize_random(rows, cols, seed, group):
    check(synth.make_dense_weights(rows, cols, seed), f"random {rows}x{cols}", group)


@pytest.mark.parametrize("group", [128, 64])
def test_quantize_special_groups(group):
    f = (np.random.default_rng(9).standard_normal((12, 256)) * 0.02).astype(np.float32)
    f[0] = 0.0                                                  # zero groups
    f[1, :128] = 0.25                                           # constant group
    f[1, 128:] = -0.125
    n = np.random.default_rng(10).integers(-7, 8, 256)
    n[0] = 7
    n[128] = -7
    f[2] = n * 2.0 ** -6                                        # exactly representable
    f[3, :8] = np.array([7, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]) * 2.0 ** -6   # exact ties
    f[4, 40] = 0.4                                              # one outlier
    f[5] *= np.float32(1e-30)                                   # tiny magnitudes
    f[6] *= np.float32(1e30)                                    # huge magnitudes
    f[7, :128] = 0.0
    f[7, 5] = 1e-39                                             # a lone subnormal
    f[8, ::2] = 0.0                                             # half zeros
    f[9] = -np.abs(f[9])                                        # one-signed
    f[10, :128] = -8 * 2.0 ** -4                                # the code -8 level
    f[10, 1] = 7 * 2.0 ** -4
    check(synth.bf16_bits(f), "special groups", group)


def test_quantize_real_expert_shapes():
    # one expert's fused gate/up [2I, H] and down [H, I] at the real shape
    check(synth.make_dense_weights(1280, 2560, 21), "gate/up 1280x2560")
    check(synth.make_dense_weights(2560, 640, 22), "down 2560x640")


def test_quantized_weights_drive_the_layer():
    # the quantizer's output is a valid weight set for the layer: dequantized
    # by the oracle it reproduces the input within the quantization error
    w = synth.make_dense_weights(256, 256, 30)
    gp, gs = gpu_quantize(w)
    deq = oracle.dequant_int4(gp, gs)
    x = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = (gs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(deq - x).reshape(256, 2, 128)
    clip = np.abs(x).reshape(256, 2, 128) > 7.5 * s[:, :, None]
    # unclipped inputs are within half a level of their code
    assert np.all(err[~clip] <= 0.5 * np.broadcast_to(s[:, :, None], err.shape)[~clip] * (1 + 1e-12))


def _sweep_weights(rows, cols, kind, seed):
    """Seeded bf16 weights of one distribution: normal, heavy-tailed
    (Student t, 2 degrees of freedom), sparse (90 % exact zeros), row scales
    spread over 10^-15 .. 10^15, or near-constant groups."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        w = rng.standard_normal((rows, cols)) * 0.02
    elif kind == "heavy":
        w = rng.standard_t(2.0, (rows, cols)) * 0.01
    elif kind == "sparse":
        w = rng.standard_normal((rows, cols)) * (rng.random((rows, cols)) < 0.1)
    elif kind == "scaled":
        w = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-15.0, 15.0, (rows, 1))
    else:
        w = 0.5 + 1e-3 * rng.standard_normal((rows, cols))
    return synth.bf16_bits(w.astype(np.float32))


def _sweep_cases(n=20, seed=99):
    rng = np.random.default_rng(seed)
    kinds = ["normal", "heavy", "sparse", "scaled", "near-constant"]
    out = []
    for i in range(n):
        group = int(rng.choice([64, 128]))
        out.append((int(rng.integers(1, 200)), group * int(rng.integers(1, 4096 // group + 1)), group,
                    kinds[i % len(kinds)], 1000 + i))
    return out


@pytest.mark.parametrize("rows,cols,group,kind,seed", _sweep_cases())
def test_quantize_random_sweep(rows, cols, group, kind, seed):
    # the GPU quantizer bit-exact against the oracle on random shapes and
    # value distributions
    check(_sweep_weights(rows, cols, kind, seed), f"sweep {kind} {rows}x{cols}", group)
