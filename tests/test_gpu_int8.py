"""GPU parity of the INT8 W8A16 linear layer ("Running 125B MoE on Three
3090s - vLLM Optimization Edition", section 3.3, "Hyper-connection
(decode-04)": four codes per int32 word, least significant byte first, each
stored as code + 128; model card "What is quantized", groups C and D:
symmetric groups of 64 and 128): the HIP path, through the C ABI, against
the CPU oracle on the same bytes.

Tolerance, from the arithmetic: the output is one bf16 rounding (relative
error <= 2^-9) of an fp32 sum of exact code * x products (fp16 activations
are exact for the N(0, 1) inputs used here, apart from magnitudes below 2^-14
whose contribution is below 2^-25 each); the fp32 sum order differs from the
oracle's, an error far below 1e-3 of the output's rms for K <= 65536.  So
every element must satisfy |gpu - o| <= 2^-8 |o| + 1e-3 rms(o), and the
aggregate bar of the MoE layer (max error <= 2e-2 rms, sum |err| / sum |o|
<= 5e-3) holds with room to spare."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_half_ulp
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


def to_dev(layer):
    x = torch.from_numpy(layer["x"].view(np.int16)).cuda()
    p = torch.from_numpy(layer["packed"]).cuda()
    s = torch.from_numpy(layer["scales"].view(np.int16)).cuda()
    return x, p, s


def run(x, p, s, T, N, K, G, out=None):
    need = B.moe_int8_linear_workspace_bytes(T, N, K, G)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    if out is None:
        out = torch.empty((T, N), dtype=torch.int16, device="cuda")
    B.moe_int8_linear(x, p, s, T, N, K, G, out, ws)
    torch.cuda.synchronize()
    return out


def as_f64(bits: torch.Tensor) -> np.ndarray:
    return bits.cpu().view(torch.bfloat16).double().numpy()


def compare(g: np.ndarray, o: np.ndarray, label: str):
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    bound = 2.0 ** -8 * np.abs(o) + 1e-3 * rms
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{label}: {len(bad)} outputs off, first {bad[:3].tolist()} "
                           f"gpu {g[tuple(bad[0])]} oracle {o[tuple(bad[0])]}")
    # the output is bf16: its own rounding of the exact value (half an ulp at
    # the oracle's value) is not counted against the fp32 accumulation
    beyond = np.maximum(err - bf16_half_ulp(o), 0.0)
    assert beyond.max() <= 2e-2 * rms, (label, float(beyond.max()), rms)
    assert err.sum() <= 5e-3 * np.abs(o).sum(), label


SMALL = [
    # (T, N, K, G).  Plan: narrow matrices (N < 8189 and K >= 1024) with at
    # most 4 tokens take one row per workgroup; other matrices with at most 4
    # tokens the dot-product GEMV; 5..16 tokens on wide matrices the
    # matrix-core GEMV (while T * (K + 8) fp16 fit 64 KB of LDS); everything
    # else the GEMM.
    (1, 37, 128, 64),      # dot GEMV: ragged row block, one partial column pass
    (1, 9, 64, 64),        # dot GEMV: single group
    (2, 130, 320, 64),     # dot GEMV: hyper-connection up row length
    (2, 9000, 1152, 128),  # dot GEMV: several row blocks per wave, two passes
    (3, 8193, 2048, 64),   # dot GEMV: ragged last row block
    (1, 300, 2560, 128),   # row split: lm_head row length
    (3, 77, 1152, 128),    # row split: ragged wave slices
    (4, 320, 4096, 64),    # row split
    (4, 64, 8192, 128),    # row split at the LDS limit
    (5, 777, 448, 64),     # matrix-core GEMV: odd step count, ragged rows
    (7, 9001, 1152, 128),  # matrix-core GEMV: several row blocks per wave
    (8, 3000, 640, 64),
    (12, 8200, 2560, 128), # matrix-core GEMV at the LDS limit for K = 2560
    (16, 2001, 320, 64),   # matrix-core GEMV: all 16 token rows
    (5, 200, 640, 64),     # matrix-core GEMV
    (6, 320, 2048, 64),    # GEMM: narrow matrix, split K, one row tile
    (1, 5, 65536, 64),     # GEMM: one token past every GEMV's LDS limit
    (33, 129, 1024, 128),  # GEMM: ragged row and weight-row tiles
    (130, 333, 1024, 64),
    (300, 256, 256, 128),  # short-K GEMM (K <= 320 loaded at once): 4 stages, group 128
    (64, 1000, 2560, 128),
    (200, 96, 4096, 64),   # GEMM: narrow, split K
    (17, 9, 64, 64),       # short-K GEMM: one stage, one ragged token tile, 9 rows
    (129, 130, 128, 128),  # short-K GEMM: one group of 128, ragged tokens, N not a multiple of 4
    (200, 333, 192, 64),   # short-K GEMM: three stages, ragged row tile
    (77, 1000, 320, 64),   # short-K GEMM: the hyper-connection up row length
    (260, 513, 256, 64),   # short-K GEMM: three token tiles, N = 2 x 256 + 1
    (96, 300, 320, 64),    # short-K GEMM: 96 tokens, three 32-row MFMA tiles
    (512, 10240, 320, 64), # short-K GEMM: the hyper-connection up projection at 512 tokens
    (2100, 8192, 320, 64), # short-K GEMM: 17 x 32 tiles, 52-token tail
    (1000, 16384, 256, 128),  # short-K GEMM, group 128: 8 x 64 tiles, 104-token tail
]


@pytest.mark.parametrize("T,N,K,G", SMALL)
def test_int8_linear_small(T, N, K, G):
    label = f"int8 T={T} N={N} K={K} G={G}"
    say(label)
    layer = synth.make_int8_linear(T, N, K, G, seed=T * 1000 + N)
    g = as_f64(run(*to_dev(layer), T, N, K, G))
    o = oracle.int8_linear(layer["x"], layer["packed"], layer["scales"], G)
    compare(g, o, label)


@pytest.mark.parametrize("T", [1, 4, 512])
@pytest.mark.parametrize("which", ["down", "up"])
def test_int8_hyper_connection_shapes(which, T):
    # the hyper-connection low-rank mixers: down [320, 10240], up [10240, 320]
    N, K = (320, 10240) if which == "down" else (10240, 320)
    label = f"hc {which} T={T}"
    say(label)
    layer = synth.make_int8_linear(T, N, K, 64, seed=17 + T)
    g = as_f64(run(*to_dev(layer), T, N, K, 64))
    # the oracle on a seeded sample of tokens (all of them below 64)
    rng = np.random.default_rng(T)
    toks = np.arange(T) if T <= 64 else np.unique(np.concatenate([[0, T - 1], rng.choice(T, 48, replace=False)]))
    o = oracle.int8_linear(layer["x"][toks], layer["packed"], layer["scales"], 64)
    compare(g[toks], o, label)


@pytest.mark.parametrize("T", [1, 2, 4, 12, 16])
def test_int8_lm_head_full_size(T):
    # lm_head [248320, 2560], group 128: every output against the oracle on
    # a seeded sample of rows (plus the first and last)
    N, K, G = 248320, 2560, 128
    label = f"lm_head T={T}"
    say(label)
    layer = synth.make_int8_linear(T, N, K, G, seed=5)
    g = as_f64(run(*to_dev(layer), T, N, K, G))
    rng = np.random.default_rng(T)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 4096, replace=False)]))
    o = oracle.int8_linear(layer["x"], layer["packed"][rows], layer["scales"][rows], G)
    compare(g[:, rows], o, label)
    assert np.isfinite(g).all()


@pytest.mark.parametrize("T,K", [(1, 256), (3, 256), (2, 1024), (6, 256), (40, 256)])
def test_int8_edge_codes_and_scales(T, K):
    # all-(-128) and all-127 rows, zero scales, a zero token, powers of two,
    # through the dot GEMV (1 and 3 tokens), the one-row-per-workgroup GEMV
    # (K = 1024), the matrix-core GEMV (6 tokens) and the GEMM (40 tokens)
    N, G = 8, 64
    x = np.zeros((T, K), np.float32)
    x[0::3] = 1.0
    x[1::3] = np.tile([1.0, -2.0, 0.5, 4.0], K // 4)
    layer = {"x": synth.bf16_bits(x)}
    packed = np.zeros((N, K // 4), np.uint32)
    packed[1] = 0xFFFFFFFF
    packed[2] = 0x80808080
    packed[3] = 0x00FF7F80
    packed[4:] = np.random.default_rng(1).integers(0, 2**32, size=(N - 4, K // 4), dtype=np.uint32)
    layer["packed"] = packed.view(np.int32)
    sc = np.full((N, K // G), 2.0 ** -7, np.float32)
    sc[5] = 0.0
    sc[6, 1] = 0.0
    layer["scales"] = synth.bf16_bits(sc)
    g = as_f64(run(*to_dev(layer), T, N, K, G))
    o = oracle.int8_linear(layer["x"], layer["packed"], layer["scales"], G)
    # every product is a multiple of 2^-8 and every partial sum stays far
    # below 2^24 of those, so the fp32 sum is exact in any order: the GPU
    # output must be the oracle value rounded once to bf16
    assert np.all(np.abs(o) * 2.0 ** 8 < 2.0 ** 24)
    expect = torch.from_numpy(o).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(g, expect), np.argwhere(g != expect)[:5]
    assert g[0, 1] == 127 * K * 2.0 ** -7 and g[0, 2] == 0.0 and g[0, 5] == 0.0


def test_int8_zero_tokens_leaves_output_and_repeat_is_deterministic():
    T, N, K, G = 512, 320, 10240, 64
    layer = synth.make_int8_linear(T, N, K, G, seed=3)
    x, p, s = to_dev(layer)
    out = torch.full((T, N), 0x1234, dtype=torch.int16, device="cuda")
    B.moe_int8_linear(x, p, s, 0, N, K, G, out, None)
    torch.cuda.synchronize()
    assert bool((out == 0x1234).all())
    a = run(x, p, s, T, N, K, G)
    b = run(x, p, s, T, N, K, G)
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,N,K,G", [(1, 4100, 2560, 128), (3, 320, 10240, 64), (8, 9001, 1152, 128),
                                     (512, 320, 10240, 64)])
def test_int8_graph_replay_matches_eager(T, N, K, G):
    # every kernel of the chosen plan captured in a HIP graph: replays, with
    # eager work and synchronisation between them, equal the eager result
    # (the split-K partials are fully rewritten by every call: no clearing)
    layer = synth.make_int8_linear(T, N, K, G, seed=77)
    x, p, s = to_dev(layer)
    need = B.moe_int8_linear_workspace_bytes(T, N, K, G)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    eager = torch.empty((T, N), dtype=torch.int16, device="cuda")
    B.moe_int8_linear(x, p, s, T, N, K, G, eager, ws)
    torch.cuda.synchronize()
    out = torch.zeros((T, N), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_int8_linear(x, p, s, T, N, K, G, out, ws)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        junk = torch.randn(1024, device="cuda") * (i + 1)   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs"
        del junk


@pytest.mark.parametrize("T,N,K,G", [(1, 1 << 24, 64, 64), (1 << 20, 64, 64, 64), (2, 3, 65536, 128)])
def test_int8_maximum_sizes(T, N, K, G):
    # the largest row count (2^24 rows: the dot GEMV's persistent grid loops
    # over 4M row blocks), the largest token count (2^20: a GEMM with 8192
    # token tiles) and the longest rows (K = 65536); the oracle on a seeded
    # sample of outputs
    label = f"int8 max T={T} N={N} K={K}"
    say(label)
    rng = np.random.default_rng(T + N)
    gen = torch.Generator(device="cuda").manual_seed(T + N + K)
    p = torch.randint(-2**31, 2**31 - 1, (N, K // 4), dtype=torch.int32, device="cuda", generator=gen)
    s = (torch.randn(N, K // G, device="cuda", generator=gen).abs() * 4e-4).to(torch.bfloat16).view(torch.int16)
    x = torch.randn(T, K, device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
    out = run(x, p, s, T, N, K, G)
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 24)]))
    rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 512)]))
    xs = x[torch.from_numpy(toks).cuda()].cpu().numpy().view(np.uint16)
    ps = p[torch.from_numpy(rows).cuda()].cpu().numpy()
    ss = s[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
    o = oracle.int8_linear(xs, ps, ss, G)
    g = as_f64(out[torch.from_numpy(toks).cuda()][:, torch.from_numpy(rows).cuda()])
    compare(g, o, label)
    del p, s, x, out
    torch.cuda.empty_cache()


def _sweep_cases(n=24, seed=77):
    """Random legal shapes over every plan: tokens log-uniform in [1, 600],
    rows log-uniform in [1, 20000], group 64 or 128, K a multiple of the
    group up to 4096 (a third of the draws at most 320, the load-at-once
    GEMM); draws whose oracle work would be large are skipped."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(np.exp(rng.uniform(0.0, np.log(600.0))))
        N = int(np.exp(rng.uniform(0.0, np.log(20000.0))))
        G = int(rng.choice([64, 128]))
        kmax = 320 if rng.uniform() < 1 / 3 else 4096
        K = G * int(rng.integers(1, kmax // G + 1))
        if T * N * K > 3e9:
            continue
        out.append((T, N, K, G))
    return out


@pytest.mark.parametrize("T,N,K,G", _sweep_cases())
def test_int8_random_shape_sweep(T, N, K, G):
    label = f"int8 sweep T={T} N={N} K={K} G={G}"
    say(label)
    layer = synth.make_int8_linear(T, N, K, G, seed=T * 7919 + N * 31 + K)
    g = as_f64(run(*to_dev(layer), T, N, K, G))
    o = oracle.int8_linear(layer["x"], layer["packed"], layer["scales"], G)
    compare(g, o, label)


@pytest.mark.parametrize("T,N,K,G", [(512, 8192, 8192, 64), (512, 8192, 16384, 128)])
def test_int8_gemm_scale_chunks(T, N, K, G):
    # 256 output tiles, so K is not split: one workgroup's K range holds 128
    # scale groups, and the GEMM restages its rows' scales in LDS after the
    # first 64; the oracle on a seeded sample of outputs
    label = f"int8 scale chunks T={T} N={N} K={K} G={G}"
    say(label)
    rng = np.random.default_rng(K + G)
    gen = torch.Generator(device="cuda").manual_seed(K + G)
    p = torch.randint(-2**31, 2**31 - 1, (N, K // 4), dtype=torch.int32, device="cuda", generator=gen)
    s = (torch.randn(N, K // G, device="cuda", generator=gen).abs() * 4e-4).to(torch.bfloat16).view(torch.int16)
    x = torch.randn(T, K, device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
    out = run(x, p, s, T, N, K, G)
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 16)]))
    rows = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.integers(0, N, 384)]))
    xs = x[torch.from_numpy(toks).cuda()].cpu().numpy().view(np.uint16)
    ps = p[torch.from_numpy(rows).cuda()].cpu().numpy()
    ss = s[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
    o = oracle.int8_linear(xs, ps, ss, G)
    g = as_f64(out[torch.from_numpy(toks).cuda()][:, torch.from_numpy(rows).cuda()])
    compare(g, o, label)
    del p, s, x, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,N,K,G", [
    (1, 2000, 128, 64),     # dot-product GEMV
    (4, 2000, 1152, 128),   # row-split GEMV
    (8, 777, 256, 64),      # matrix-core GEMV
    (40, 300, 320, 64),     # short-K GEMM
    (200, 96, 4096, 64),    # GEMM with its K split and the partial sum
])
def test_int8_bf16_rounding_ties_exact(T, N, K, G):
    # One-hot activations (x[t, c_t] = 1): every output is code * scale,
    # exact in fp32 whatever the summation order (at most 16 significant
    # bits), so the one bf16 rounding of the output must be round to nearest
    # even of the oracle's exact value, bit for bit.  Scales (1 + m/128) 2^e
    # make many of those values fall exactly halfway between two bf16 values.
    label = f"int8 ties T={T} N={N} K={K} G={G}"
    say(label)
    rng = np.random.default_rng(T * 131 + K)
    x = np.zeros((T, K), dtype=np.uint16)
    x[np.arange(T), rng.integers(0, K, T)] = 0x3F80
    q = rng.integers(-128, 128, (N, K))
    packed = np.ascontiguousarray((q + 128).astype(np.uint8)).view("<i4").reshape(N, K // 4)
    e = rng.integers(-6, 3, (N, K // G))
    scales = (((e + 127) << 7) | rng.integers(0, 128, (N, K // G))).astype(np.uint16)
    g = as_f64(run(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(packed).cuda(),
                   torch.from_numpy(scales.view(np.int16)).cuda(), T, N, K, G))
    o = oracle.int8_linear(x, packed, scales, G)
    o32 = o.astype(np.float32)
    assert np.array_equal(o32.astype(np.float64), o), "every exact value fits fp32"
    want = torch.from_numpy(o32).to(torch.bfloat16).double().numpy()   # round to nearest even
    bits = o32.view(np.uint32)
    tie = (bits & 0xFFFF) == 0x8000
    up = tie & ((bits >> 16) & 1 == 1)
    assert tie.sum() >= 50 and up.sum() >= 10 and (tie & ~up).sum() >= 10, (label, int(tie.sum()), int(up.sum()))
    bad = np.argwhere(g != want)
    assert bad.size == 0, (f"{label}: {len(bad)} outputs differ, first {bad[:3].tolist()} "
                           f"gpu {g[tuple(bad[0])]} exact {o[tuple(bad[0])]} rne {want[tuple(bad[0])]}")
