"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Rules (tests/parity.py): expert ids bit-exact except near-tie tokens (oracle
k-th/(k+1)-th logit gap < 1e-3), histogram/offsets/permutation bit-exact,
bf16 output within max <= 2e-2 * rms and mean relative error <= 5e-3 of the
fp64 oracle.  Tokens whose ids legitimately differ are compared under oracle
routing through moe_int4_experts.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, check_output, check_routing
from quantized_moe_router_amd import _binding as B
from quantized_moe_router_amd import synth
from quantized_moe_router_amd.layer import MoeInt4Layer

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # the HIP library must be built; never fall back
    yield


REAL = synth.LayerShape(tokens=1)


@pytest.fixture(scope="module")
def real_weights():
    say("generating real-shape weights (seed 0)")
    w = synth.make_weights(REAL, seed=0)
    dev = {k: (torch.from_numpy(v.view(np.int16)).cuda() if v.dtype == np.uint16 else torch.from_numpy(v).cuda())
           for k, v in w.items() if k != "router_f32"}
    return w, dev


def _device_layer(host, real_dev=None):
    """Device copy of a host layer; reuses resident real-shape expert weights."""
    small = {k: v for k, v in host.items() if not (real_dev is not None and k in real_dev)}
    dev = synth.to_device(small)
    if real_dev is not None:
        dev.update(real_dev)
    return dev


def run_and_check(host, tokens=None, real_dev=None, label=""):
    shape = host["shape"]
    say(f"case {label}: T={shape.tokens} H={shape.hidden} E={shape.experts} k={shape.top_k} "
        f"I={shape.inter} shared={'shared' in host}")
    dev = _device_layer(host, real_dev)
    L = MoeInt4Layer(dev, shape.top_k, group=host["group"], shared=dev.get("shared"))
    out = L.forward(dev["x"])
    r = L.route(dev["x"])
    torch.cuda.synchronize()
    ref = oracle.forward(host, tokens=tokens)
    g = {k: v.cpu().numpy() for k, v in r.items()}
    T, k = shape.tokens, shape.top_k
    differ = check_routing(g["ids"], g["weights"], g["counts"], g["offsets"], g["sorted_slots"][:T * k],
                           ref["logits"], ref["ids"], ref["weights"], shape.experts)
    got = bf16_to_f64(out.cpu().numpy())[ref["tokens"]]
    if differ[ref["tokens"]].any():
        ids_o = torch.from_numpy(ref["ids"]).cuda()
        w_o = torch.from_numpy(ref["weights"].astype(np.float32)).cuda()
        out_o = L.experts(dev["x"], ids_o, w_o)
        torch.cuda.synchronize()
        got_o = bf16_to_f64(out_o.cpu().numpy())[ref["tokens"]]
        sel = differ[ref["tokens"]]
        got[sel] = got_o[sel]
        say(f"  {sel.sum()} near-tie token(s) compared under oracle routing")
    mx, mean, raw = check_output(got, ref["out"], label=label)
    say(f"  ok: max(beyond half-ulp)/rms={mx:.2e} raw max/rms={raw:.2e} mean-rel={mean:.2e} "
        f"exempt-differ={int(differ.sum())}")
    assert_workspaces_clean(L)
    return out, L, dev


def assert_workspaces_clean(L):
    """After a call completes: the sticky status word is zero (no bounded
    wait gave up) and the rest of the control prefix is back at zero."""
    torch.cuda.synchronize()
    for ws in L.workspaces():
        assert B.workspace_status(ws) == 0, f"status word {B.workspace_status(ws):#x}"
        assert B.workspace_prefix_clean(ws), "the workspace control prefix was not returned to zero"


# ---------------------------------------------------------------------------
# tiny shapes: every path, ragged sizes, edge cases
# ---------------------------------------------------------------------------

def test_tiny_config():
    run_and_check(synth.make_layer(synth.TINY, seed=0), label="tiny")


@pytest.mark.parametrize("T", [1, 2, 3, 7, 16, 17, 33, 100])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_tiny_ragged(T, k):
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=k, inter=128)
    run_and_check(synth.make_layer(shape, seed=10 + T, x_seed=100 + T * 7 + k), label=f"ragged T={T} k={k}")


@pytest.mark.parametrize("T", [5, 40])
def test_all_experts_selected(T):
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=16, inter=128)
    run_and_check(synth.make_layer(shape, seed=3), label=f"k=E T={T}")


@pytest.mark.parametrize("T,E,k", [(9, 64, 8), (21, 1000, 32), (3, 1024, 32)])
def test_many_experts_and_max_topk(T, E, k):
    shape = synth.LayerShape(tokens=T, hidden=256, experts=E, top_k=k, inter=128)
    run_and_check(synth.make_layer(shape, seed=4), label=f"E={E} k={k}")


@pytest.mark.parametrize("T", [3, 20])
def test_max_hidden_and_inter(T):
    shape = synth.LayerShape(tokens=T, hidden=4096, experts=8, top_k=2, inter=1024)
    run_and_check(synth.make_layer(shape, seed=5), label=f"H=4096 I=1024 T={T}")


@pytest.mark.parametrize("T", [4, 24])
def test_exact_ties_pick_lower_id(T):
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=4, inter=128)
    host = synth.make_layer(shape, seed=6)
    rw = host["router_w"].copy()
    rw[[3, 5, 9, 12]] = rw[1]           # five identical router rows: exact logit ties
    rw[[7, 8]] = rw[2]
    host["router_w"] = rw
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, shape.top_k)
    r = L.route(dev["x"])
    torch.cuda.synchronize()
    logits = oracle.router_logits(host["x"], rw)
    ids, _ = oracle.topk_softmax(logits, shape.top_k)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    run_and_check(host, label=f"ties T={T}")


def test_zero_tokens_is_a_no_op():
    shape = synth.LayerShape(tokens=0, hidden=256, experts=16, top_k=2, inter=128)
    dev = synth.to_device(synth.make_layer(shape, seed=0))
    L = MoeInt4Layer(dev, 2)
    out = torch.full((1, 256), 7, dtype=torch.int16, device="cuda")
    L.forward(dev["x"], out=out)
    torch.cuda.synchronize()
    assert (out == 7).all()


@pytest.mark.parametrize("T", [6, 50, 600])
def test_caller_routing_entry(T):
    """moe_int4_experts under arbitrary caller routing (distinct ids per token)."""
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=3, inter=128)
    host = synth.make_layer(shape, seed=7)
    rng = np.random.default_rng(T)
    ids = np.stack([rng.permutation(16)[:3] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, 3)).astype(np.float32)
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, 3)
    out = L.experts(dev["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = oracle.experts(host["x"], ids, w.astype(np.float64), host["w13_packed"], host["w13_scales"],
                         host["w2_packed"], host["w2_scales"])
    check_output(bf16_to_f64(out.cpu().numpy()), ref, label=f"caller routing T={T}")
    assert_workspaces_clean(L)


@pytest.mark.parametrize("T", [10240, 17000])
def test_large_permutation_against_stable_sort(T):
    """The three-pass permutation of many slots (S = 81920: 128 chunks, whose
    counts the scan keeps in registers; S = 136000: 133 chunks, the batched
    scan) against numpy's stable argsort of the returned ids: bit-exact
    counts, offsets and sorted slots (integer work, one correct answer)."""
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=8, inter=128)
    host = synth.make_layer(shape, seed=90 + T)
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, 8)
    r = L.route(dev["x"])
    torch.cuda.synchronize()
    ids = r["ids"].cpu().numpy().reshape(-1)
    counts = np.bincount(ids, minlength=16)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(r["sorted_slots"].cpu().numpy(), np.argsort(ids, kind="stable"))
    assert_workspaces_clean(L)


@pytest.mark.parametrize("T,shared", [(600, False), (1111, False), (700, True)])
def test_many_rows_per_expert(T, shared):
    """Over 128 rows per expert on average: every expert spans several
    128-row tiles with a ragged last one, and the dense shared-expert GEMMs
    end in a ragged token tile.  Every token checked against the oracle."""
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=4, inter=256)
    host = synth.make_layer(shape, seed=30 + T, shared=shared)
    assert T * 4 >= 128 * 16
    run_and_check(host, label=f"many rows per expert T={T} shared={shared}")


def test_shared_expert_whole_chunk_gemm_ragged():
    """From 6144 tokens the shared expert's gate/up runs as the whole-chunk
    GEMM (192 tokens per workgroup): 6211 tokens end in a ragged chunk of 67.
    Tokens of the first chunk, the last full one, the ragged one and random
    ones are checked against the oracle."""
    T = 6211
    shape = synth.LayerShape(tokens=T, hidden=512, experts=16, top_k=2, inter=128)
    host = synth.make_layer(shape, seed=61, shared=True)
    rng = np.random.default_rng(61)
    tokens = np.unique(np.concatenate([[0, 1, 191, 192], np.arange(5952, 5952 + 3), np.arange(T - 67, T),
                                       rng.choice(T, 24, replace=False)]))
    run_and_check(host, tokens=tokens, label="shared whole-chunk ragged T=6211")


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("H,I", [(256, 128), (768, 384), (512, 768), (512, 896)])
def test_whole_expert_gemm_row_counts(H, I, group):
    """Caller routing that gives the experts every row count the whole-expert
    grouped GEMM distinguishes: 0, 1 and 2 to 6 row tiles of 32 (ragged and
    full), exactly one chunk (192 rows) and counts that split into two or
    three chunks; ids may repeat within a token.  Every token is checked.
    The down projection keeps half a chunk's h rows in LDS up to I = 768
    (with fewer 64-column output groups than waves at H = 256, and an uneven
    share at H = 768); I = 896 takes the block-loop kernel instead.  At group
    64 a 128-input stage holds two scale groups (MFMA step j reads group
    j / 4)."""
    counts = [0, 1, 5, 31, 32, 33, 63, 64, 96, 150, 160, 191, 192, 193, 300, 385]
    k = 4
    S = sum(counts)
    counts[-1] += (-S) % k
    S = sum(counts)
    T = S // k
    assert S >= 64 * 16   # the whole-expert path is the one taken
    shape = synth.LayerShape(tokens=T, hidden=H, experts=16, top_k=k, inter=I, group=group)
    host = synth.make_layer(shape, seed=77 + H + group)
    rng = np.random.default_rng(H)
    ids = rng.permutation(np.repeat(np.arange(16), counts)).astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, k, group=group)
    out = L.experts(dev["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = oracle.experts(host["x"], ids, w.astype(np.float64), host["w13_packed"], host["w13_scales"],
                         host["w2_packed"], host["w2_scales"], group=group)
    check_output(bf16_to_f64(out.cpu().numpy()), ref,
                 label=f"whole-expert GEMM row counts H={H} I={I} group={group}")
    assert_workspaces_clean(L)


@pytest.mark.parametrize("T", [2, 30])
def test_deterministic(T):
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=2, inter=128)
    dev = synth.to_device(synth.make_layer(shape, seed=8))
    L = MoeInt4Layer(dev, 2)
    a = L.forward(dev["x"]).clone()
    b = L.forward(dev["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_repeated_calls_share_workspace(T):
    """Consecutive decode forwards on one workspace, alternating inputs: each
    call sees only its own routing and activations, and the counters at the
    head of the workspace are back at zero after each call."""
    shape = synth.LayerShape(tokens=T, hidden=512, experts=64, top_k=4, inter=256)
    host = synth.make_layer(shape, seed=21)
    dev = synth.to_device(host)
    x2 = synth.to_device(synth.make_layer(shape, seed=21, x_seed=77))["x"]
    L = MoeInt4Layer(dev, shape.top_k)
    first = [L.forward(dev["x"]).clone(), L.forward(x2).clone()]
    torch.cuda.synchronize()
    for i in range(6):
        got = L.forward(dev["x"] if i % 2 == 0 else x2)
        torch.cuda.synchronize()
        assert torch.equal(got, first[i % 2]), f"call {i}"
    assert_workspaces_clean(L)
    fresh = MoeInt4Layer(dev, shape.top_k).forward(dev["x"])   # a new zeroed workspace
    torch.cuda.synchronize()
    assert torch.equal(fresh, first[0])


def test_one_workspace_across_shapes():
    """One workspace buffer serves calls of different token counts (decode and
    many-token paths, forward and routing-only) in any order: each result
    equals the result on a fresh workspace, and the control prefix is zero
    after every call (the status word included)."""
    base = dict(hidden=512, experts=64, top_k=4, inter=256)
    host = synth.make_layer(synth.LayerShape(tokens=40, **base), seed=23)
    dev = synth.to_device(host)
    L = MoeInt4Layer(dev, base["top_k"])
    xs = {T: synth.to_device(synth.make_layer(synth.LayerShape(tokens=T, **base), seed=23,
                                              x_seed=100 + T))["x"] for T in (1, 4, 16, 40)}
    nbytes = max(B.workspace_bytes(L.shape(T)) for T in xs)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    w = dev
    for T, what in [(4, "forward"), (40, "forward"), (1, "forward"), (16, "route"), (4, "forward"),
                    (16, "forward"), (1, "route")]:
        say(f"T={T} {what}")
        ref = MoeInt4Layer(dev, base["top_k"])   # fresh workspaces
        if what == "forward":
            want = ref.forward(xs[T])
            got = torch.empty_like(want)
            B.moe_int4_forward(xs[T], w["router_w"], w["w13_packed"], w["w13_scales"], w["w2_packed"],
                               w["w2_scales"], base["top_k"], got, L.shape(T), None, ws)
            torch.cuda.synchronize()
            assert torch.equal(got, want), f"T={T} forward"
        else:
            want = ref.route(xs[T])
            k = base["top_k"]
            got = {"ids": torch.empty(T, k, dtype=torch.int32, device="cuda"),
                   "weights": torch.empty(T, k, dtype=torch.float32, device="cuda"),
                   "counts": torch.empty(64, dtype=torch.int32, device="cuda"),
                   "offsets": torch.empty(65, dtype=torch.int32, device="cuda"),
                   "sorted_slots": torch.empty(T * k, dtype=torch.int32, device="cuda")}
            B.moe_int4_route(xs[T], w["router_w"], L.shape(T), got["ids"], got["weights"], got["counts"],
                             got["offsets"], got["sorted_slots"], ws)
            torch.cuda.synchronize()
            for key in got:
                assert torch.equal(got[key], want[key]), f"T={T} route {key}"
        assert B.workspace_prefix_clean(ws), f"T={T} {what}: the control prefix was not returned to zero"


@pytest.mark.parametrize("H,I,E,k", [(768, 384, 40, 6), (1280, 128, 100, 3)])
@pytest.mark.parametrize("T", [1, 3, 19, 70])
@pytest.mark.parametrize("shared", [False, True])
def test_ragged_widths(H, I, E, k, T, shared):
    """Widths that leave partial lane chunks: hidden 768 / 1280 is 24 / 40
    chunks of 32 over the 16 lanes of a decode row group, 3 / 5 blocks of 256
    rows in the many-token down GEMM; 40 and 100 experts leave the last
    64-expert key block partly empty."""
    shape = synth.LayerShape(tokens=T, hidden=H, experts=E, top_k=k, inter=I)
    host = synth.make_layer(shape, seed=31 + T + H, shared=shared)
    run_and_check(host, label=f"ragged widths H={H} I={I} E={E} k={k} T={T} shared={shared}")


def test_tiny_shared_expert():
    for T in (3, 40):
        shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=2, inter=128)
        host = synth.make_layer(shape, seed=9, shared=True)
        run_and_check(host, label=f"tiny shared T={T}")


# ---------------------------------------------------------------------------
# real shape (hidden 2560, 512 experts, top-10, intermediate 640)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 4])
def test_real_decode(real_weights, T):
    w, dev = real_weights
    shape = synth.LayerShape(tokens=T)
    host = synth.make_layer(shape, seed=0, x_seed=1000 + T, weights=w)
    run_and_check(host, real_dev=dev, label=f"real decode T={T}")


@pytest.mark.parametrize("T,shared", [(6, False), (8, False), (16, False), (8, True)])
def test_real_decode_token_groups(real_weights, T, shared):
    """Few-token batches of 6 to 16 tokens at the real shape, group 128: more
    slots than one pass of the down projection's lane groups covers, and
    (T = 16) the largest batch of the few-token path."""
    w, dev = real_weights
    shape = synth.LayerShape(tokens=T)
    host = synth.make_layer(shape, seed=0, x_seed=5000 + T, weights=w, shared=shared)
    run_and_check(host, real_dev=dev, label=f"real decode T={T} shared={shared}")


def _extreme_layer(T, seed):
    """Activations whose magnitudes are spread log-uniformly over [1e-4, 6e4]
    with random signs (bf16, inside fp16's exact range), with the router and
    gate/up scales taken down by 2^-16 (exact in bf16) so that logits and the
    SwiGLU activation stay in their usual range."""
    shape = synth.LayerShape(tokens=T, hidden=1024, experts=32, top_k=4, inter=256)
    host = synth.make_layer(shape, seed=seed)
    rng = np.random.default_rng(seed + 99)
    mag = np.exp(rng.uniform(np.log(1e-4), np.log(6e4), (T, 1024)))
    x = (mag * rng.choice([-1.0, 1.0], (T, 1024))).astype(np.float32)
    host["x"] = synth.bf16_bits(x)
    xf = bf16_to_f64(host["x"])
    assert np.abs(xf).max() <= 65504 and np.abs(xf).min() >= 2.0 ** -14
    def down16(b):   # bf16 bits * 2^-16: exponent field - 16 (all values are normal)
        b = b.astype(np.uint16)
        e = (b >> 7) & 0xFF
        assert (e > 16).all()
        return ((b & 0x807F) | ((e - 16) << 7)).astype(np.uint16)
    host["router_w"] = down16(host["router_w"])
    host["w13_scales"] = down16(host["w13_scales"])
    return host


@pytest.mark.parametrize("T", [16, 17])
def test_extreme_activations_in_range(T):
    """The largest few-token batch (bf16 activations used as they are) and the
    smallest matrix-core batch (activations converted to fp16) give the same
    parity on activations from 1e-4 to 6e4 in magnitude."""
    run_and_check(_extreme_layer(T, 4100), label=f"extreme activations T={T}")


def test_real_decode_batch64(real_weights):
    w, dev = real_weights
    shape = synth.LayerShape(tokens=64)
    host = synth.make_layer(shape, seed=0, x_seed=2064, weights=w)
    run_and_check(host, tokens=np.arange(0, 64, 4), real_dev=dev, label="real decode T=64")


def test_real_prefill512_zipf(real_weights):
    w, dev = real_weights
    shape = synth.LayerShape(tokens=512)
    host = synth.make_layer(shape, seed=0, x_seed=3512, zipf_s=1.1, weights=w)
    counts = None
    tokens = np.random.default_rng(0).choice(512, 40, replace=False)
    out, L, ddev = run_and_check(host, tokens=tokens, real_dev=dev, label="prefill 512 zipf")
    counts = L.route(ddev["x"])["counts"].cpu().numpy()
    say(f"  zipf: {np.count_nonzero(counts)} experts touched, max {counts.max()} slots")
    assert counts.max() >= 100 and np.count_nonzero(counts) < 400


def test_real_prefill8192_shared(real_weights):
    w, dev = real_weights
    shape = synth.LayerShape(tokens=8192)
    host = synth.make_layer(shape, seed=0, x_seed=48192, shared=True, weights=w)
    tokens = np.random.default_rng(1).choice(8192, 24, replace=False)
    run_and_check(host, tokens=tokens, real_dev=dev, label="prefill 8192 + shared")


@pytest.mark.parametrize("T,shared", [(1, False), (5, False), (40, False), (40, True), (300, True)])
def test_graph_replay_matches_eager(T, shared):
    """The forward captured in a HIP graph gives the eager result on every
    replay, with other eager work in between (no memset nodes; the
    workspace counters return to zero after each call).  With the shared
    expert, a many-token forward forks it onto a second stream and joins it
    before the combine; the capture records that fork and join."""
    shape = synth.LayerShape(tokens=T, hidden=256, experts=16, top_k=2, inter=128)
    a = synth.to_device(synth.make_layer(shape, seed=11, shared=shared))
    b = synth.to_device(synth.make_layer(shape, seed=12, shared=shared))
    La = MoeInt4Layer(a, 2, shared=a.get("shared"))
    Lb = MoeInt4Layer(b, 2, shared=b.get("shared"))
    eager = La.forward(a["x"]).clone()
    other = Lb.forward(b["x"]).clone()
    out = torch.empty_like(eager)
    La.forward(a["x"], out=out)            # workspace exists before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        La.forward(a["x"], out=out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(Lb.forward(b["x"]), other)
        torch.cuda.synchronize()


def test_shared_expert_side_stream_from_two_threads():
    """Many-token forwards with the shared expert fork it onto one side stream
    per device.  Two host threads enqueue forwards of two layers (own
    workspaces) on two torch streams at once, several times each: every
    result equals that layer's result computed alone."""
    import threading
    shape = synth.LayerShape(tokens=300, hidden=256, experts=16, top_k=2, inter=128)
    devs = [synth.to_device(synth.make_layer(shape, seed=70 + i, shared=True)) for i in range(2)]
    layers = [MoeInt4Layer(d, 2, shared=d.get("shared")) for d in devs]
    want = [layers[i].forward(devs[i]["x"]).clone() for i in range(2)]
    torch.cuda.synchronize()
    got = [[], []]
    errors = []

    def run(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(6):
                    got[i].append(layers[i].forward(devs[i]["x"]).clone())
            st.synchronize()
        except Exception as exc:   # reported below, in the test's thread
            errors.append(exc)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(got[i]) == 6
        for r in got[i]:
            assert torch.equal(r, want[i])


# ---- INT4 group 64 on the same kernels ("Running 125B MoE on Three 3090s -
# vLLM Edition", section 2: the group-64 alternative to group 128) ----

@pytest.mark.parametrize("T", [1, 4, 16, 17, 70, 600])
def test_group64_ragged(T):
    shape = synth.LayerShape(tokens=T, hidden=768, experts=40, top_k=6, inter=384, group=64)
    run_and_check(synth.make_layer(shape, seed=500 + T), label=f"group64 T={T}")


@pytest.mark.parametrize("T,shared", [(1, False), (4, True), (512, True)])
def test_group64_real_width(T, shared):
    # hidden 2560, intermediate 640, top-10 over 64 experts (one GPU's share
    # under 8-way expert parallelism)
    shape = synth.LayerShape(tokens=T, experts=64, group=64)
    host = synth.make_layer(shape, seed=600 + T, shared=shared)
    toks = None if T <= 64 else np.arange(0, T, 7)
    run_and_check(host, tokens=toks, label=f"group64 real-width T={T}")


def test_y_past_2gib_sampled():
    """16384 tokens at top-32 over 64 experts (hidden 2048, intermediate 128):
    524,288 slots, so y (T x 33 rows x 2048 fp16) is 2.2 GB, past the 2^31
    bytes the resident down GEMM addresses through a buffer resource; it
    stores through 64-bit addresses instead.  The permutation runs its
    batched scan (more than 128 chunks).  Routing is checked for every token,
    outputs for sampled ones."""
    shape = synth.LayerShape(tokens=16384, hidden=2048, experts=64, top_k=32, inter=128)
    host = synth.make_layer(shape, seed=91)
    rng = np.random.default_rng(91)
    tokens = np.unique(np.concatenate([[0, 1, 8191, 16383], rng.choice(16384, 24, replace=False)]))
    run_and_check(host, tokens=tokens, label="y past 2 GiB, T=16384 k=32")


def test_large_permutation_many_experts():
    # 700 tokens x top-32 over 1000 experts: 22400 slots, past the
    # one-workgroup permutation (16384), so the three-pass path runs with
    # nearly the largest expert count
    shape = synth.LayerShape(tokens=700, hidden=256, experts=1000, top_k=32, inter=128)
    run_and_check(synth.make_layer(shape, seed=4242), label="large permutation, E=1000, k=32")


# ---- seeded sweep over random legal shapes ----
def _sweep_cases(n=32, seed=2026):
    """Shapes drawn uniformly from what the boundary accepts (hidden a
    multiple of 256 up to 4096, intermediate a multiple of 128 up to 1024,
    1-1024 experts, top-k up to 32, group 64 or 128, with or without the
    shared expert), tokens log-uniform in [1, 700]; draws whose host weights
    or oracle work would be large are skipped, so the sweep stays a few
    seconds per case."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        H = 256 * int(rng.integers(1, 17))
        I = 128 * int(rng.integers(1, 9))
        E = int(rng.integers(1, 1025))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(np.exp(rng.uniform(0.0, np.log(700.0))))
        shared = bool(rng.integers(0, 2))
        group = int(rng.choice([64, 128]))
        if E * I * H > 1.3e8 or T * k * H * I * 3 > 3e9:
            continue
        out.append((T, H, I, E, k, shared, group))
    return out


@pytest.mark.parametrize("T,H,I,E,k,shared,group", _sweep_cases())
def test_random_shape_sweep(T, H, I, E, k, shared, group):
    shape = synth.LayerShape(tokens=T, hidden=H, experts=E, top_k=k, inter=I, group=group)
    host = synth.make_layer(shape, seed=7000 + T + E, shared=shared)
    run_and_check(host, label=f"sweep T={T} H={H} I={I} E={E} k={k} shared={shared} group={group}")


def test_topk_one_split_many_experts():
    """8192 tokens over 1024 experts (hidden 256): 512 router output tiles, so
    the router GEMM does not split K and the top-k kernel runs its one-split
    variant with 16 experts per lane.  Routing is checked for every token,
    outputs for sampled ones."""
    shape = synth.LayerShape(tokens=8192, hidden=256, experts=1024, top_k=8, inter=128)
    host = synth.make_layer(shape, seed=8192)
    rng = np.random.default_rng(8192)
    tokens = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 30, replace=False)]))
    run_and_check(host, tokens=tokens, label="top-k one split, T=8192 E=1024")


def test_group64_prefill8192_share():
    """Group 64 through the whole-expert GEMMs at the real width: 8192 tokens,
    top-10 over 64 experts (1,280 rows per expert, seven chunks each) and the
    shared expert; routing for every token, outputs for sampled ones."""
    shape = synth.LayerShape(tokens=8192, experts=64, group=64)
    host = synth.make_layer(shape, seed=6464, shared=True)
    rng = np.random.default_rng(6464)
    tokens = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 30, replace=False)]))
    run_and_check(host, tokens=tokens, label="group64 real-width T=8192 E=64 shared")
