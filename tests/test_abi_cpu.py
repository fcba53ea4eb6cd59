"""The C-ABI library loads, exports what include/moe_int4.h declares, and
rejects bad arguments on the host (no GPU needed: every check runs before
anything touches a device)."""
import ctypes
import os
import re

import pytest

from quantized_moe_router_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moe_int4.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(moe_int[48]_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared()
    assert set(names) >= {"moe_int4_forward", "moe_int4_route", "moe_int4_experts",
                          "moe_int4_workspace_bytes", "moe_int4_last_error", "moe_int8_linear",
                          "moe_int8_linear_workspace_bytes"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTED) <= set(names)
    assert B.version().startswith("moe_int4")


def _shape(**kw):
    d = dict(tokens=4, hidden=2560, experts=512, inter=640, top_k=10, group=128)
    d.update(kw)
    return B.make_shape(d["tokens"], d["hidden"], d["experts"], d["inter"], d["top_k"], d["group"])


@pytest.mark.parametrize("kw,msg", [
    (dict(group=32), "group"),
    (dict(group=256), "group"),
    (dict(hidden=2500), "hidden"),
    (dict(hidden=8192), "hidden"),
    (dict(inter=100), "inter"),
    (dict(experts=0), "experts"),
    (dict(experts=2048), "experts"),
    (dict(top_k=0), "top_k"),
    (dict(top_k=33), "top_k"),
    (dict(experts=8, top_k=9), "top_k"),
    (dict(tokens=-1), "tokens"),
])
def test_bad_shapes_rejected(kw, msg):
    n = ctypes.c_size_t(0)
    rc = B.lib().moe_int4_workspace_bytes(ctypes.byref(_shape(**kw)), None, ctypes.byref(n))
    assert rc == B.EINVAL
    assert msg in B.lib().moe_int4_last_error().decode()


def test_workspace_size_grows_with_tokens():
    a = B.workspace_bytes(_shape(tokens=1))
    b = B.workspace_bytes(_shape(tokens=4))
    c = B.workspace_bytes(_shape(tokens=8192))
    assert 0 < a < b < c
    assert B.workspace_bytes(_shape(tokens=0)) > 0


FAKE = 0x10000  # never dereferenced: validation fails before any device access


def _forward(shape, ptrs=None, top_k=10, ws_bytes=1 << 40):
    p = dict(x=FAKE, router=FAKE, w13p=FAKE, w13s=FAKE, w2p=FAKE, w2s=FAKE, out=FAKE * 2, ws=FAKE)
    p.update(ptrs or {})
    return B.lib().moe_int4_forward(p["x"], p["router"], p["w13p"], p["w13s"], p["w2p"], p["w2s"],
                                    top_k, p["out"], ctypes.byref(shape), None, p["ws"], ws_bytes, None)


def test_forward_argument_errors():
    s = _shape()
    assert _forward(s, {"x": None}) == B.EINVAL
    assert "x is NULL" in B.lib().moe_int4_last_error().decode()
    assert _forward(s, {"w13p": FAKE + 4}) == B.EALIGN
    assert _forward(s, top_k=8) == B.EINVAL
    assert "top_k" in B.lib().moe_int4_last_error().decode()
    assert _forward(s, {"out": FAKE}) == B.EINVAL          # out aliases x
    assert _forward(s, ws_bytes=16) == B.EWORKSPACE
    assert _forward(s, {"ws": None}) == B.EINVAL


def _noalloc(shape, ptrs=None, top_k=10, status=None):
    p = dict(x=FAKE, router=FAKE, w13p=FAKE, w13s=FAKE, w2p=FAKE, w2s=FAKE, out=FAKE * 2)
    p.update(ptrs or {})
    return B.lib().moe_int4_forward_noalloc(p["x"], p["router"], p["w13p"], p["w13s"], p["w2p"], p["w2s"],
                                            top_k, p["out"], ctypes.byref(shape), None, status, None)


def test_noalloc_argument_errors():
    L = B.lib()
    s = _shape()
    assert _noalloc(s, {"x": None}) == B.EINVAL
    assert "x is NULL" in L.moe_int4_last_error().decode()
    assert _noalloc(s, top_k=8) == B.EINVAL
    assert _noalloc(s, {"out": FAKE}) == B.EINVAL          # out aliases x
    assert _noalloc(s, status=FAKE + 2) == B.EALIGN
    big = _shape(tokens=8192)
    assert B.workspace_bytes(big) > B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == B.EWORKSPACE
    assert "static scratch" in L.moe_int4_last_error().decode()
    assert _noalloc(_shape(tokens=0)) == B.OK              # no-op
    with open(os.path.join(ROOT, "include", "moe_int4.h")) as f:
        m = re.search(r"#define MOE_INT4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES


def test_route_and_experts_argument_errors():
    s = _shape()
    L = B.lib()
    rc = L.moe_int4_route(FAKE, FAKE, ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert rc == B.EINVAL and "sorted_slots" in L.moe_int4_last_error().decode()
    rc = L.moe_int4_experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), None, FAKE * 2,
                            FAKE, 8, None)
    assert rc == B.EWORKSPACE
    bad = B.MoeSharedInt6(FAKE, FAKE, FAKE, FAKE, FAKE, 640, 128)
    rc = L.moe_int4_experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(bad),
                            FAKE * 2, FAKE, 1 << 40, None)
    assert rc == B.EINVAL and "group" in L.moe_int4_last_error().decode()


def test_no_device_is_reported_not_crashed():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = _forward(_shape())
    assert rc == B.EDEVICE
    assert _noalloc(_shape()) == B.EDEVICE


@pytest.mark.parametrize("rows,cols,group,msg", [
    (4, 256, 32, "group"),
    (4, 200, 128, "cols"),
    (-1, 256, 128, "rows"),
    (4, 0, 128, "cols"),
    (1 << 16, 1 << 15, 128, "2^31"),
])
def test_quantize_bad_arguments_rejected(rows, cols, group, msg):
    rc = B.lib().moe_int4_quantize(None, rows, cols, group, None, None, None)
    assert rc == B.EINVAL
    assert msg in B.lib().moe_int4_last_error().decode()


def test_quantize_zero_rows_is_a_no_op_and_null_buffers_rejected():
    assert B.lib().moe_int4_quantize(None, 0, 256, 128, None, None, None) == 0
    rc = B.lib().moe_int4_quantize(None, 2, 256, 128, None, None, None)
    assert rc == B.EINVAL and "w" in B.lib().moe_int4_last_error().decode()


# ---- INT8 W8A16 linear ----

def _i8_ws(tokens, n, k, group):
    b = ctypes.c_size_t(0)
    rc = B.lib().moe_int8_linear_workspace_bytes(tokens, n, k, group, ctypes.byref(b))
    return rc, b.value


@pytest.mark.parametrize("tokens,n,k,group,msg", [
    (1, 320, 10240, 32, "group"),
    (1, 320, 10240, 256, "group"),
    (1, 320, 10200, 64, "k="),
    (1, 320, 0, 64, "k="),
    (1, 320, 131072, 64, "k="),
    (1, 0, 2560, 128, "n="),
    (-1, 320, 2560, 128, "tokens"),
    (1 << 20, 1 << 12, 2560, 128, "2^31"),
])
def test_int8_bad_arguments_rejected(tokens, n, k, group, msg):
    rc, _ = _i8_ws(tokens, n, k, group)
    assert rc == B.EINVAL and msg in B.lib().moe_int4_last_error().decode()
    rc = B.lib().moe_int8_linear(None, None, None, tokens, n, k, group, None, None, 0, None)
    assert rc == B.EINVAL and msg in B.lib().moe_int4_last_error().decode()


def test_int8_workspace_plan():
    # few tokens: GEMV, no workspace; lm_head-like many rows: no K split;
    # the narrow hyper-connection down projection splits K (fp32 partials)
    assert _i8_ws(1, 248320, 2560, 128) == (0, 0)
    assert _i8_ws(4, 320, 2560, 64) == (0, 0)
    assert _i8_ws(512, 10240, 320, 64) == (0, 0)
    rc, b = _i8_ws(512, 320, 10240, 64)
    assert rc == 0 and b > 0 and b % (512 * 320 * 4) == 0 and 2 <= b // (512 * 320 * 4) <= 16


def test_int8_zero_tokens_no_op_and_checks_before_device():
    assert B.lib().moe_int8_linear(None, None, None, 0, 320, 10240, 64, None, None, 0, None) == 0
    rc = B.lib().moe_int8_linear(None, None, None, 2, 320, 10240, 64, None, None, 0, None)
    assert rc == B.EINVAL and "x" in B.lib().moe_int4_last_error().decode()
    fake = 1 << 20   # aligned, never dereferenced: every check runs on the host first
    rc = B.lib().moe_int8_linear(fake + 8, fake, fake, 2, 320, 2560, 64, fake, None, 0, None)
    assert rc == B.EALIGN and "x" in B.lib().moe_int4_last_error().decode()
    rc, need = _i8_ws(512, 320, 10240, 64)
    rc = B.lib().moe_int8_linear(fake, fake, fake, 512, 320, 10240, 64, fake, None, 0, None)
    assert rc == B.EINVAL and "workspace" in B.lib().moe_int4_last_error().decode()
    rc = B.lib().moe_int8_linear(fake, fake, fake, 512, 320, 10240, 64, fake, fake, need - 16, None)
    assert rc == B.EWORKSPACE
    import torch
    if not torch.cuda.is_available():
        rc = B.lib().moe_int8_linear(fake, fake, fake, 512, 320, 10240, 64, fake, fake, need, None)
        assert rc == B.EDEVICE
