"""ctypes binding of libmoe_int4.so (include/moe_int4.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors on the current HIP device; bf16 data may be passed
as torch.bfloat16 or as int16/uint16 bit patterns.  Work is enqueued on
torch's current stream unless a stream is given.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_int4.so")

OK, EINVAL, EALIGN, EWORKSPACE, ELAUNCH, EDEVICE = 0, -1, -2, -3, -4, -5

_c_void_p = ctypes.c_void_p
_c_i32 = ctypes.c_int32


class MoeShape(ctypes.Structure):
    _fields_ = [("tokens", _c_i32), ("hidden", _c_i32), ("experts", _c_i32),
                ("inter", _c_i32), ("group", _c_i32), ("top_k", _c_i32)]


class MoeSharedInt6(ctypes.Structure):
    _fields_ = [("gate_w", _c_void_p), ("w13_packed", _c_void_p), ("w13_scales", _c_void_p),
                ("w2_packed", _c_void_p), ("w2_scales", _c_void_p),
                ("inter", _c_i32), ("group", _c_i32)]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_int4 error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m quantized_moe_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = _c_void_p
        L.moe_int4_workspace_bytes.argtypes = [P, P, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_int4_route.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_int4_experts.argtypes = [P] * 11 + [ctypes.c_size_t, P]
        L.moe_int4_forward.argtypes = [P] * 6 + [_c_i32, P, P, P, P, ctypes.c_size_t, P]
        L.moe_int4_forward_traced.argtypes = [P] * 6 + [_c_i32, P, P, P, P, ctypes.c_size_t, P, P]
        L.moe_int4_forward_noalloc.argtypes = [P] * 6 + [_c_i32, P, P, P, P, P]
        L.moe_int4_quantize.argtypes = [P, _c_i32, _c_i32, _c_i32, P, P, P]
        L.moe_int8_linear_workspace_bytes.argtypes = [_c_i32] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
        L.moe_int8_linear.argtypes = [P, P, P] + [_c_i32] * 4 + [P, P, ctypes.c_size_t, P]
        L.moe_int4_last_error.restype = ctypes.c_char_p
        L.moe_int4_version.restype = ctypes.c_char_p
        for f in ("moe_int4_workspace_bytes", "moe_int4_route", "moe_int4_experts", "moe_int4_forward",
                  "moe_int4_forward_traced", "moe_int4_forward_noalloc", "moe_int4_quantize",
                  "moe_int8_linear_workspace_bytes", "moe_int8_linear"):
            getattr(L, f).restype = _c_i32
        _lib = L
    return _lib


EXPORTED = ("moe_int4_workspace_bytes", "moe_int4_route", "moe_int4_experts",
            "moe_int4_forward", "moe_int4_forward_traced", "moe_int4_forward_noalloc",
            "moe_int4_quantize",
            "moe_int8_linear_workspace_bytes", "moe_int8_linear",
            "moe_int4_last_error", "moe_int4_version")


def _check(rc: int):
    if rc != OK:
        raise MoeError(rc, lib().moe_int4_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_shape(tokens, hidden, experts, inter, top_k, group=128) -> MoeShape:
    return MoeShape(tokens, hidden, experts, inter, group, top_k)


def make_shared(sh: dict | None) -> MoeSharedInt6 | None:
    """sh: dict of device tensors gate_w, w13_packed, w13_scales, w2_packed, w2_scales."""
    if sh is None:
        return None
    inter = sh["w2_packed"].shape[1] // 6 * 32
    return MoeSharedInt6(_ptr(sh["gate_w"]), _ptr(sh["w13_packed"]), _ptr(sh["w13_scales"]),
                         _ptr(sh["w2_packed"]), _ptr(sh["w2_scales"]), inter, int(sh.get("group", 64)))


def workspace_bytes(shape: MoeShape, shared: MoeSharedInt6 | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_int4_workspace_bytes(ctypes.byref(shape),
                                          ctypes.byref(shared) if shared else None, ctypes.byref(n)))
    return n.value


# Workspace control prefix (include/moe_int4.h): zero between calls, except
# the sticky status word at WS_STATUS_OFFSET.
WS_PREFIX_BYTES = 65792
WS_STATUS_OFFSET = 65536
STATUS_KEY_WAIT, STATUS_ROUTE_WAIT, STATUS_H_WAIT = 1, 2, 4


def new_workspace(shape: MoeShape, shared: MoeSharedInt6 | None = None, device="cuda"):
    """A zero-filled workspace (the library keeps its counters at zero after each call)."""
    import torch
    return torch.zeros(workspace_bytes(shape, shared), dtype=torch.uint8, device=device)


def workspace_status(workspace) -> int:
    """The sticky status word of a workspace (reads device memory: call after
    the stream has completed)."""
    w = workspace[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 4].cpu().numpy()
    return int(w.view("<u4")[0])


def workspace_prefix_clean(workspace) -> bool:
    """Whether the control prefix is back at zero, status word included."""
    return not bool(workspace[:WS_PREFIX_BYTES].any().item())


def moe_int4_route(x, router_w, shape: MoeShape, topk_ids, topk_w, expert_counts,
                   expert_offsets, sorted_slots, workspace, stream=None):
    _check(lib().moe_int4_route(_ptr(x), _ptr(router_w), ctypes.byref(shape), _ptr(topk_ids),
                                _ptr(topk_w), _ptr(expert_counts), _ptr(expert_offsets),
                                _ptr(sorted_slots), _ptr(workspace), workspace.numel(),
                                _stream(stream)))


def moe_int4_experts(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales,
                     shape: MoeShape, shared: MoeSharedInt6 | None, out, workspace, stream=None):
    _check(lib().moe_int4_experts(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w13_packed),
                                  _ptr(w13_scales), _ptr(w2_packed), _ptr(w2_scales),
                                  ctypes.byref(shape), ctypes.byref(shared) if shared else None,
                                  _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_int4_forward(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k: int, out,
                     shape: MoeShape, shared: MoeSharedInt6 | None, workspace, stream=None):
    _check(lib().moe_int4_forward(_ptr(x), _ptr(router_w), _ptr(w13_packed), _ptr(w13_scales),
                                  _ptr(w2_packed), _ptr(w2_scales), int(top_k), _ptr(out),
                                  ctypes.byref(shape), ctypes.byref(shared) if shared else None,
                                  _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_int4_forward_traced(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k: int,
                            out, shape: MoeShape, shared: MoeSharedInt6 | None, workspace, events,
                            stream=None):
    """events: four hipEvent_t handles (ints), or four torch.cuda.Event(enable_timing=True)
    already recorded once (torch creates the underlying event lazily); they are
    re-recorded between the stages."""
    arr = (ctypes.c_void_p * 4)(*[e.cuda_event if hasattr(e, "cuda_event") else int(e) for e in events])
    if not all(arr):
        raise ValueError("record each torch.cuda.Event once before passing it (lazy creation)")
    _check(lib().moe_int4_forward_traced(_ptr(x), _ptr(router_w), _ptr(w13_packed), _ptr(w13_scales),
                                         _ptr(w2_packed), _ptr(w2_scales), int(top_k), _ptr(out),
                                         ctypes.byref(shape), ctypes.byref(shared) if shared else None,
                                         _ptr(workspace), workspace.numel(), _stream(stream), arr))


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_INT4_NOALLOC_SCRATCH_BYTES


def moe_int4_forward_noalloc(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k: int,
                             out, shape: MoeShape, shared: MoeSharedInt6 | None, status=None,
                             stream=None):
    """moe_int4_forward without a workspace (the library's static per-device
    scratch); status: optional device uint32 tensor that failed waits OR into."""
    _check(lib().moe_int4_forward_noalloc(_ptr(x), _ptr(router_w), _ptr(w13_packed), _ptr(w13_scales),
                                          _ptr(w2_packed), _ptr(w2_scales), int(top_k), _ptr(out),
                                          ctypes.byref(shape), ctypes.byref(shared) if shared else None,
                                          _ptr(status), _stream(stream)))


def moe_int4_quantize(w, rows: int, cols: int, packed, scales, group: int = 128, stream=None):
    """w bf16 [rows, cols] (device) -> packed int32 [rows, cols/8], scales bf16 [rows, cols/group]."""
    _check(lib().moe_int4_quantize(_ptr(w), int(rows), int(cols), int(group), _ptr(packed),
                                   _ptr(scales), _stream(stream)))


def moe_int8_linear_workspace_bytes(tokens: int, n: int, k: int, group: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().moe_int8_linear_workspace_bytes(int(tokens), int(n), int(k), int(group), ctypes.byref(b)))
    return b.value


def moe_int8_linear(x, w_packed, w_scales, tokens: int, n: int, k: int, group: int, out,
                    workspace=None, stream=None):
    """x bf16 [tokens, k], w_packed int32 [n, k/4], w_scales bf16 [n, k/group] ->
    out bf16 [tokens, n] (device tensors; workspace uint8, may be None when the
    shape needs none)."""
    _check(lib().moe_int8_linear(_ptr(x), _ptr(w_packed), _ptr(w_scales), int(tokens), int(n), int(k),
                                 int(group), _ptr(out), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(stream)))


def version() -> str:
    return lib().moe_int4_version().decode()
