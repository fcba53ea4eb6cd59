"""CPU oracle for the INT4 group-quantized routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product library
and its binding never do.  It wraps ``moe_oracle.c`` (plain C, fp64, every
value computed from its definition) with ctypes and numpy and shares no code
with the HIP path.

Pages cited (by title and section):
  * "Running 125B MoE on Three 3090s - vLLM Optimization Edition", section 3.3,
    "MoE block (decode-05)": fused router + shared gate GEMV, top-k with ties
    to the lower id, renormalised softmax, block alignment (grouping slots by
    expert), INT6 shared expert combined as routed + sigmoid(gate) * shared;
    "Hyper-connection (decode-04)": pack-quantized words are least
    significant element first, stored with a +2^(bits-1) bias.
  * "Running 125B MoE on Three 3090s - vLLM Edition", section 1: hidden 2560,
    512 experts, top-10, expert intermediate 640.
  * Model card "Qwen3.8-Flash-Next-INT4-Mixed-AutoRound", "What is quantized":
    routed experts INT4 group 128 symmetric, shared expert INT6 group 64,
    router in bf16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_c_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into oracle/libmoe_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.oracle_int4_code.restype = ctypes.c_int
        L.oracle_int4_code.argtypes = [_ptr, _c_i64]
        L.oracle_int6_code.restype = ctypes.c_int
        L.oracle_int6_code.argtypes = [_ptr, _c_i64]
        L.oracle_dequant_int4.argtypes = [_ptr, _ptr, _c_i64, _c_i64, _c_i64, _ptr]
        L.oracle_dequant_int6.argtypes = [_ptr, _ptr, _c_i64, _c_i64, _c_i64, _ptr]
        L.oracle_router_logits.argtypes = [_ptr, _ptr, _c_i64, _c_i64, _c_i64, _ptr]
        L.oracle_topk_softmax.argtypes = [_ptr, _c_i64, _c_i64, _c_i64, _ptr, _ptr]
        L.oracle_permutation.argtypes = [_ptr, _c_i64, _c_i64, _c_i64, _ptr, _ptr, _ptr]
        L.oracle_experts.argtypes = [_ptr] * 7 + [_c_i64] * 5 + [_ptr, _ptr, ctypes.c_int]
        L.oracle_shared_int6.argtypes = [_ptr] * 6 + [_c_i64] * 4 + [_ptr, _ptr, _ptr, ctypes.c_int]
        L.oracle_forward.argtypes = ([_ptr] * 6 + [_c_i64] * 6 + [_ptr] * 5 + [_c_i64] * 3
                                     + [_ptr, _ptr, _ptr, _ptr, _ptr, ctypes.c_int])
        L.oracle_quantize_int4.argtypes = [_ptr, _c_i64, _c_i64, _c_i64, _ptr, _ptr, _ptr, _ptr]
        L.oracle_int8_code.restype = ctypes.c_int
        L.oracle_int8_code.argtypes = [_ptr, _c_i64]
        L.oracle_int8_linear.argtypes = [_ptr, _ptr, _ptr] + [_c_i64] * 4 + [_ptr]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _p(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def int4_code(row_words: np.ndarray, k: int) -> int:
    w = _c(row_words, np.int32)
    return int(lib().oracle_int4_code(_p(w), k))


def int6_code(row_words: np.ndarray, k: int) -> int:
    w = _c(row_words, np.int32)
    return int(lib().oracle_int6_code(_p(w), k))


def dequant_int4(packed: np.ndarray, scales: np.ndarray, group: int = 128) -> np.ndarray:
    """packed int32 [rows, K/8], scales bf16-bits uint16 [rows, K/group] -> fp64 [rows, K]."""
    p = _c(packed, np.int32)
    s = _c(scales, np.uint16)
    rows, K = p.shape[0], p.shape[1] * 8
    out = np.empty((rows, K), np.float64)
    lib().oracle_dequant_int4(_p(p), _p(s), rows, K, group, _p(out))
    return out


def dequant_int6(packed: np.ndarray, scales: np.ndarray, group: int = 64) -> np.ndarray:
    """packed int32 [rows, K/32*6], scales uint16 [rows, K/group] -> fp64 [rows, K]."""
    p = _c(packed, np.int32)
    s = _c(scales, np.uint16)
    rows, K = p.shape[0], p.shape[1] // 6 * 32
    out = np.empty((rows, K), np.float64)
    lib().oracle_dequant_int6(_p(p), _p(s), rows, K, group, _p(out))
    return out


def quantize_int4(w: np.ndarray, group: int = 128):
    """bf16-bits uint16 [rows, K] -> (packed int32 [rows, K/8], scales uint16
    [rows, K/group], best_err fp32 [rows, K/group], second_err fp32 [...]).

    Round to nearest, group 128, symmetric, per-group clip search minimising
    the squared error ("Running 125B MoE on Three 3090s - vLLM Optimization
    Edition", section 7); the readings are listed in moe_oracle.c."""
    w = _c(w, np.uint16)
    rows, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group")
    packed = np.empty((rows, K // 8), np.int32)
    scales = np.empty((rows, K // group), np.uint16)
    e1 = np.empty((rows, K // group), np.float32)
    e2 = np.empty((rows, K // group), np.float32)
    lib().oracle_quantize_int4(_p(w), rows, K, group, _p(packed), _p(scales), _p(e1), _p(e2))
    return packed, scales, e1, e2


def int8_code(row_words: np.ndarray, k: int) -> int:
    w = _c(row_words, np.int32)
    return int(lib().oracle_int8_code(_p(w), k))


def int8_linear(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """x bf16-bits uint16 [T, K], packed int32 [N, K/4], scales uint16
    [N, K/group] -> fp64 [T, N] = x . dequant(W)^T, exact up to fp64 sums.

    INT8 pack-quantized words ("Running 125B MoE on Three 3090s - vLLM
    Optimization Edition", section 3.3, "Hyper-connection (decode-04)"),
    symmetric groups of 64 or 128 (model card "What is quantized", groups C
    and D)."""
    x = _c(x, np.uint16)
    p = _c(packed, np.int32)
    s = _c(scales, np.uint16)
    T, K = x.shape
    N = p.shape[0]
    if p.shape[1] * 4 != K or s.shape != (N, K // group) or K % group:
        raise ValueError("inconsistent INT8 linear shapes")
    y = np.empty((T, N), np.float64)
    lib().oracle_int8_linear(_p(x), _p(p), _p(s), T, N, K, group, _p(y))
    return y


def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """x uint16 [T,H], router_w uint16 [E,H] (bf16 bits) -> fp32 [T,E]."""
    x = _c(x, np.uint16)
    w = _c(router_w, np.uint16)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_p(x), _p(w), T, H, E, _p(out))
    return out


def topk_softmax(logits: np.ndarray, k: int):
    """fp32 logits [T,E] -> (ids int32 [T,k], weights fp64 [T,k])."""
    l = _c(logits, np.float32)
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_topk_softmax(_p(l), T, E, k, _p(ids), _p(w))
    return ids, w


def permutation(ids: np.ndarray, E: int):
    """ids int32 [T,k] -> (counts [E], offsets [E+1], sorted_slots [T*k]), all int32."""
    i = _c(ids, np.int32)
    T, k = i.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slots = np.empty(T * k, np.int32)
    lib().oracle_permutation(_p(i), T, k, E, _p(counts), _p(offsets), _p(slots))
    return counts, offsets, slots


def experts(x, ids, weights, w13_packed, w13_scales, w2_packed, w2_scales,
            group: int = 128, tokens=None, nthreads: int = 0) -> np.ndarray:
    """Routed-expert combine for `tokens` (default: all) -> fp64 [len(tokens), H]."""
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float64)
    w13p, w13s = _c(w13_packed, np.int32), _c(w13_scales, np.uint16)
    w2p, w2s = _c(w2_packed, np.int32), _c(w2_scales, np.uint16)
    T, H = x.shape
    k = ids.shape[1]
    I = w2p.shape[2] * 8
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    out = np.empty((len(tok), H), np.float64)
    lib().oracle_experts(_p(x), _p(ids), _p(weights), _p(w13p), _p(w13s), _p(w2p), _p(w2s),
                         H, I, k, group, len(tok), _p(tok), _p(out), nthreads)
    return out


def shared_int6(x, gate_w, w13_packed, w13_scales, w2_packed, w2_scales,
                group: int = 64, tokens=None, nthreads: int = 0):
    """INT6 shared expert -> (ys fp64 [n,H], gate logits fp64 [n])."""
    x = _c(x, np.uint16)
    g = _c(gate_w, np.uint16)
    w13p, w13s = _c(w13_packed, np.int32), _c(w13_scales, np.uint16)
    w2p, w2s = _c(w2_packed, np.int32), _c(w2_scales, np.uint16)
    T, H = x.shape
    I = w2p.shape[1] // 6 * 32
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    ys = np.empty((len(tok), H), np.float64)
    gl = np.empty(len(tok), np.float64)
    lib().oracle_shared_int6(_p(x), _p(g), _p(w13p), _p(w13s), _p(w2p), _p(w2s),
                             H, I, group, len(tok), _p(tok), _p(ys), _p(gl), nthreads)
    return ys, gl


def forward(layer: dict, tokens=None, nthreads: int = 0):
    """Whole layer.  `layer` holds numpy arrays: x, router_w, w13_packed, w13_scales,
    w2_packed, w2_scales, top_k, group and optionally a 'shared' dict with gate_w,
    w13_packed, w13_scales, w2_packed, w2_scales, group.

    Returns dict(logits fp32 [T,E], ids [T,k], weights fp64 [T,k],
    out fp64 [n,H], tokens)."""
    x = _c(layer["x"], np.uint16)
    wr = _c(layer["router_w"], np.uint16)
    w13p, w13s = _c(layer["w13_packed"], np.int32), _c(layer["w13_scales"], np.uint16)
    w2p, w2s = _c(layer["w2_packed"], np.int32), _c(layer["w2_scales"], np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    I = w2p.shape[2] * 8
    k = int(layer["top_k"])
    group = int(layer.get("group", 128))
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    out = np.empty((len(tok), H), np.float64)
    sh = layer.get("shared")
    if sh is not None:
        sg = _c(sh["gate_w"], np.uint16)
        s13p, s13s = _c(sh["w13_packed"], np.int32), _c(sh["w13_scales"], np.uint16)
        s2p, s2s = _c(sh["w2_packed"], np.int32), _c(sh["w2_scales"], np.uint16)
        s_inter = s2p.shape[1] // 6 * 32
        s_group = int(sh.get("group", 64))
    else:
        sg = s13p = s13s = s2p = s2s = None
        s_inter = s_group = 0
    lib().oracle_forward(_p(x), _p(wr), _p(w13p), _p(w13s), _p(w2p), _p(w2s),
                         T, H, E, I, k, group,
                         _p(sg), _p(s13p), _p(s13s), _p(s2p), _p(s2s), s_inter, s_group,
                         len(tok), _p(tok), _p(logits), _p(ids), _p(w), _p(out), nthreads)
    return {"logits": logits, "ids": ids, "weights": w, "out": out, "tokens": tok}


def exempt_tokens(logits: np.ndarray, k: int, gap: float = 1e-3) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest logits differ by less than `gap`:
    their selection may legitimately differ between two correct summation orders."""
    T, E = logits.shape
    if k >= E:
        return np.zeros(T, bool)
    s = -np.sort(-logits.astype(np.float64), axis=1)
    return (s[:, k - 1] - s[:, k]) < gap
