"""CPU oracle for the batch-invariant linear, MoE and indexer top-k paths.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The HIP library
never imports, links or calls it, and it never imports the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, binary64 throughout, one
round-to-nearest-even per storage point, ascending-index sums); this module
only marshals numpy arrays into it.  bf16 tensors travel as ``numpy.uint16``
bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-std=c99", "-D_DEFAULT_SOURCE"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        L = ctypes.c_long
        lib.oracle_linear_f32.argtypes = [P, P, P, P, P, L, L, L]
        lib.oracle_linear_bf16.argtypes = [P, P, P, P, P, P, L, L, L]
        lib.oracle_topk.argtypes = [P, P, L, L, L]
        lib.oracle_moe.argtypes = [P, P, P, P, P, L, L, L, L, L, P, P, P, P, P]
        lib.oracle_f64_to_bf16.argtypes = [P, P, L]
        lib.oracle_topk_rows.argtypes = [P, L, L, L, P, P, L, P, L]
        C = ctypes.c_int
        lib.oracle_moe_ex.argtypes = [P, P, P, P, P, L, L, L, L, L, C, C, C, C, P, P, P, P, P]
        lib.oracle_moe_stages.argtypes = [P, P, P, P, P, L, L, L, L, L, C, C, C, C, P, P, P, P, P, P, P, P]
        lib.oracle_moe_activation.argtypes = [P, P, L, L, C, C, P]
        lib.oracle_moe_combine.argtypes = [P, P, L, L, L, C, C, P]
        for f in (lib.oracle_linear_f32, lib.oracle_linear_bf16, lib.oracle_topk,
                  lib.oracle_moe, lib.oracle_f64_to_bf16, lib.oracle_num_threads,
                  lib.oracle_topk_rows, lib.oracle_moe_ex, lib.oracle_moe_stages, lib.oracle_moe_activation,
                  lib.oracle_moe_combine):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def linear_f32(x, w, bias=None, want_f64=False):
    """y = RN_f32(x @ w.T + bias) with binary64 accumulation; w is [N, K]."""
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    bias = _c(bias, np.float32)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2 and (bias is None or bias.shape == (N,))
    y = np.empty((M, N), np.float32)
    y64 = np.empty((M, N), np.float64) if want_f64 else None
    rc = _load().oracle_linear_f32(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(y64), M, N, K)
    if rc:
        raise ValueError("oracle_linear_f32 rejected its arguments")
    return (y, y64) if want_f64 else y


def linear_bf16(x, w, bias=None, out="bf16", want_f64=False):
    """Same definition with bf16 operands (uint16 bit patterns).

    ``out`` is "bf16" (uint16 result) or "f32" (float32 result)."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    bias = _c(bias, np.float32)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2 and (bias is None or bias.shape == (N,))
    yb = np.empty((M, N), np.uint16) if out == "bf16" else None
    yf = np.empty((M, N), np.float32) if out == "f32" else None
    if yb is None and yf is None:
        raise ValueError("out must be 'bf16' or 'f32'")
    y64 = np.empty((M, N), np.float64) if want_f64 else None
    rc = _load().oracle_linear_bf16(_ptr(x), _ptr(w), _ptr(bias), _ptr(yb), _ptr(yf),
                                    _ptr(y64), M, N, K)
    if rc:
        raise ValueError("oracle_linear_bf16 rejected its arguments")
    y = yb if yb is not None else yf
    return (y, y64) if want_f64 else y


def topk(scores, k):
    """Per-row top-k ids: descending score, ties to the lower index, +-0 equal."""
    s = _c(scores, np.float32)
    M, E = s.shape
    ids = np.empty((M, k), np.int32)
    if _load().oracle_topk(_ptr(s), _ptr(ids), M, E, k):
        raise ValueError("oracle_topk rejected its arguments (NaN score or bad k)")
    return ids


def topk_rows(scores, topk, row_start=None, row_end=None):
    """Indexer top-k per row (Sparse-MLA page, deterministic top-k notes).

    ``scores`` is float32 [rows, cols] (any fp32 bit pattern); ``row_start`` /
    ``row_end`` are int64 [rows] window bounds (clamped to [0, cols]; None means
    0 / cols).  Returns int32 [rows, topk]: the selected row-local column
    indices in ascending order, then -1."""
    s = _c(scores, np.float32)
    rows, cols = s.shape
    rs = _c(row_start, np.int64)
    re = _c(row_end, np.int64)
    assert rs is None or rs.shape == (rows,)
    assert re is None or re.shape == (rows,)
    out = np.empty((rows, topk), np.int32)
    if _load().oracle_topk_rows(_ptr(s), cols, rows, cols, _ptr(rs), _ptr(re), topk, _ptr(out), topk):
        raise ValueError("oracle_topk_rows rejected its arguments")
    return out


def moe(x, w_router, b_router, w13, w2, topk, ids=None):
    """Batch-invariant MoE layer, binary64 with the method's storage points.

    Returns (y [M,H] f32, ids [M,topk] i32, probs [M,topk] f64, logits [M,E] f32).
    ``ids`` forces the expert choice instead of selecting it."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    b_router = _c(b_router, np.float32)
    w13 = _c(w13, np.uint16)
    w2 = _c(w2, np.uint16)
    M, H = x.shape
    E, H2 = w_router.shape
    E2, I2, H3 = w13.shape
    E3, H4, I = w2.shape
    assert H == H2 == H3 == H4 and E == E2 == E3 and I2 == 2 * I
    ids_in = _c(ids, np.int32)
    if ids_in is not None:
        assert ids_in.shape == (M, topk)
    y = np.empty((M, H), np.float32)
    ids_out = np.empty((M, topk), np.int32)
    probs = np.empty((M, topk), np.float64)
    logits = np.empty((M, E), np.float32)
    rc = _load().oracle_moe(_ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w13), _ptr(w2),
                            M, H, E, I, topk, _ptr(ids_in), _ptr(logits), _ptr(ids_out),
                            _ptr(probs), _ptr(y))
    if rc:
        raise ValueError("oracle_moe rejected its arguments")
    return y, ids_out, probs, logits


ACT_SWIGLU, ACT_SQRELU = 1, 2


def moe_ex(x, w_router, b_router, w1, w2, topk, act=ACT_SWIGLU, probs_at_act=True, apply_weights=False,
           acc_fp64=True, ids=None):
    """MoE layer with the activation and combine options: act ACT_SWIGLU (w1
    [E, 2I, H], gate rows first) or ACT_SQRELU (w1 [E, I, H]); the routing
    probability applied at the activation and/or as a weight in the top-k
    sum; the sum in binary64 or in fp32.  Same returns as moe()."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    b_router = _c(b_router, np.float32)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    M, H = x.shape
    E, H2 = w_router.shape
    E2, R1, H3 = w1.shape
    E3, H4, I = w2.shape
    assert H == H2 == H3 == H4 and E == E2 == E3 and R1 == (2 * I if act == ACT_SWIGLU else I)
    ids_in = _c(ids, np.int32)
    if ids_in is not None:
        assert ids_in.shape == (M, topk)
    y = np.empty((M, H), np.float32)
    ids_out = np.empty((M, topk), np.int32)
    probs = np.empty((M, topk), np.float64)
    logits = np.empty((M, E), np.float32)
    rc = _load().oracle_moe_ex(_ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w1), _ptr(w2),
                               M, H, E, I, topk, int(act), int(bool(probs_at_act)), int(bool(apply_weights)),
                               int(bool(acc_fp64)), _ptr(ids_in), _ptr(logits), _ptr(ids_out),
                               _ptr(probs), _ptr(y))
    if rc:
        raise ValueError("oracle_moe_ex rejected its arguments")
    return y, ids_out, probs, logits


def moe_stages(x, w_router, b_router, w1, w2, topk, act=ACT_SWIGLU, probs_at_act=True, apply_weights=False,
               acc_fp64=True, ids=None):
    """moe_ex() plus the layer's storage points per (token, slot) pair:
    returns (y, ids, probs, logits, h, a, part) with h uint16 [M, topk,
    rows of w1[e]] (first projection, bf16), a uint16 [M, topk, I]
    (activation, bf16) and part float64 [M, topk, H] (down projection of
    the slot, before any weight)."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    b_router = _c(b_router, np.float32)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    M, H = x.shape
    E, H2 = w_router.shape
    E2, R1, H3 = w1.shape
    E3, H4, I = w2.shape
    assert H == H2 == H3 == H4 and E == E2 == E3 and R1 == (2 * I if act == ACT_SWIGLU else I)
    ids_in = _c(ids, np.int32)
    if ids_in is not None:
        assert ids_in.shape == (M, topk)
    y = np.empty((M, H), np.float32)
    ids_out = np.empty((M, topk), np.int32)
    probs = np.empty((M, topk), np.float64)
    logits = np.empty((M, E), np.float32)
    h = np.empty((M, topk, R1), np.uint16)
    a = np.empty((M, topk, I), np.uint16)
    part = np.empty((M, topk, H), np.float64)
    rc = _load().oracle_moe_stages(_ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w1), _ptr(w2),
                                   M, H, E, I, topk, int(act), int(bool(probs_at_act)), int(bool(apply_weights)),
                                   int(bool(acc_fp64)), _ptr(ids_in), _ptr(logits), _ptr(ids_out),
                                   _ptr(probs), _ptr(y), _ptr(h), _ptr(a), _ptr(part))
    if rc:
        raise ValueError("oracle_moe_stages rejected its arguments")
    return y, ids_out, probs, logits, h, a, part


def moe_activation(h, p, act=ACT_SWIGLU, probs_at_act=True):
    """The MoE layer's activation step alone: h uint16 [P, 2I] (SwiGLU, gate
    half first) or [P, I] (squared-ReLU) bf16 first-projection outputs, p
    float64 [P]; returns a uint16 [P, I] = RN_bf16(act(h) * (p or 1))."""
    h = _c(h, np.uint16)
    p = _c(np.asarray(p, np.float64), np.float64)
    P, R = h.shape
    I = R // 2 if act == ACT_SWIGLU else R
    assert p.shape == (P,)
    a = np.empty((P, I), np.uint16)
    if _load().oracle_moe_activation(_ptr(h), _ptr(p), P, I, int(act), int(bool(probs_at_act)), _ptr(a)):
        raise ValueError("oracle_moe_activation rejected its arguments")
    return a


def moe_combine(part, p, apply_weights=False, acc_fp64=True):
    """The MoE layer's top-k sum alone: part float64 [M, topk, H] slot values,
    p float64 [M, topk]; returns float32 [M, H]."""
    part = _c(np.asarray(part, np.float64), np.float64)
    p = _c(np.asarray(p, np.float64), np.float64)
    M, k, H = part.shape
    assert p.shape == (M, k)
    y = np.empty((M, H), np.float32)
    if _load().oracle_moe_combine(_ptr(part), _ptr(p), M, k, H, int(bool(apply_weights)), int(bool(acc_fp64)),
                                  _ptr(y)):
        raise ValueError("oracle_moe_combine rejected its arguments")
    return y


def f64_to_bf16(v):
    """Round binary64 values to bf16 bit patterns (one RNE step)."""
    v = _c(np.asarray(v, np.float64), np.float64)
    out = np.empty(v.shape, np.uint16)
    if _load().oracle_f64_to_bf16(_ptr(v), _ptr(out), v.size):
        raise ValueError("bad arguments")
    return out
