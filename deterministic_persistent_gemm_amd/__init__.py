"""Batch-invariant GEMM for MI355X (gfx950): thin Python binding of libbi.so.

Every computation runs in the HIP kernels behind the C ABI declared in
``include/bi.h``; this module only checks tensor metadata, allocates outputs
and workspaces with PyTorch, and passes raw device pointers plus the current
HIP stream.  The library must be built (``python -m
deterministic_persistent_gemm_amd._build``); importing without it raises.

Weights are taken in the production ``weight.t()`` layout: ``wt`` is the
[K, N] transposed view of an nn.Linear weight [N, K], i.e. ``wt.stride(0) ==
1``.  The names match the C entry points.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbi.so")

BI_OK, BI_EINVAL, BI_EUNSUPPORTED, BI_EWORKSPACE, BI_EHIP = range(5)
BI_F32, BI_BF16 = 0, 1
BI_PATH_AUTO, BI_PATH_DECODE, BI_PATH_PERSISTENT, BI_PATH_DECODE_WG, BI_PATH_DECODE_DMA, BI_PATH_DECODE_XCD = (
    0, 1, 2, 3, 4, 5)
# bytes at the start of every workspace that hold the one-launch decode's
# arrival counters (zero at first use; every call leaves them zero)
WS_COUNTER_BYTES = 16384
BI_R2_TILE_PARTIAL = 2
BI_MFMA_F32_16X16X4_F32, BI_MFMA_F32_16X16X32_BF16 = 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m deterministic_persistent_gemm_amd._build`")

_lib = ctypes.CDLL(LIB_PATH)


class Recipe(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dtype", "mfma", "k_group", "reduce", "block_k", "bias_last", "m_decode_max", "reserved")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_lib.bi_linear_f32.argtypes = [_P, _I64, _P, _I64, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]
_lib.bi_linear_bf16.argtypes = [_P, _I64, _P, _I64, _P, _P, _I32, _I64, _I64, _I64, _I64, _P, _SZ, _P]
_lib.bi_negctl_linear_f32.argtypes = _lib.bi_linear_f32.argtypes
_lib.bi_lab_linear.argtypes = [_P, _I64, _P, _I64, _P, _P, _I32, _I64, _I64, _I64, _I64,
                               ctypes.POINTER(Recipe), _I32, _P, _SZ, _P]
_lib.bi_moe_grouped_gemm.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                     _P, _SZ, _P]
_lib.bi_linear_workspace_size.argtypes = [_I32, _I64, _I64, _I64]
_lib.bi_lab_workspace_size.argtypes = [ctypes.POINTER(Recipe), _I32, _I64, _I64, _I64]
_lib.bi_moe_workspace_size.argtypes = [_I64, _I64, _I64, _I64, _I64]
_lib.bi_describe_recipe.argtypes = [_I32, _I64, _I64, ctypes.POINTER(Recipe)]
_lib.bi_status_str.argtypes = [_I32]
_lib.bi_indexer_topk.argtypes = [_P, _I64, _I64, _I64, _P, _P, _I64, _P, _I64, _P]
_lib.bi_moe_grouped_gemm_ex.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                        _P, _SZ, _P]
_lib.bi_lab_xcc_ids.argtypes = [_P, _I32, _I32, _P]
_lib.bi_lab_empty.argtypes = [_I32, _I32, _P]
_lib.bi_lab_stream_read.argtypes = [_P, _I64, _P, _I32, _P]
_lib.bi_lab_l2_read.argtypes = [_P, _I64, _I32, _P, _I32, _P]
_lib.bi_lab_clock.argtypes = [_P, _I32, _I32, _P]
_lib.bi_lab_lds_read.argtypes = [_P, _I32, _I32, _P]
_lib.bi_lab_mfma_rate.argtypes = [_P, _I32, _I32, _I32, _I32, _P]
_lib.bi_lab_plan.argtypes = [_I32, _I64, _I64, _I64, ctypes.POINTER(_I32)]
_lib.bi_lab_moe_layout.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.POINTER(_I64)]
_lib.bi_linear_f32_noalloc.argtypes = [_P, _I64, _P, _I64, _P, _P, _I64, _I64, _I64, _I64, _P]
for _f in (_lib.bi_linear_f32, _lib.bi_linear_bf16, _lib.bi_negctl_linear_f32, _lib.bi_lab_linear,
           _lib.bi_moe_grouped_gemm, _lib.bi_describe_recipe, _lib.bi_indexer_topk,
           _lib.bi_moe_grouped_gemm_ex, _lib.bi_lab_xcc_ids, _lib.bi_lab_empty, _lib.bi_lab_stream_read,
           _lib.bi_lab_clock, _lib.bi_lab_plan, _lib.bi_lab_moe_layout, _lib.bi_linear_f32_noalloc,
           _lib.bi_lab_lds_read, _lib.bi_lab_mfma_rate, _lib.bi_lab_l2_read):
    _f.restype = _I32
for _f in (_lib.bi_linear_workspace_size, _lib.bi_lab_workspace_size, _lib.bi_moe_workspace_size):
    _f.restype = _SZ
_lib.bi_status_str.restype = ctypes.c_char_p


class BIError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.bi_status_str(status).decode()}")


def _check(status: int, where: str):
    if status != BI_OK:
        raise BIError(status, where)


# ------------------------------------------------------------------ workspace

_ws_lock = threading.Lock()
_ws_cache: dict = {}
# Workspaces replaced by larger ones.  They are never freed: a HIP graph
# captured while one of them was current keeps its address and writes there on
# every replay, so releasing it to the caching allocator could hand that memory
# to another tensor.
_ws_retired: list = []


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace of at least `nbytes` bytes (the first
    WS_COUNTER_BYTES hold counters that must be zero at first use)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _workspace(nbytes: int, device: torch.device, stream: torch.cuda.Stream,
               given: torch.Tensor | None = None) -> torch.Tensor | None:
    """The caller's workspace if one is given (checked), else a grow-only
    workspace cached per (device, stream).  Growing it inside a graph capture
    is refused: run the call once eagerly at the largest shape first, or pass
    `ws=` explicitly."""
    if given is not None:
        if given.dtype != torch.uint8 or given.dim() != 1 or not given.is_contiguous() or given.device != device:
            raise ValueError(f"ws must be a contiguous 1-D uint8 tensor on {device}")
        if given.numel() < nbytes:
            raise ValueError(f"ws holds {given.numel()} bytes; this call needs {nbytes}")
        return given
    if nbytes == 0:
        return None
    key = (device.index, stream.cuda_stream)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            if torch.cuda.is_current_stream_capturing():
                raise RuntimeError("the cached workspace must grow during a graph capture; call once eagerly "
                                   "at the largest shape before capturing, or pass ws=")
            if ws is not None:
                _ws_retired.append(ws)
            ws = alloc_workspace(max(nbytes, 1 << 20, 0 if ws is None else 2 * ws.numel()), device)
            _ws_cache[key] = ws
        return ws


def _stream(device) -> torch.cuda.Stream:
    return torch.cuda.current_stream(device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_xw(x: torch.Tensor, wt: torch.Tensor, dtype: torch.dtype, name: str):
    if x.dtype != dtype or wt.dtype != dtype:
        raise TypeError(f"{name}: x and wt must be {dtype}, got {x.dtype} and {wt.dtype}")
    if not (x.is_cuda and wt.is_cuda and x.device == wt.device):
        raise ValueError(f"{name}: x and wt must be on the same GPU")
    if x.dim() != 2 or wt.dim() != 2:
        raise ValueError(f"{name}: x is [M, K] and wt is [K, N]")
    if x.shape[1] != wt.shape[0]:
        raise ValueError(f"{name}: K mismatch {tuple(x.shape)} x {tuple(wt.shape)}")
    if x.stride(1) != 1:
        raise ValueError(f"{name}: x rows must be contiguous")
    if wt.stride(0) != 1:
        raise ValueError(f"{name}: wt must be the weight.t() view of an [N, K] weight (wt.stride(0) == 1)")


def _check_out(out, shape, dtypes, device, name):
    """A caller-supplied output: on the inputs' GPU, of the call's shape and
    dtype, unit column stride and a row pitch of at least its width."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != device:
        raise ValueError(f"{name}: out must be a tensor on {device}")
    if out.dtype not in dtypes:
        raise TypeError(f"{name}: out must be one of {dtypes}, got {out.dtype}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name}: out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.dim() != 2 or out.stride(1) != 1 or (shape[0] > 1 and out.stride(0) < shape[1]):
        raise ValueError(f"{name}: out must have unit column stride and a row pitch >= {shape[1]}")


def _check_bias(bias, N, device, name):
    if bias is None:
        return
    if bias.dtype != torch.float32 or bias.shape != (N,) or not bias.is_contiguous() or bias.device != device:
        raise ValueError(f"{name}: bias must be a contiguous fp32 [{N}] tensor on {device}")


# ---------------------------------------------------------------- entry points


def bi_linear_f32(x: torch.Tensor, wt: torch.Tensor, bias: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """y = x @ wt + bias in fp32, batch-invariant.  x [M, K], wt = weight.t() [K, N].
    ws: optional caller-owned workspace (alloc_workspace), else a cached one."""
    _check_xw(x, wt, torch.float32, "bi_linear_f32")
    M, K = x.shape
    N = wt.shape[1]
    _check_bias(bias, N, x.device, "bi_linear_f32")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_out(out, (M, N), (torch.float32,), x.device, "bi_linear_f32")
    s = _stream(x.device)
    nbytes = _lib.bi_linear_workspace_size(BI_F32, M, N, K)
    ws = _workspace(nbytes, x.device, s, ws)
    _check(_lib.bi_linear_f32(_ptr(x), x.stride(0), _ptr(wt), wt.stride(1), _ptr(bias), _ptr(out),
                              out.stride(0), M, N, K, _ptr(ws), 0 if ws is None else ws.numel(),
                              ctypes.c_void_p(s.cuda_stream)), "bi_linear_f32")
    return out


def bi_linear_f32_noalloc(x: torch.Tensor, wt: torch.Tensor, bias: torch.Tensor | None, out: torch.Tensor
                          ) -> torch.Tensor:
    """bi_linear_f32 into a caller-given `out`, with the library's static
    scratch instead of a workspace: nothing is allocated (calls that overlap
    on one GPU race on that scratch)."""
    _check_xw(x, wt, torch.float32, "bi_linear_f32_noalloc")
    M, K = x.shape
    N = wt.shape[1]
    _check_bias(bias, N, x.device, "bi_linear_f32_noalloc")
    _check_out(out, (M, N), (torch.float32,), x.device, "bi_linear_f32_noalloc")
    s = _stream(x.device)
    _check(_lib.bi_linear_f32_noalloc(_ptr(x), x.stride(0), _ptr(wt), wt.stride(1), _ptr(bias), _ptr(out),
                                      out.stride(0), M, N, K, ctypes.c_void_p(s.cuda_stream)),
           "bi_linear_f32_noalloc")
    return out


def bi_linear_bf16(x: torch.Tensor, wt: torch.Tensor, bias: torch.Tensor | None = None,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None) -> torch.Tensor:
    """y = x @ wt + bias with bf16 operands, fp32 accumulation, bf16 or fp32 out."""
    _check_xw(x, wt, torch.bfloat16, "bi_linear_bf16")
    M, K = x.shape
    N = wt.shape[1]
    _check_bias(bias, N, x.device, "bi_linear_bf16")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _check_out(out, (M, N), (torch.bfloat16, torch.float32), x.device, "bi_linear_bf16")
    s = _stream(x.device)
    nbytes = _lib.bi_linear_workspace_size(BI_BF16, M, N, K)
    ws = _workspace(nbytes, x.device, s, ws)
    _check(_lib.bi_linear_bf16(_ptr(x), x.stride(0), _ptr(wt), wt.stride(1), _ptr(bias), _ptr(out),
                               BI_BF16 if out.dtype == torch.bfloat16 else BI_F32, out.stride(0), M, N, K,
                               _ptr(ws), 0 if ws is None else ws.numel(), ctypes.c_void_p(s.cuda_stream)),
           "bi_linear_bf16")
    return out


def bi_negctl_linear_f32(x, wt, bias=None, out=None):
    """Negative control: same call with an M-dependent BLOCK_K (expected to break invariance)."""
    _check_xw(x, wt, torch.float32, "bi_negctl_linear_f32")
    M, K = x.shape
    N = wt.shape[1]
    _check_bias(bias, N, x.device, "bi_negctl_linear_f32")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_out(out, (M, N), (torch.float32,), x.device, "bi_negctl_linear_f32")
    s = _stream(x.device)
    ws = _workspace(_lib.bi_linear_workspace_size(BI_F32, M, N, K), x.device, s)
    _check(_lib.bi_negctl_linear_f32(_ptr(x), x.stride(0), _ptr(wt), wt.stride(1), _ptr(bias), _ptr(out),
                                     out.stride(0), M, N, K, _ptr(ws), 0 if ws is None else ws.numel(),
                                     ctypes.c_void_p(s.cuda_stream)), "bi_negctl_linear_f32")
    return out


def bi_describe_recipe(dtype: int, N: int, K: int) -> Recipe:
    r = Recipe()
    _check(_lib.bi_describe_recipe(dtype, N, K, ctypes.byref(r)), "bi_describe_recipe")
    return r


def bi_lab_linear(x, wt, bias=None, recipe: Recipe | None = None, path: int = BI_PATH_AUTO,
                  out_dtype=None, out=None):
    """Linear layer with an explicit recipe and kernel path (experiments only)."""
    dt = torch.float32 if x.dtype == torch.float32 else torch.bfloat16
    _check_xw(x, wt, dt, "bi_lab_linear")
    M, K = x.shape
    N = wt.shape[1]
    _check_bias(bias, N, x.device, "bi_lab_linear")
    if recipe is None:
        recipe = bi_describe_recipe(BI_F32 if dt == torch.float32 else BI_BF16, N, K)
    out_dtype = out_dtype or (torch.float32 if dt == torch.float32 else torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _check_out(out, (M, N), (torch.float32, torch.bfloat16), x.device, "bi_lab_linear")
    s = _stream(x.device)
    ws = _workspace(_lib.bi_lab_workspace_size(ctypes.byref(recipe), path, M, N, K), x.device, s)
    _check(_lib.bi_lab_linear(_ptr(x), x.stride(0), _ptr(wt), wt.stride(1), _ptr(bias), _ptr(out),
                              BI_BF16 if out.dtype == torch.bfloat16 else BI_F32, out.stride(0), M, N, K,
                              ctypes.byref(recipe), path, _ptr(ws), 0 if ws is None else ws.numel(),
                              ctypes.c_void_p(s.cuda_stream)), "bi_lab_linear")
    return out


class MoEOptions(ctypes.Structure):
    """bi_moe_options_t."""
    _fields_ = [("activation", ctypes.c_int32), ("probs_at_activation", ctypes.c_int32),
                ("apply_weights", ctypes.c_int32), ("acc_fp64", ctypes.c_int32)]


BI_ACT_SWIGLU, BI_ACT_SQRELU = 0, 1


def bi_moe_grouped_gemm(x, w_router, b_router, w13, w2, topk: int, ws=None):
    """Batch-invariant MoE layer.  Returns (y fp32 [M,H], topk_ids int32 [M,topk],
    topk_probs fp32 [M,topk]).  w13 [E, 2I, H] and w2 [E, H, I] are the experts'
    nn.Linear weights (their .t() views are what the GEMMs consume)."""
    return _moe(x, w_router, b_router, w13, w2, topk, None, "bi_moe_grouped_gemm", ws)


def bi_moe_grouped_gemm_ex(x, w_router, b_router, w1, w2, topk: int, activation: int = BI_ACT_SWIGLU,
                           probs_at_activation: bool = True, apply_weights: bool = False,
                           acc_fp64: bool = True, ws=None):
    """The MoE layer with explicit activation and top-k-sum options.  SwiGLU:
    w1 [E, 2I, H]; squared-ReLU: w1 [E, I, H].  Same returns."""
    opt = MoEOptions(int(activation), int(bool(probs_at_activation)), int(bool(apply_weights)),
                     int(bool(acc_fp64)))
    return _moe(x, w_router, b_router, w1, w2, topk, opt, "bi_moe_grouped_gemm_ex", ws)


def _moe(x, w_router, b_router, w1, w2, topk, opt, name, ws_given=None):
    if x.dtype != torch.bfloat16 or w1.dtype != torch.bfloat16 or w2.dtype != torch.bfloat16:
        raise TypeError(f"{name}: x, w1, w2 must be bfloat16")
    if w_router.dtype != torch.float32:
        raise TypeError(f"{name}: w_router must be float32")
    for t in (x, w_router, w1, w2) + (() if b_router is None else (b_router,)):
        if not t.is_contiguous() or not t.is_cuda or t.device != x.device:
            raise ValueError(f"{name}: tensors must be contiguous and on the same GPU")
    M, H = x.shape
    E = w_router.shape[0]
    I = w2.shape[2]
    rows1 = I if (opt is not None and opt.activation == BI_ACT_SQRELU) else 2 * I
    if w_router.shape != (E, H) or w1.shape != (E, rows1, H) or w2.shape != (E, H, I):
        raise ValueError(f"{name}: inconsistent shapes")
    _check_bias(b_router, E, x.device, name)
    y = torch.empty((M, H), dtype=torch.float32, device=x.device)
    ids = torch.empty((M, topk), dtype=torch.int32, device=x.device)
    probs = torch.empty((M, topk), dtype=torch.float32, device=x.device)
    s = _stream(x.device)
    ws = _workspace(_lib.bi_moe_workspace_size(M, H, E, I, topk), x.device, s, ws_given)
    common = (_ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w1), _ptr(w2), M, H, E, I, topk)
    tail = (_ptr(ids), _ptr(probs), _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
            ctypes.c_void_p(s.cuda_stream))
    if opt is None:
        _check(_lib.bi_moe_grouped_gemm(*common, *tail), name)
    else:
        _check(_lib.bi_moe_grouped_gemm_ex(*common, ctypes.byref(opt), *tail), name)
    return y, ids, probs


def bi_indexer_topk(scores, topk: int, row_start=None, row_end=None, out=None):
    """Deterministic per-row top-k of fp32 indexer scores [rows, cols] (row pitch
    may exceed cols).  row_start / row_end: int64 [rows] window bounds or None.
    Returns int32 [rows, topk]: ascending window-relative indices, then -1."""
    if scores.dtype != torch.float32 or scores.dim() != 2 or not scores.is_cuda or scores.stride(1) != 1:
        raise ValueError("bi_indexer_topk: scores must be a 2-D float32 CUDA tensor with unit column stride")
    rows, cols = scores.shape
    for name, t in (("row_start", row_start), ("row_end", row_end)):
        if t is not None and (t.dtype != torch.int64 or t.shape != (rows,) or not t.is_contiguous()
                              or t.device != scores.device):
            raise ValueError(f"bi_indexer_topk: {name} must be a contiguous int64 [rows] tensor on the same GPU")
    if out is None:
        out = torch.empty((rows, topk), dtype=torch.int32, device=scores.device)
    _check_out(out, (rows, topk), (torch.int32,), scores.device, "bi_indexer_topk")
    s = _stream(scores.device)
    _check(_lib.bi_indexer_topk(_ptr(scores), max(scores.stride(0), cols), rows, cols, _ptr(row_start),
                                _ptr(row_end), topk, _ptr(out), out.stride(0),
                                ctypes.c_void_p(s.cuda_stream)), "bi_indexer_topk")
    return out


def bi_lab_xcc_ids(grid_x: int, grid_y: int = 1, device=None) -> torch.Tensor:
    """XCD id each workgroup of a grid_x x grid_y grid ran on (int64 [grid_y, grid_x])."""
    device = torch.device(device or "cuda")
    out = torch.empty((grid_y, grid_x), dtype=torch.int32, device=device)
    s = _stream(device)
    _check(_lib.bi_lab_xcc_ids(_ptr(out), grid_x, grid_y, ctypes.c_void_p(s.cuda_stream)), "bi_lab_xcc_ids")
    return out.long() & 0xffffffff


def plan_path(dtype: int, M: int, N: int, K: int) -> int:
    """The kernel path (BI_PATH_*) the production entry points pick for M rows."""
    p = ctypes.c_int32(-1)
    _check(_lib.bi_lab_plan(dtype, M, N, K, ctypes.byref(p)), "bi_lab_plan")
    return p.value


def moe_layout(M: int, H: int, E: int, I: int, topk: int) -> dict:
    """Byte offsets of the MoE workspace's sorted pair list, activations and
    slot partials, and its size (bi_lab_moe_layout)."""
    out = (_I64 * 4)()
    _check(_lib.bi_lab_moe_layout(M, H, E, I, topk, out), "bi_lab_moe_layout")
    return {"sorted": out[0], "act": out[1], "part": out[2], "total": out[3]}


def bi_lab_empty(grid: int, threads: int = 64):
    """Enqueue an empty kernel of `grid` workgroups (the per-launch floor)."""
    s = _stream(torch.device("cuda", torch.cuda.current_device()))
    _check(_lib.bi_lab_empty(grid, threads, ctypes.c_void_p(s.cuda_stream)), "bi_lab_empty")


def bi_lab_stream_read(src: torch.Tensor, sink: torch.Tensor, grid: int):
    """Read every byte of `src` once on the GPU (cold-read rate); sink: int32 [>= grid]."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= grid and src.device == sink.device):
        raise ValueError("bi_lab_stream_read: contiguous CUDA src and an int32 sink of >= grid entries")
    s = _stream(src.device)
    _check(_lib.bi_lab_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), grid,
                                   ctypes.c_void_p(s.cuda_stream)), "bi_lab_stream_read")


def bi_lab_l2_read(src: torch.Tensor, sink: torch.Tensor, grid: int, iters: int):
    """Every one of `grid` workgroups reads all of `src` (32 KiB .. 2 MiB, a
    power of two: L2-resident after the first pass) `iters` times (L2-to-CU
    delivery rate); sink: int32 [>= grid]."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= grid and src.device == sink.device):
        raise ValueError("bi_lab_l2_read: contiguous CUDA src and an int32 sink of >= grid entries")
    s = _stream(src.device)
    _check(_lib.bi_lab_l2_read(_ptr(src), src.numel() * src.element_size(), iters, _ptr(sink), grid,
                               ctypes.c_void_p(s.cuda_stream)), "bi_lab_l2_read")


def bi_lab_clock(out: torch.Tensor, grid: int, iters: int):
    """Shader-clock probe: out int64 [grid, 3] gets (cycles, wall ticks, keep-alive) per workgroup."""
    if not (out.is_cuda and out.dtype == torch.int64 and out.is_contiguous() and out.numel() >= 3 * grid):
        raise ValueError("bi_lab_clock: out must be a contiguous int64 CUDA tensor of >= 3 * grid entries")
    s = _stream(out.device)
    _check(_lib.bi_lab_clock(_ptr(out), grid, iters, ctypes.c_void_p(s.cuda_stream)), "bi_lab_clock")


def _check_probe_out(out: torch.Tensor, grid: int, where: str):
    if not (out.is_cuda and out.dtype == torch.int64 and out.is_contiguous() and out.numel() >= 3 * grid):
        raise ValueError(f"{where}: out must be a contiguous int64 CUDA tensor of >= 3 * grid entries")


def bi_lab_lds_read(out: torch.Tensor, grid: int, iters: int):
    """LDS read-rate probe: out int64 [grid, 3] gets (cycles, wall ticks, keep-alive) per workgroup."""
    _check_probe_out(out, grid, "bi_lab_lds_read")
    s = _stream(out.device)
    _check(_lib.bi_lab_lds_read(_ptr(out), grid, iters, ctypes.c_void_p(s.cuda_stream)), "bi_lab_lds_read")


def bi_lab_mfma_rate(out: torch.Tensor, dtype: int, grid: int, iters: int, chains: int = 8):
    """MFMA issue-rate probe (BI_F32: 16x16x4 f32, BI_BF16: 16x16x32 bf16) over `chains`
    independent accumulators per wave: out int64 [grid, 3]."""
    _check_probe_out(out, grid, "bi_lab_mfma_rate")
    s = _stream(out.device)
    _check(_lib.bi_lab_mfma_rate(_ptr(out), dtype, chains, grid, iters, ctypes.c_void_p(s.cuda_stream)),
           "bi_lab_mfma_rate")


def lib():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib
