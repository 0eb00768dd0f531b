"""Helpers for the GPU tests: device transfer, tolerance checks, case banners."""
import sys

import numpy as np

F32_ATOL, F32_RTOL = 2e-3, 1e-4     # GateLinear page, "Tests"


def banner(msg: str):
    """Name the case on the real stderr before a GPU step, so a fault that
    ends the process still tells which case was running."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def dev(a: np.ndarray, dtype=None):
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def weight_t(w_dev):
    """The production layout: nn.Linear weight [N, K] handed over as its .t() view."""
    wt = w_dev.t()
    assert wt.stride(0) == 1
    return wt


def assert_close(got, want, atol, rtol, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements outside atol={atol} rtol={rtol}; "
                             f"first {idx.tolist()}: got {got[tuple(idx.T)]}, want {want[tuple(idx.T)]}")
    return float(err.max()) if err.size else 0.0


def assert_bitwise(a, b, what=""):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ua = a.view(np.uint32 if a.dtype == np.float32 else np.uint16)
    ub = b.view(np.uint32 if b.dtype == np.float32 else np.uint16)
    diff = np.argwhere(ua != ub)
    if diff.size:
        raise AssertionError(f"{what}: {len(diff)} elements differ bitwise, first at {diff[:5].tolist()}")


def bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
