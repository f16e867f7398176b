"""Helpers for the GPU tests: move seeded inputs to the device, build the oracle problem from the
same bytes, sample channels of large problems for the oracle."""
import numpy as np
import torch

import oracle


def dev_pre(inp, device="cuda"):
    """Pre-activation planes as device tensors (bf16 bits are reinterpreted, not re-rounded)."""
    out = []
    for p in inp.pre:
        if inp.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(p).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(p))
        out.append(t.to(device))
    return out


def dev(x, device="cuda"):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)


def oracle_problem(inp, s0=None, channels=None, cu_seqlens=None):
    """Oracle problem over all channels, or over a list of (b, d) channels (as B=1, D=len)."""
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.F32
    if channels is None:
        return oracle.Problem(inp.cell, inp.pre, inp.w, inp.bias, s0=s0, dtype=dt, cu_seqlens=cu_seqlens)
    bs = np.array([c[0] for c in channels])
    ds = np.array([c[1] for c in channels])
    pre = [np.ascontiguousarray(p[bs, :, ds].T[None]) for p in inp.pre]   # [1, T, n]
    w = None if inp.w is None else np.ascontiguousarray(inp.w[:, ds])
    bias = None if inp.bias is None else np.ascontiguousarray(inp.bias[:, ds])
    s0s = None if s0 is None else np.ascontiguousarray(s0[:, bs, ds][:, None, :])
    return oracle.Problem(inp.cell, pre, w, bias, s0=s0s, dtype=dt, cu_seqlens=cu_seqlens)


def take_channels(x, channels):
    """x [..., B, T, D] -> [..., 1, T, n] for the listed (b, d) channels."""
    bs = np.array([c[0] for c in channels])
    ds = np.array([c[1] for c in channels])
    y = x[..., bs, :, ds]                 # [n, ..., T] by numpy advanced-index rules
    y = np.moveaxis(y, 0, -1)             # [..., T, n]
    return np.ascontiguousarray(y[..., None, :, :])


def sample_channels(B, D, n, seed):
    rng = np.random.default_rng(seed)
    idx = set()
    # always include both edges of the channel range and of each tile boundary region
    for c in [(0, 0), (0, 1), (B - 1, D - 1), (B - 1, D - 2)]:
        idx.add(c)
    while len(idx) < n:
        idx.add((int(rng.integers(B)), int(rng.integers(D))))
    return sorted(idx)


def lane_channels(B, D, n_extra, seed):
    """Sampled channels that hold every lane position of a tile: 64 consecutive channels of one batch row,
    starting at a multiple of 64 (the kernels' tiles are 32 or 64 channels wide and start at multiples of
    their width), plus the edges and n_extra random channels."""
    rng = np.random.default_rng(seed)
    b0 = int(rng.integers(B))
    d0 = 64 * int(rng.integers(max(1, D // 64)))
    idx = {(b0, d) for d in range(d0, min(d0 + 64, D))}
    return sorted(idx | set(sample_channels(B, D, n_extra, seed)))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
