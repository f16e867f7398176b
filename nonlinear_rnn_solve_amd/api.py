"""Thin Python binding over libpararnn.so (C ABI in include/pararnn.h).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback -- if the library or a GPU is missing, calls raise.

Method references (pararnn-torch README on PyPI, "Method"; ParaRNN abstract):
Newton on F(H)_t = h_t - f(h_{t-1}, x_t) = 0 with scan-based linear solves, and
the adjoint (reverse scan) for gradients.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpararnn.so")

CELLS = {"linear": 0, "gru": 1, "lstm": 2, "slstm": 3, "head_gru": 4}
GATES = {0: 2, 1: 3, 2: 4, 3: 4, 4: 3}
STATE = {0: 1, 1: 1, 2: 2, 3: 4, 4: 1}
HEAD_GRU = 4
MAX_ITERS = 64
MAX_FUSE = 8          # PARARNN_MAX_FUSE
ABI_VERSION = 6
INIT_ZERO, INIT_WARM = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration", -3: "workspace", -4: "HIP error",
          -5: "Newton diverged"}


class PararnnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, STATUS.get(status, "?"), status))
        self.status = status


class NewtonDivergenceError(PararnnError):
    """Raised when a tolerance-mode solve sees a non-finite max residual, or spends its budget without
    converging and ends above the residual Newton started from; carries the history."""

    def __init__(self, status, what, report):
        super().__init__(status, what)
        self.report = report


class _Problem(ctypes.Structure):
    _fields_ = [("cell", ctypes.c_int32), ("pre_dtype", ctypes.c_int32),
                ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
                ("pre", ctypes.c_void_p * 4), ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("s0", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int64),
                ("head_size", ctypes.c_int64)]


class _Opts(ctypes.Structure):
    _fields_ = [("max_iters", ctypes.c_int32), ("tol", ctypes.c_float), ("init_guess", ctypes.c_void_p),
                ("final_residual", ctypes.c_int32), ("init_mode", ctypes.c_int32), ("picard_iters", ctypes.c_int32),
                ("fuse_iters", ctypes.c_int32)]


class _Report(ctypes.Structure):
    _fields_ = [("iters", ctypes.c_int32), ("converged", ctypes.c_int32), ("n_residual", ctypes.c_int32),
                ("residual", ctypes.c_float * (MAX_ITERS + 1))]


@dataclass
class NewtonReport:
    iters: int
    converged: bool
    residuals: list = field(default_factory=list)   # R_0 .. R_{iters-1}
    # max residual of the returned trajectory (final_residual=True), else None
    final_residual: float | None = None


_libs: dict = {}
_active = _LIB_PATH
STRESS_LIB_PATH = os.path.join(_HERE, "libpararnn_stress.so")


def library_path() -> str:
    return _active


@contextlib.contextmanager
def using_library(path):
    """Route the calls made inside the block to the library at `path` (the look-back stress build,
    libpararnn_stress.so, in the tests); the default library afterwards."""
    global _active
    old = _active
    _active = path
    try:
        yield load_library()
    finally:
        _active = old


def load_library():
    """Load libpararnn.so (built by ``python -m nonlinear_rnn_solve_amd.build``); raises if absent."""
    lib = _libs.get(_active)
    if lib is not None:
        return lib
    if not os.path.exists(_active):
        raise RuntimeError("%s not built: run `python -m nonlinear_rnn_solve_amd.build` "
                           "(there is no CPU fallback)" % os.path.basename(_active))
    lib = ctypes.CDLL(_active)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.pararnn_abi_version.restype = i32
    lib.pararnn_status_string.restype = ctypes.c_char_p
    lib.pararnn_status_string.argtypes = [i32]
    lib.pararnn_newton_workspace_bytes.restype = sz
    lib.pararnn_newton_workspace_bytes.argtypes = [vp, vp]
    lib.pararnn_newton_solve.restype = i32
    lib.pararnn_newton_solve.argtypes = [vp, vp, vp, vp, sz, vp, vp]
    lib.pararnn_newton_solve_noalloc.restype = i32
    lib.pararnn_newton_solve_noalloc.argtypes = [vp, vp, vp, vp, vp]
    lib.pararnn_newton_prepare.restype = i32
    lib.pararnn_newton_prepare.argtypes = [vp, vp, vp, sz, vp]
    lib.pararnn_newton_iterate.restype = i32
    lib.pararnn_newton_iterate.argtypes = [vp, vp, i32, vp, vp, sz, vp]
    lib.pararnn_newton_report.restype = i32
    lib.pararnn_newton_report.argtypes = [vp, vp, vp, vp, sz, vp, vp]
    lib.pararnn_newton_budget.restype = i32
    lib.pararnn_newton_budget.argtypes = [i32, i32, i64, i32]
    lib.pararnn_scan_workspace_bytes.restype = sz
    lib.pararnn_scan_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.pararnn_linear_scan.restype = i32
    lib.pararnn_linear_scan.argtypes = [i32, i64, i64, i64, i32, vp, vp, vp, vp, i64, vp, i32, vp, sz, vp]
    lib.pararnn_vjp_workspace_bytes.restype = sz
    lib.pararnn_vjp_workspace_bytes.argtypes = [vp]
    lib.pararnn_scan_vjp.restype = i32
    lib.pararnn_scan_vjp.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    if hasattr(lib, "pararnn_debug_lookback_depth"):
        lib.pararnn_debug_lookback_depth.restype = i32
        lib.pararnn_debug_lookback_depth.argtypes = [i32]
    if lib.pararnn_abi_version() != ABI_VERSION:
        raise RuntimeError("%s ABI mismatch" % os.path.basename(_active))
    _libs[_active] = lib
    return lib


def lookback_depth(reset=True) -> int:
    """(stress build only) the deepest look-back walk since the last reset, in aggregates passed."""
    lib = load_library()
    if not hasattr(lib, "pararnn_debug_lookback_depth"):
        raise RuntimeError("%s is not the look-back stress build" % os.path.basename(_active))
    d = lib.pararnn_debug_lookback_depth(1 if reset else 0)
    if d < 0:
        raise PararnnError(d, "pararnn_debug_lookback_depth")
    return d


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (no CPU path exists)" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


_ws_cache: dict = {}


def _workspace(nbytes: int, device, key: str):
    """A cached device workspace per (device, current stream, key); grown on demand, 256-byte aligned by torch.

    One per stream because the library's calls use their workspace until they finish on their stream: calls on
    different streams may overlap, and a graph captured on a stream keeps using that stream's buffer (capture
    on a stream that has already run the same call, so that nothing is allocated during capture)."""
    k = (str(device), torch.cuda.current_stream(device).cuda_stream, key)
    buf = _ws_cache.get(k)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[k] = buf
    return buf


def _seqlens(cu_seqlens, device):
    """Packed-sequence offsets: an int32 tensor [n_seqs + 1] on the GPU (or None)."""
    if cu_seqlens is None:
        return None, 0
    _check_dev(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of n_seqs + 1 offsets")
    if cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be on the same device as the inputs")
    return cu_seqlens.data_ptr(), cu_seqlens.numel() - 1


def _problem(cell, pre, w, bias, s0, cu_seqlens=None):
    c = CELLS[cell] if isinstance(cell, str) else int(cell)
    G, S = GATES[c], STATE[c]
    if len(pre) != G:
        raise ValueError("cell needs %d pre-activation planes, got %d" % (G, len(pre)))
    dt = pre[0].dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("pre-activations must be float32 or bfloat16")
    for i, p in enumerate(pre):
        _check_dev(p, "pre[%d]" % i, dt)
        if p.shape != pre[0].shape or p.dim() != 3:
            raise ValueError("pre planes must all be [B, T, D]")
    B, T, D = pre[0].shape
    head_size = 0
    if c != 0:
        _check_dev(w, "w", torch.float32)
        _check_dev(bias, "bias", torch.float32)
        if c == HEAD_GRU:
            # w: [3, n_heads, hs, hs] dense blocks (block row = output channel)
            if w.dim() != 4 or w.shape[0] != G or w.shape[2] != w.shape[3] or w.shape[1] * w.shape[2] != D:
                raise ValueError("head_gru w must be [3, n_heads, hs, hs] with n_heads * hs = D = %d" % D)
            head_size = int(w.shape[2])
            if tuple(bias.shape) != (G, D):
                raise ValueError("bias must be [G, D] = [%d, %d]" % (G, D))
        elif tuple(w.shape) != (G, D) or tuple(bias.shape) != (G, D):
            raise ValueError("w and bias must be [G, D] = [%d, %d]" % (G, D))
    _check_dev(s0, "s0", torch.float32)
    if s0 is not None and tuple(s0.shape) != (S, B, D):
        raise ValueError("s0 must be [S, B, D] = [%d, %d, %d]" % (S, B, D))
    st = _Problem()
    st.cell, st.pre_dtype, st.B, st.T, st.D = c, 1 if dt == torch.bfloat16 else 0, B, T, D
    for i in range(4):
        st.pre[i] = pre[i].data_ptr() if i < G else None
    st.w = w.data_ptr() if (c != 0 and w is not None) else None
    st.bias = bias.data_ptr() if (c != 0 and bias is not None) else None
    st.s0 = s0.data_ptr() if s0 is not None else None
    st.cu_seqlens, st.n_seqs = _seqlens(cu_seqlens, pre[0].device)
    st.head_size = head_size
    _same_device(list(pre) + [w if c != 0 else None, bias if c != 0 else None, s0], pre[0].device)
    return st, c, G, S, (B, T, D)


def newton_workspace_bytes(cell, pre, w=None, bias=None, s0=None, cu_seqlens=None) -> int:
    st, *_ = _problem(cell, pre, w, bias, s0, cu_seqlens)
    return int(load_library().pararnn_newton_workspace_bytes(ctypes.byref(st), None))


def newton_budget(cell, T, warm_start=False, max_iters=None) -> int:
    """The Newton budget a solve runs: max_iters, or the measured K*(T) when it is None or 0."""
    c = CELLS[cell] if isinstance(cell, str) else int(cell)
    k = load_library().pararnn_newton_budget(c, INIT_WARM if warm_start else INIT_ZERO, int(T), int(max_iters or 0))
    if k < 1:
        raise PararnnError(k, "pararnn_newton_budget")
    return k


def _same_device(tensors, device):
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError("all tensors must be on %s (got %s)" % (device, t.device))


def _on_device(pos, name):
    """Run a call with the device of its argument `pos` / `name` (a tensor or a list of them) current, so
    that the kernels launch on the device that holds the data."""
    def deco(fn):
        @functools.wraps(fn)
        def wrapped(*args, **kwargs):
            x = args[pos] if len(args) > pos else kwargs.get(name)
            t = x[0] if isinstance(x, (list, tuple)) and len(x) else x
            if isinstance(t, torch.Tensor) and t.is_cuda:
                with torch.cuda.device(t.device):
                    return fn(*args, **kwargs)
            return fn(*args, **kwargs)
        return wrapped
    return deco


@_on_device(1, "pre")
def newton_solve(cell, pre, w=None, bias=None, max_iters=3, tol=0.0, s0=None, init_guess=None, out=None,
                 final_residual=False, report=True, on_iteration=None, warm_start=False, cu_seqlens=None,
                 picard_iters=0, fuse_iters=0, noalloc=False):
    """Newton solve of F(H) = 0.  Returns (trajectory [S, B, T, D] float32, NewtonReport or None).

    pre: G planes [B, T, D] (float32 or bfloat16) on the GPU; w, bias: [G, D] float32 (head_gru: w is
    [3, n_heads, hs, hs], the dense recurrent block of each head); s0: [S, B, D].
    max_iters None or 0: the measured budget K*(T) (see newton_budget).
    tol <= 0: exactly max_iters iterations; tol > 0: stop after the first iteration whose max residual
    (evaluated at its input iterate) is below tol.  report=True waits for the stream.
    warm_start: without init_guess, start from H^0_t = f(0, x_t) instead of zeros.
    cu_seqlens: int32 [n_seqs + 1] offsets of sequences packed along T (every batch row); each sequence
    after the first starts from the zero state.
    picard_iters: the first picard_iters of the iterations are Picard sweeps H_t = f(H_{t-1}, x_t).
    fuse_iters: iterations per launch (gru / lstm): 1 = one launch per iteration, 2..MAX_FUSE = up to that
    many in one launch that keeps the trajectory in registers, 0 = the library's choice.  The result is the
    same bit for bit; only the launches (and the workspace size) change.
    on_iteration: optional callable(k, phase) with phase "before"/"after", invoked on the host around the
    launch of iteration k (e.g. to record stream events); the solve then runs through the step-wise
    entry points prepare / iterate / report, which launch exactly the same kernels.
    noalloc: call pararnn_newton_solve_noalloc, whose workspace is the library's static device array (no
    workspace is allocated here either); calls that overlap on one GPU must not use it.
    """
    lib = load_library()
    st, c, G, S, (B, T, D) = _problem(cell, pre, w, bias, s0, cu_seqlens)
    dev = pre[0].device
    if out is None:
        out = torch.empty((S, B, T, D), dtype=torch.float32, device=dev)
    _check_dev(out, "out", torch.float32)
    _check_dev(init_guess, "init_guess", torch.float32)
    _same_device([out, init_guess], dev)
    if tuple(out.shape) != (S, B, T, D):
        raise ValueError("out must be [S, B, T, D]")
    if init_guess is not None and tuple(init_guess.shape) != (S, B, T, D):
        raise ValueError("init_guess must be [S, B, T, D]")
    opts = _Opts(int(max_iters or 0), float(tol), init_guess.data_ptr() if init_guess is not None else None,
                 1 if final_residual else 0, INIT_WARM if warm_start else INIT_ZERO, int(picard_iters),
                 int(fuse_iters))
    rep = _Report() if report else None
    stream = _stream(dev)
    if noalloc:
        if on_iteration is not None:
            raise ValueError("on_iteration needs the step-wise entry points, which take a workspace")
        rc = lib.pararnn_newton_solve_noalloc(ctypes.byref(st), ctypes.byref(opts), _ptr(out), stream,
                                              ctypes.byref(rep) if rep is not None else None)
        return _newton_result(rc, rep, final_residual, out)
    nbytes = lib.pararnn_newton_workspace_bytes(ctypes.byref(st), ctypes.byref(opts))
    ws = _workspace(nbytes, dev, "newton")
    if on_iteration is None:
        rc = lib.pararnn_newton_solve(ctypes.byref(st), ctypes.byref(opts), _ptr(out), _ptr(ws), ws.numel(),
                                      stream, ctypes.byref(rep) if rep is not None else None)
    else:
        rc = lib.pararnn_newton_prepare(ctypes.byref(st), ctypes.byref(opts), _ptr(ws), ws.numel(), stream)
        K = newton_budget(cell, T, warm_start and init_guess is None, max_iters)
        for k in range(K):
            if rc != 0:
                break
            on_iteration(k, "before")
            rc = lib.pararnn_newton_iterate(ctypes.byref(st), ctypes.byref(opts), k, _ptr(out), _ptr(ws),
                                            ws.numel(), stream)
            on_iteration(k, "after")
        if rc == 0:
            rc = lib.pararnn_newton_report(ctypes.byref(st), ctypes.byref(opts), _ptr(out), _ptr(ws), ws.numel(),
                                           stream, ctypes.byref(rep) if rep is not None else None)
    return _newton_result(rc, rep, final_residual, out)


def _newton_result(rc, rep, final_residual, out):
    r = None
    if rep is not None:
        res = [float(rep.residual[i]) for i in range(rep.n_residual)]
        r = NewtonReport(int(rep.iters), bool(rep.converged), res[:rep.iters],
                         res[rep.iters] if final_residual and rep.n_residual > rep.iters else None)
    if rc == -5:
        raise NewtonDivergenceError(rc, "pararnn_newton_solve", r)
    if rc != 0:
        raise PararnnError(rc, "pararnn_newton_solve")
    return out, r


def scan_workspace_bytes(S, B, T, D) -> int:
    return int(load_library().pararnn_scan_workspace_bytes(S, B, T, D))


@_on_device(0, "a")
def linear_scan(a, b, s0=None, reverse=False, out=None, cu_seqlens=None):
    """Single-pass parallel linear recurrence.

    S=1: a, b [B, T, D];  S=2: a [4, B, T, D] (A00, A01, A10, A11), b [2, B, T, D].
    forward: s_t = A_t s_{t-1} + b_t (s_{-1} = s0);  reverse: s_t = A_t s_{t+1} + b_t (s_T = s0).
    cu_seqlens: int32 [n_seqs + 1] offsets of packed sequences; the state entering each is zero, s0
    entering the one at the scan's starting end.
    Returns float32 [B, T, D] (S=1) or [2, B, T, D] (S=2).
    """
    lib = load_library()
    S = 2 if a.dim() == 4 else 1
    _check_dev(a, "a")
    _check_dev(b, "b", a.dtype)
    if a.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("a, b must be float32 or bfloat16")
    B, T, D = b.shape[-3:]
    if S == 2 and (tuple(a.shape) != (4, B, T, D) or tuple(b.shape) != (2, B, T, D)):
        raise ValueError("S=2 needs a [4,B,T,D] and b [2,B,T,D]")
    if S == 1 and tuple(a.shape) != (B, T, D):
        raise ValueError("a and b must have the same [B,T,D] shape")
    _check_dev(s0, "s0", torch.float32)
    if s0 is not None and s0.numel() != S * B * D:
        raise ValueError("s0 must hold S*B*D values")
    if out is None:
        out = torch.empty(b.shape, dtype=torch.float32, device=a.device)
    _check_dev(out, "out", torch.float32)
    _same_device([b, s0, out, cu_seqlens], a.device)
    if out.shape != b.shape:
        raise ValueError("out must have b's shape")
    cu, n_seqs = _seqlens(cu_seqlens, a.device)
    nbytes = lib.pararnn_scan_workspace_bytes(S, B, T, D)
    ws = _workspace(nbytes, a.device, "scan")
    rc = lib.pararnn_linear_scan(S, B, T, D, 1 if a.dtype == torch.bfloat16 else 0, _ptr(a), _ptr(b), _ptr(s0),
                                 cu, n_seqs, _ptr(out), 1 if reverse else 0, _ptr(ws), ws.numel(),
                                 _stream(a.device))
    if rc != 0:
        raise PararnnError(rc, "pararnn_linear_scan")
    return out


def vjp_workspace_bytes(cell, pre, w=None, bias=None, s0=None, cu_seqlens=None) -> int:
    st, *_ = _problem(cell, pre, w, bias, s0, cu_seqlens)
    return int(load_library().pararnn_vjp_workspace_bytes(ctypes.byref(st)))


@_on_device(1, "pre")
def scan_vjp(cell, pre, s, g, w=None, bias=None, s0=None, want_lambda=False, want_params=True, want_s0=True,
             cu_seqlens=None):
    """Gradients at trajectory s ([S,B,T,D] float32) for upstream g = dL/dh ([B,T,D] float32).

    Returns dict: d_pre [G,B,T,D]; d_w, d_bias [G,D] (gated cells; head_gru d_w is [3, n_heads, hs, hs]);
    d_s0 [S,B,D]; lam [S,B,T,D] if asked.
    """
    lib = load_library()
    st, c, G, S, (B, T, D) = _problem(cell, pre, w, bias, s0, cu_seqlens)
    dev = pre[0].device
    _check_dev(s, "s", torch.float32)
    _check_dev(g, "g", torch.float32)
    _same_device([s, g], dev)
    if tuple(s.shape) != (S, B, T, D) or tuple(g.shape) != (B, T, D):
        raise ValueError("s must be [S,B,T,D] and g [B,T,D]")
    d_pre = torch.empty((G, B, T, D), dtype=torch.float32, device=dev)
    wshape = tuple(w.shape) if c == HEAD_GRU else (G, D)   # head_gru: [3, n_heads, hs, hs]
    d_w = torch.empty(wshape, dtype=torch.float32, device=dev) if (c != 0 and want_params) else None
    d_b = torch.empty((G, D), dtype=torch.float32, device=dev) if (c != 0 and want_params) else None
    d_s0 = torch.empty((S, B, D), dtype=torch.float32, device=dev) if want_s0 else None
    lam = torch.empty((S, B, T, D), dtype=torch.float32, device=dev) if want_lambda else None
    nbytes = lib.pararnn_vjp_workspace_bytes(ctypes.byref(st))
    ws = _workspace(nbytes, dev, "vjp")
    rc = lib.pararnn_scan_vjp(ctypes.byref(st), _ptr(s), _ptr(g), _ptr(d_pre), _ptr(d_w), _ptr(d_b), _ptr(d_s0),
                              _ptr(lam), _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise PararnnError(rc, "pararnn_scan_vjp")
    out = {"d_pre": d_pre, "d_s0": d_s0, "lam": lam}
    if c != 0 and want_params:
        out["d_w"], out["d_bias"] = d_w, d_b
    return out
