"""CPU oracle for the ParaRNN hot path -- TEST INFRASTRUCTURE ONLY.

A plain fp64 implementation (``pararnn_oracle.c``) of what the GPU library
computes: the sequential unroll of a diagonal GRU / LSTM / sLSTM / linear cell or of the
head-wise block GRU (dense recurrent block per head), Newton
on F(H)_t = h_t - f(h_{t-1}, x_t) = 0 with a *sequential* linear solve, the
linear recurrence itself (forward and reverse, state size 1 or 2), and the
adjoint (VJP) at a solved trajectory.  Sources: pararnn-torch README (PyPI
page), section "Method"; ParaRNN abstract (HF paper list).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the GPU library and does
not import it; the two meet only through the seeded input generator, which
holds none of the method's arithmetic.

Pins (what checks this oracle against something other than itself) live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pararnn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

LINEAR, GRU, LSTM, SLSTM, HEAD_GRU = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
CELLS = {"linear": LINEAR, "gru": GRU, "lstm": LSTM, "slstm": SLSTM, "head_gru": HEAD_GRU}
OK, EINVAL, ENOMEM, DIVERGED = 0, -1, -2, -5


def state_size(cell: int) -> int:
    return {LINEAR: 1, GRU: 1, LSTM: 2, SLSTM: 4, HEAD_GRU: 1}[cell]


def gate_count(cell: int) -> int:
    return {LINEAR: 2, GRU: 3, LSTM: 4, SLSTM: 4, HEAD_GRU: 3}[cell]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.or_cell_step.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.or_unroll.argtypes = [vp, vp, i32]
        lib.or_residual.argtypes = [vp, vp, vp, i32]
        lib.or_newton.argtypes = [vp, vp, i32, i32, i32, dbl, vp, vp, vp, vp, i32]
        lib.or_linear_scan.argtypes = [i32, i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, i32]
        lib.or_vjp.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.or_hgru_step.argtypes = [i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        assert lib.or_abi_version() == 7
        _lib = lib
    return _lib


class _Problem(ctypes.Structure):
    _fields_ = [("cell", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
                ("pre", ctypes.c_void_p * 4), ("w", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("s0", ctypes.c_void_p), ("seg_start", ctypes.c_void_p),
                ("head_size", ctypes.c_int64)]


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def seg_start_flags(cu_seqlens, T):
    """Packed sequences: offsets cu_seqlens (sequence j covers steps cu[j] .. cu[j+1]-1) -> a [T]
    uint8 array that is 1 where a sequence other than the first begins.  None -> None."""
    if cu_seqlens is None:
        return None
    flags = np.zeros(max(T, 1), np.uint8)
    for c in np.asarray(cu_seqlens).ravel():
        if 0 < int(c) < T:
            flags[int(c)] = 1
    return flags


def _as_pre(pre, dtype):
    """pre planes: float32 arrays (dtype F32) or uint16 bf16 bit patterns (BF16)."""
    want = np.float32 if dtype == F32 else np.uint16
    return [np.ascontiguousarray(p, dtype=want) for p in pre]


class Problem:
    """Holds contiguous copies of the inputs and the ctypes struct that points at them."""

    def __init__(self, cell, pre, w=None, bias=None, s0=None, dtype=F32, cu_seqlens=None, head_size=None):
        """head_gru: w is [3][n_heads][hs][hs] (block row = output channel) and head_size = hs."""
        cell = CELLS.get(cell, cell)
        self.cell, self.dtype = cell, dtype
        self.pre = _as_pre(pre, dtype)
        G = gate_count(cell)
        assert len(self.pre) == G, "cell needs %d pre-activation planes" % G
        B, T, D = self.pre[0].shape
        for p in self.pre:
            assert p.shape == (B, T, D)
        self.B, self.T, self.D = B, T, D
        self.S = state_size(cell)
        self.head_size = 1
        if cell == HEAD_GRU:
            assert head_size is not None and head_size >= 1 and D % head_size == 0
            self.head_size = int(head_size)
        wcols = D * self.head_size
        self.w = None if w is None else np.ascontiguousarray(w, dtype=np.float32).reshape(G, wcols)
        self.bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32).reshape(G, D)
        if cell != LINEAR:
            assert self.w is not None and self.bias is not None
        self.s0 = None if s0 is None else np.ascontiguousarray(s0, dtype=np.float32).reshape(self.S, B, D)
        st = _Problem()
        st.cell, st.dtype, st.B, st.T, st.D = cell, dtype, B, T, D
        for g in range(4):
            st.pre[g] = _ptr(self.pre[g]) if g < G else None
        st.w, st.bias, st.s0 = _ptr(self.w), _ptr(self.bias), _ptr(self.s0)
        self.seg_start = seg_start_flags(cu_seqlens, T)
        st.seg_start = _ptr(self.seg_start)
        st.head_size = self.head_size
        self.struct = st

    def traj_shape(self):
        return (self.S, self.B, self.T, self.D)


def _check(rc, what):
    if rc not in (OK, DIVERGED):
        raise RuntimeError("oracle %s failed with status %d" % (what, rc))
    return rc


def cell_step(cell, u, w, bias, s):
    """One step of one channel in fp64: returns (s_next, J[S,S], dfdu[S,G], wcoef[G])."""
    cell = CELLS.get(cell, cell)
    S, G = state_size(cell), gate_count(cell)
    u = np.ascontiguousarray(u, dtype=np.float64)
    w = np.ascontiguousarray(np.zeros(G) if w is None else w, dtype=np.float64)
    bias = np.ascontiguousarray(np.zeros(G) if bias is None else bias, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    sn, J = np.zeros(S), np.zeros(S * S)
    dfdu, wc = np.zeros(S * G), np.zeros(G)
    _check(_load().or_cell_step(cell, _ptr(u), _ptr(w), _ptr(bias), _ptr(s), _ptr(sn),
                                _ptr(J), _ptr(dfdu), _ptr(wc)), "cell_step")
    return sn, J.reshape(S, S), dfdu.reshape(S, G), wc


def hgru_step(u, A, bias, h):
    """One step of one head of the head-wise block GRU in fp64.  u [3][hs], A [3][hs][hs],
    bias [3][hs], h [hs].  Returns (h_next, J [hs][hs], dz [hs], dc [hs], dr [hs][hs], rh [hs])."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    hs = A.shape[-1]
    u = np.ascontiguousarray(u, dtype=np.float64).reshape(3 * hs)
    bias = np.ascontiguousarray(bias, dtype=np.float64).reshape(3 * hs)
    h = np.ascontiguousarray(h, dtype=np.float64).reshape(hs)
    hn, dz, dc, rh = np.zeros(hs), np.zeros(hs), np.zeros(hs), np.zeros(hs)
    J, dr = np.zeros(hs * hs), np.zeros(hs * hs)
    _check(_load().or_hgru_step(hs, _ptr(u), _ptr(A), _ptr(bias), _ptr(h), _ptr(hn), _ptr(J), _ptr(dz), _ptr(dc),
                                _ptr(dr), _ptr(rh)), "hgru_step")
    return hn, J.reshape(hs, hs), dz, dc, dr.reshape(hs, hs), rh


def unroll(prob: Problem, nthreads=None):
    """Sequential unroll s_t = f(s_{t-1}, x_t); returns fp64 [S][B][T][D]."""
    out = np.zeros(prob.traj_shape(), dtype=np.float64)
    _check(_load().or_unroll(ctypes.byref(prob.struct), _ptr(out), nthreads or default_threads()), "unroll")
    return out


def residual(prob: Problem, H, nthreads=None) -> float:
    H = np.ascontiguousarray(H, dtype=np.float64).reshape(prob.traj_shape())
    m = np.zeros(1)
    _check(_load().or_residual(ctypes.byref(prob.struct), _ptr(H), _ptr(m), nthreads or default_threads()),
           "residual")
    return float(m[0])


def newton(prob: Problem, max_iters, tol=0.0, init_guess=None, nthreads=None, warm=False, picard=0):
    """Newton with sequential linear solves. Returns (H fp64, residuals[iters], iters, converged, status).

    warm=True starts from H^0_t = f(0, x_t) (ignored when init_guess is given); the first `picard`
    of the max_iters updates are Picard sweeps H^{k+1}_t = f(H^k_{t-1}, x_t)."""
    H = np.zeros(prob.traj_shape(), dtype=np.float64)
    res = np.zeros(max(1, max_iters))
    it, conv = ctypes.c_int(0), ctypes.c_int(0)
    ig = None if init_guess is None else np.ascontiguousarray(init_guess, dtype=np.float32).reshape(prob.traj_shape())
    rc = _check(_load().or_newton(ctypes.byref(prob.struct), _ptr(ig), 1 if warm else 0, int(picard), int(max_iters),
                                  float(tol), _ptr(H),
                                  _ptr(res), ctypes.byref(it), ctypes.byref(conv), nthreads or default_threads()),
                "newton")
    return H, res[: it.value].copy(), it.value, bool(conv.value), rc


def linear_scan(a, b, s0=None, reverse=False, S=1, dtype=F32, nthreads=None, cu_seqlens=None):
    """Sequential linear recurrence in fp64. S=1: a,b [B][T][D]; S=2: a [4][B][T][D], b [2][B][T][D]."""
    want = np.float32 if dtype == F32 else np.uint16
    a = np.ascontiguousarray(a, dtype=want)
    b = np.ascontiguousarray(b, dtype=want)
    B, T, D = b.shape[-3:]
    if S == 2:
        assert a.shape == (4, B, T, D) and b.shape == (2, B, T, D)
    else:
        assert a.shape == (B, T, D) and b.shape == (B, T, D)
    s0a = None if s0 is None else np.ascontiguousarray(s0, dtype=np.float32).reshape(S, B, D)
    out = np.zeros((S, B, T, D) if S == 2 else (B, T, D), dtype=np.float64)
    seg = seg_start_flags(cu_seqlens, T)
    _check(_load().or_linear_scan(S, B, T, D, dtype, _ptr(a), _ptr(b), _ptr(s0a), _ptr(seg), 1 if reverse else 0,
                                  _ptr(out), nthreads or default_threads()), "linear_scan")
    return out


def vjp(prob: Problem, s, g, want_lambda=True, nthreads=None):
    """Adjoint at trajectory s ([S][B][T][D]); g = dL/dh [B][T][D].

    Returns dict with d_pre [G][B][T][D], d_w [G][D] (head_gru: [3][n_heads][hs][hs]), d_bias [G][D],
    d_s0 [S][B][D], lam [S][B][T][D].
    """
    G = gate_count(prob.cell)
    s = np.ascontiguousarray(s, dtype=np.float64).reshape(prob.traj_shape())
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(prob.B, prob.T, prob.D)
    d_pre = np.zeros((G, prob.B, prob.T, prob.D))
    if prob.cell == HEAD_GRU:
        hs = prob.head_size
        d_w = np.zeros((G, prob.D // hs, hs, hs))
    else:
        d_w = np.zeros((G, prob.D))
    d_bias = np.zeros((G, prob.D))
    d_s0 = np.zeros((prob.S, prob.B, prob.D))
    lam = np.zeros(prob.traj_shape()) if want_lambda else None
    _check(_load().or_vjp(ctypes.byref(prob.struct), _ptr(s), _ptr(g), _ptr(d_pre), _ptr(d_w), _ptr(d_bias),
                          _ptr(d_s0), _ptr(lam), nthreads or default_threads()), "vjp")
    out = {"d_pre": d_pre, "d_s0": d_s0, "lam": lam}
    if prob.cell != LINEAR:
        out["d_w"], out["d_bias"] = d_w, d_bias
    return out
