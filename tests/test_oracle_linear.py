"""Pins for the oracle's linear recurrence (forward / reverse, state size 1 and 2).

The linear recurrence s_t = A_t s_{t-1} + b_t is what every Newton linear solve
reduces to (pararnn-torch README, "Method": the linearised system is solved by a
parallel scan along time).  The oracle evaluates it step by step; these tests check it
against closed forms and brute-force sums that share nothing with it.
"""
import numpy as np
import pytest

import oracle
from nonlinear_rnn_solve_amd import synth


def brute_forward(a, b, s0):
    """h_t = (prod_{u<=t} a_u) s0 + sum_{s<=t} (prod_{u=s+1}^{t} a_u) b_s, O(T^2) per channel."""
    B, T, D = b.shape
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    out = np.zeros((B, T, D))
    for t in range(T):
        acc = np.prod(a[:, : t + 1, :], axis=1) * s0
        for s in range(t + 1):
            acc = acc + np.prod(a[:, s + 1: t + 1, :], axis=1) * b[:, s, :]
        out[:, t, :] = acc
    return out


def brute_reverse(a, b, sT):
    """h_t = (prod_{u=t}^{T-1} a_u) sT + sum_{s>=t} (prod_{u=t}^{s-1} a_u) b_s."""
    B, T, D = b.shape
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    out = np.zeros((B, T, D))
    for t in range(T):
        acc = np.prod(a[:, t:, :], axis=1) * sT
        for s in range(t, T):
            acc = acc + np.prod(a[:, t:s, :], axis=1) * b[:, s, :]
        out[:, t, :] = acc
    return out


@pytest.mark.parametrize("a,b,s0", [(0.5, 1.0, 0.0), (0.9, -0.3, 2.0), (-0.7, 0.25, -1.5), (0.999, 1.0, 0.0)])
def test_geometric_series_closed_form(a, b, s0):
    # constant coefficients: h_t = a^{t+1} s0 + b (1 - a^{t+1}) / (1 - a)   (t = 0-based)
    T = 300
    A = np.full((1, T, 1), a, np.float32)
    Bv = np.full((1, T, 1), b, np.float32)
    out = oracle.linear_scan(A, Bv, s0=np.array([s0], np.float32))
    af, bf = float(np.float32(a)), float(np.float32(b))
    n = np.arange(1, T + 1)
    want = af ** n * float(np.float32(s0)) + bf * (1 - af ** n) / (1 - af)
    np.testing.assert_allclose(out[0, :, 0], want, rtol=1e-12, atol=1e-12)


def test_constant_a_convolution_form():
    # constant a, varying b: h_t = sum_{s<=t} a^{t-s} b_s
    rng = np.random.default_rng(5)
    T, a = 200, np.float32(0.8)
    b = rng.standard_normal((2, T, 3)).astype(np.float32)
    out = oracle.linear_scan(np.full(b.shape, a, np.float32), b)
    k = float(a) ** np.arange(T)
    for bi in range(2):
        for d in range(3):
            want = np.convolve(b[bi, :, d].astype(np.float64), k)[:T]
            np.testing.assert_allclose(out[bi, :, d], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [1000, 1001])
def test_forward_brute_force(seed):
    inp = synth.make_inputs("linear", 2, 23, 5, seed=seed)
    a, b = inp.pre
    s0 = synth.random_state(1, 2, 5, seed + 7)
    out = oracle.linear_scan(a, b, s0=s0)
    np.testing.assert_allclose(out, brute_forward(a, b, s0[0].astype(np.float64)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [1002, 1003])
def test_reverse_brute_force(seed):
    inp = synth.make_inputs("linear", 2, 19, 4, seed=seed)
    a, b = inp.pre
    sT = synth.random_state(1, 2, 4, seed + 9)
    out = oracle.linear_scan(a, b, s0=sT, reverse=True)
    np.testing.assert_allclose(out, brute_reverse(a, b, sT[0].astype(np.float64)), rtol=1e-12, atol=1e-12)


def test_state2_brute_force_matrix_products():
    rng = np.random.default_rng(11)
    B, T, D = 2, 9, 3
    A = (rng.standard_normal((4, B, T, D)) * 0.6).astype(np.float32)
    b = rng.standard_normal((2, B, T, D)).astype(np.float32)
    s0 = rng.standard_normal((2, B, D)).astype(np.float32)
    out = oracle.linear_scan(A, b, s0=s0, S=2)
    outr = oracle.linear_scan(A, b, s0=s0, S=2, reverse=True)
    for bi in range(B):
        for d in range(D):
            M = [A[:, bi, t, d].astype(np.float64).reshape(2, 2) for t in range(T)]
            v = [b[:, bi, t, d].astype(np.float64) for t in range(T)]
            x0 = s0[:, bi, d].astype(np.float64)
            for t in range(T):
                P = np.eye(2)
                for u in range(t + 1):
                    P = M[u] @ P
                want = P @ x0
                for s in range(t + 1):
                    Q = np.eye(2)
                    for u in range(s + 1, t + 1):
                        Q = M[u] @ Q
                    want = want + Q @ v[s]
                np.testing.assert_allclose(out[:, bi, t, d], want, rtol=1e-12, atol=1e-12)
                # reverse: s_t = A_t s_{t+1} + b_t with s_T = s0
                P = np.eye(2)
                for u in range(T - 1, t - 1, -1):
                    P = M[u] @ P
                want = P @ x0
                for s in range(t, T):
                    Q = np.eye(2)
                    for u in range(s - 1, t - 1, -1):
                        Q = M[u] @ Q
                    want = want + Q @ v[s]
                np.testing.assert_allclose(outr[:, bi, t, d], want, rtol=1e-12, atol=1e-12)


def test_state2_jordan_block_powers_catch_transpose():
    # A = [[p, q], [0, p]] constant, b = 0:  s_t = A^{t+1} s0,  A^n = [[p^n, n p^{n-1} q], [0, p^n]]
    p, q, T = 0.9, 0.5, 40
    A = np.zeros((4, 1, T, 1), np.float32)
    A[0], A[1], A[3] = p, q, p
    s0 = np.array([[[0.0]], [[1.0]]], np.float32)   # (c, h) = (0, 1)
    out = oracle.linear_scan(A, np.zeros((2, 1, T, 1), np.float32), s0=s0, S=2)
    pf, qf = float(np.float32(p)), float(np.float32(q))
    n = np.arange(1, T + 1)
    np.testing.assert_allclose(out[0, 0, :, 0], n * pf ** (n - 1) * qf, rtol=1e-12)
    np.testing.assert_allclose(out[1, 0, :, 0], pf ** n, rtol=1e-12)


def test_bf16_inputs_decode_exactly():
    inp = synth.make_inputs("linear", 1, 50, 8, dtype="bf16", seed=3)
    a16, b16 = inp.pre
    out16 = oracle.linear_scan(a16, b16, dtype=oracle.BF16)
    a32, b32 = inp.pre_f32()
    out32 = oracle.linear_scan(a32, b32)
    np.testing.assert_array_equal(out16, out32)


def test_empty_and_single_step():
    a = np.zeros((1, 0, 4), np.float32)
    assert oracle.linear_scan(a, a).shape == (1, 0, 4)
    a1 = np.full((1, 1, 2), 0.5, np.float32)
    b1 = np.array([[[1.0, -2.0]]], np.float32)
    out = oracle.linear_scan(a1, b1, s0=np.array([[4.0, 4.0]], np.float32))
    np.testing.assert_allclose(out[0, 0], [3.0, 0.0])
