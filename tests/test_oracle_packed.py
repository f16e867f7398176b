"""Pins for the oracle on packed variable-length sequences (pararnn-torch README, "Compatibility":
shapes and packing, with packed batches described by cumulative sequence offsets, cu_seqlens).

Reading: the [B][T][D] planes hold several sequences back to back along T; sequence j covers steps
cu_seqlens[j] .. cu_seqlens[j+1]-1.  The state entering each sequence after the first is zero (s0
is the first sequence's initial state), nothing flows across a boundary in either direction, and
the same offsets apply to every batch row.  Each system therefore splits into independent
per-sequence systems.  Pinned against
  * dense Newton on the full packed system (torch library cells, autograd Jacobian, numpy solve);
  * torch autograd through the unroll with the state reset at each sequence start;
  * the definition itself: the packed result equals the concatenation of independent
    per-sequence results of the unpacked oracle (which the other oracle tests pin).
"""
import numpy as np
import pytest
import torch

import oracle
from nonlinear_rnn_solve_amd import synth
from test_oracle_newton import dense_newton
from test_oracle_vjp import autograd_reference


@pytest.fixture(autouse=True)
def _fp64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def segments(cu):
    return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])]


def sliced(inp, a, b):
    """The inputs of steps a .. b-1 as their own problem (same weights)."""
    return [np.ascontiguousarray(p[:, a:b]) for p in inp.pre]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_packed_newton_matches_dense_newton(cell, K):
    inp = synth.make_inputs(cell, 1, 9, 2, seed=1020)
    s0 = synth.random_state(inp.S, 1, 2, seed=21)
    cu = [0, 3, 5, 9]
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0, cu_seqlens=cu)
    H = oracle.newton(prob, K)[0]
    np.testing.assert_allclose(H, dense_newton(inp, s0, K, starts={3, 5}), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("cell", ["linear", "gru", "lstm"])
def test_packed_unroll_newton_and_vjp_split_into_sequences(cell):
    B, T, D = 2, 120, 3
    inp = synth.make_inputs(cell, B, T, D, seed=1021, with_grad=True)
    s0 = synth.random_state(inp.S, B, D, seed=22)
    cu = [0, 1, 17, 17, 64, 119, 120]          # includes a length-1 and an empty sequence
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0, cu_seqlens=cu)
    U = oracle.unroll(prob)
    assert oracle.residual(prob, U) == 0.0
    K = 2
    Hk = oracle.newton(prob, K)[0]
    V = oracle.vjp(prob, U, inp.g)
    dw = np.zeros_like(V["d_w"]) if cell != "linear" else None
    for j, (a, b) in enumerate(segments(cu)):
        if a == b:
            continue
        sub = oracle.Problem(cell, sliced(inp, a, b), inp.w, inp.bias, s0=s0 if j == 0 else None)
        Us = oracle.unroll(sub)
        np.testing.assert_array_equal(U[:, :, a:b], Us)
        np.testing.assert_allclose(Hk[:, :, a:b], oracle.newton(sub, K)[0], rtol=0, atol=1e-14)
        Vs = oracle.vjp(sub, Us, np.ascontiguousarray(inp.g[:, a:b]))
        np.testing.assert_allclose(V["d_pre"][:, :, a:b], Vs["d_pre"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(V["lam"][:, :, a:b], Vs["lam"], rtol=0, atol=1e-14)
        if j == 0:
            np.testing.assert_allclose(V["d_s0"], Vs["d_s0"], rtol=0, atol=1e-14)
        if dw is not None:
            dw += Vs["d_w"]
    if dw is not None:
        np.testing.assert_allclose(V["d_w"], dw, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cell", ["linear", "gru", "lstm"])
def test_packed_vjp_matches_autograd(cell):
    inp = synth.make_inputs(cell, 2, 23, 3, seed=1022, with_grad=True)
    s0 = synth.random_state(inp.S, 2, 3, seed=23)
    cu = [0, 4, 5, 15, 23]
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0, cu_seqlens=cu)
    got = oracle.vjp(prob, oracle.unroll(prob), inp.g)
    want = autograd_reference(inp, s0, inp.g, starts={4, 5, 15})
    if cell == "lstm":   # only lambda_h is the same quantity as autograd's (see test_oracle_vjp)
        want["lam"] = want["lam"][1:]
        got = dict(got, lam=got["lam"][1:])
    for k in want:
        np.testing.assert_allclose(got[k], want[k], rtol=1e-11, atol=1e-12, err_msg=k)


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
def test_packed_linear_scan_splits_into_sequences(S, reverse):
    B, T, D = 2, 50, 4
    rng = np.random.default_rng(1023)
    a = rng.uniform(-0.9, 0.9, ((4,) if S == 2 else ()) + (B, T, D)).astype(np.float32)
    b = rng.standard_normal(((2,) if S == 2 else ()) + (B, T, D)).astype(np.float32)
    s0 = rng.standard_normal((S, B, D)).astype(np.float32)
    cu = [0, 7, 8, 30, 50]
    got = oracle.linear_scan(a, b, s0=s0, reverse=reverse, S=S, cu_seqlens=cu)
    segs = segments(cu)
    for j, (lo, hi) in enumerate(segs):
        edge = (j == len(segs) - 1) if reverse else (j == 0)   # s0 enters at the scan's starting end
        want = oracle.linear_scan(np.ascontiguousarray(a[..., lo:hi, :]), np.ascontiguousarray(b[..., lo:hi, :]),
                                  s0=s0 if edge else None, reverse=reverse, S=S)
        np.testing.assert_array_equal(got[..., lo:hi, :], want)


def test_trivial_offsets_change_nothing():
    inp = synth.make_inputs("lstm", 1, 40, 2, seed=1024)
    plain = oracle.Problem("lstm", inp.pre, inp.w, inp.bias)
    for cu in ([0, 40], [0, 0, 40, 40], None):
        p = oracle.Problem("lstm", inp.pre, inp.w, inp.bias, cu_seqlens=cu)
        np.testing.assert_array_equal(oracle.newton(p, 3)[0], oracle.newton(plain, 3)[0])
