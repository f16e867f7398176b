"""Pins for the oracle's VJP at a solved trajectory.

The backward pass follows the paper's adjoint equation (pararnn-torch README,
"Method"): a reverse linear recurrence with transposed Jacobians, then the gate
gradients.  At the exact solution this equals the gradient of the sequential
unroll, so torch autograd through the library cells (float64, CPU) is an
independent reference for every output: dU, dw, dbias, ds0 and lambda.
"""
import numpy as np
import pytest
import torch

import oracle
from nonlinear_rnn_solve_amd import synth
from test_oracle_cells import torch_gru_cell, torch_lstm_cell


@pytest.fixture(autouse=True)
def _fp64_default():
    # the torch reference cells here run in fp64; restore the default so other modules are unaffected
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def autograd_reference(inp, s0, g, starts=()):
    """Gradients of L = sum g * h through the sequential torch unroll.  starts: steps where a new
    packed sequence begins (the state entering them is replaced by zeros)."""
    B, T, D, S = inp.B, inp.T, inp.D, inp.S
    pre = [torch.tensor(p.astype(np.float64), requires_grad=True) for p in inp.pre_f32()]
    s0t = torch.tensor(s0.astype(np.float64), requires_grad=True)
    gt = torch.tensor(g.astype(np.float64))
    if inp.cell == "linear":
        a, b = pre
        h = s0t[0]
        hs = []
        for t in range(T):
            if t in starts:
                h = torch.zeros_like(h)
            h = a[:, t, :] * h + b[:, t, :]
            h.retain_grad()
            hs.append(h)
        loss = (torch.stack(hs, 1) * gt).sum()
        loss.backward()
        lam = np.stack([x.grad.numpy() for x in hs], 1)[None]
        return {"d_pre": np.stack([p.grad.numpy() for p in pre]), "d_s0": s0t.grad.numpy(), "lam": lam}
    # autograd through the torch library cell itself; the parameter gradients are read back
    # from its (diagonal) recurrent weight and input-bias gradients
    if inp.cell == "gru":
        cell = torch_gru_cell(inp.w.astype(np.float64), inp.bias.astype(np.float64))
        rows, sign = [1, 0, 2], [-1.0, 1.0, 1.0]       # our gate z, r, c -> torch row block, sign
    else:
        cell = torch_lstm_cell(inp.w.astype(np.float64), inp.bias.astype(np.float64))
        rows, sign = [0, 1, 3, 2], [1.0, 1.0, 1.0, 1.0]  # our gate i, f, o, g -> torch row block
    states = []
    if S == 1:
        h = s0t[0]
        for t in range(T):
            if t in starts:
                h = torch.zeros_like(h)
            h = cell(torch.cat([p[:, t, :] for p in pre], 1), h)
            h.retain_grad()
            states.append([h])
    else:
        c, h = s0t[0], s0t[1]
        for t in range(T):
            if t in starts:
                c, h = torch.zeros_like(c), torch.zeros_like(h)
            h, c = cell(torch.cat([p[:, t, :] for p in pre], 1), (h, c))
            c.retain_grad()
            h.retain_grad()
            states.append([c, h])
    loss = sum((states[t][S - 1] * gt[:, t]).sum() for t in range(T))
    loss.backward()
    Whh, bih = cell.weight_hh.grad.numpy(), cell.bias_ih.grad.numpy()
    d_w = np.stack([sign[g] * np.diag(Whh[rows[g] * D:(rows[g] + 1) * D]) for g in range(inp.G)])
    d_bias = np.stack([sign[g] * bih[rows[g] * D:(rows[g] + 1) * D] for g in range(inp.G)])
    lam = np.stack([np.stack([states[t][k].grad.numpy() for t in range(T)], 1) for k in range(S)])
    return {"d_pre": np.stack([p.grad.numpy() for p in pre]), "d_w": d_w,
            "d_bias": d_bias, "d_s0": s0t.grad.numpy(), "lam": lam}


@pytest.mark.parametrize("cell", ["linear", "gru", "lstm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_vjp_matches_autograd_of_unroll(cell, dtype):
    inp = synth.make_inputs(cell, 2, 29, 5, dtype=dtype, seed=1014, with_grad=True)
    s0 = synth.random_state(inp.S, 2, 5, seed=6)
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0,
                          dtype=oracle.BF16 if dtype == "bf16" else oracle.F32)
    traj = oracle.unroll(prob)
    got = oracle.vjp(prob, traj, inp.g)
    want = autograd_reference(inp, s0, inp.g)
    if cell == "lstm":
        # autograd's c_t.grad also follows h_t = o tanh(c_t) inside step t; the system adjoint
        # treats (c, h) as independent unknowns, so only lambda_h is the same quantity there
        # (lambda as a whole is pinned by the dense adjoint test below)
        want["lam"] = want["lam"][1:]
        got = dict(got, lam=got["lam"][1:])
    for k in want:
        np.testing.assert_allclose(got[k], want[k], rtol=1e-11, atol=1e-12, err_msg=k)


@pytest.mark.parametrize("cell", ["linear", "gru", "lstm"])
def test_lambda_solves_the_dense_adjoint_system(cell):
    # lambda is the multiplier of F(H) = 0:  (dF/dH)^T lambda = dL/dH = e_h g
    from test_oracle_newton import dense_F
    inp = synth.make_inputs(cell, 1, 6, 2, seed=1017, with_grad=True)
    s0 = synth.random_state(inp.S, 1, 2, seed=9)
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0)
    H = oracle.unroll(prob)
    F = dense_F(inp, s0)
    Jf = torch.autograd.functional.jacobian(F, torch.tensor(H.reshape(-1))).numpy()
    rhs = np.zeros(H.shape)
    rhs[inp.S - 1] = inp.g.astype(np.float64)
    lam = np.linalg.solve(Jf.T, rhs.reshape(-1)).reshape(H.shape)
    np.testing.assert_allclose(oracle.vjp(prob, H, inp.g)["lam"], lam, rtol=1e-11, atol=1e-12)


def test_vjp_finite_differences_through_unroll():
    # an independent second pin: central differences of L = sum g*h on a few entries
    inp = synth.make_inputs("gru", 1, 8, 2, seed=1015, with_grad=True)
    s0 = synth.random_state(1, 1, 2, seed=8)

    def loss(pre, w, bias, s0v):
        pr = oracle.Problem("gru", pre, w, bias, s0=s0v)
        return float((oracle.unroll(pr)[0] * inp.g.astype(np.float64)).sum())

    prob = oracle.Problem("gru", inp.pre, inp.w, inp.bias, s0=s0)
    got = oracle.vjp(prob, oracle.unroll(prob), inp.g)
    eps = 1e-3   # inputs are float32: perturb by a representable step and use a wide stencil
    for (g, t, d) in [(0, 3, 1), (1, 0, 0), (2, 7, 1)]:
        pp = [p.copy() for p in inp.pre]
        pm = [p.copy() for p in inp.pre]
        pp[g][0, t, d] += eps
        pm[g][0, t, d] -= eps
        fd = (loss(pp, inp.w, inp.bias, s0) - loss(pm, inp.w, inp.bias, s0)) / (
            float(pp[g][0, t, d]) - float(pm[g][0, t, d]))
        assert abs(fd - got["d_pre"][g, 0, t, d]) < 1e-5 * max(1, abs(fd))
    for g in range(3):
        wp, wm = inp.w.copy(), inp.w.copy()
        wp[g, 1] += eps
        wm[g, 1] -= eps
        fd = (loss(inp.pre, wp, inp.bias, s0) - loss(inp.pre, wm, inp.bias, s0)) / (float(wp[g, 1]) - float(wm[g, 1]))
        assert abs(fd - got["d_w"][g, 1]) < 1e-5 * max(1, abs(fd))


def test_linear_scan_adjoint_closed_form():
    # db_s = sum_{t>=s} g_t prod_{u=s+1}^{t} a_u
    inp = synth.make_inputs("linear", 1, 15, 3, seed=1016, with_grad=True)
    a, b = inp.pre
    prob = oracle.Problem("linear", inp.pre)
    got = oracle.vjp(prob, oracle.unroll(prob), inp.g)
    a64, g64 = a.astype(np.float64), inp.g.astype(np.float64)
    for s in range(15):
        want = sum(g64[0, t] * np.prod(a64[0, s + 1: t + 1], axis=0) for t in range(s, 15))
        np.testing.assert_allclose(got["d_pre"][1, 0, s], want, rtol=1e-12)
