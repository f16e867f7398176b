"""Pins for the oracle's cell step f, its Jacobian and its gate partials.

The cells:
  * diag GRU -- the benchmark statement of this project:
      z = sig(U_z + a_z h + b_z), r = sig(U_r + a_r h + b_r),
      c = tanh(U_c + a_c (r h) + b_c), h' = (1 - z) h + z c.
  * diag LSTM -- textbook LSTM without peepholes, diagonal recurrent weights on h
    (a reading: the pages name LSTM adaptations -- ParaRNN abstract, HF paper list --
    but print no equations).
Both reduce to library cells: torch.nn.GRUCell / LSTMCell with identity input
weights and diagonal recurrent weights (GRUCell's update gate weights the old
state, so its z-gate pre-activation is the negated one of the GRU above).  The
torch cells are evaluated in float64 on the CPU and share nothing with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from nonlinear_rnn_solve_amd import synth


@pytest.fixture(autouse=True)
def _fp64_default():
    # the torch reference cells here run in fp64; restore the default so other modules are unaffected
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def torch_gru_cell(w, bias):
    """torch.nn.GRUCell computing the diag GRU above; input x_t = [U_z, U_r, U_c]."""
    D = w.shape[1]
    cell = torch.nn.GRUCell(3 * D, D, bias=True)
    I, Z = torch.eye(D), torch.zeros(D, D)
    with torch.no_grad():
        # weight_ih rows: [r; z; n], columns [U_z, U_r, U_c]
        cell.weight_ih.copy_(torch.cat([torch.cat([Z, I, Z], 1), torch.cat([-I, Z, Z], 1), torch.cat([Z, Z, I], 1)], 0))
        cell.bias_ih.copy_(torch.cat([torch.tensor(bias[1]), -torch.tensor(bias[0]), torch.tensor(bias[2])]))
        cell.weight_hh.copy_(torch.cat([torch.diag(torch.tensor(w[1])), torch.diag(-torch.tensor(w[0])),
                                        torch.diag(torch.tensor(w[2]))], 0))
        cell.bias_hh.zero_()
    return cell


def torch_lstm_cell(w, bias):
    """torch.nn.LSTMCell computing the diag LSTM; input x_t = [U_i, U_f, U_o, U_g]."""
    D = w.shape[1]
    cell = torch.nn.LSTMCell(4 * D, D, bias=True)
    I, Z = torch.eye(D), torch.zeros(D, D)
    blocks = {0: [I, Z, Z, Z], 1: [Z, I, Z, Z], 2: [Z, Z, I, Z], 3: [Z, Z, Z, I]}   # our gate -> x slot
    order = [0, 1, 3, 2]   # torch rows: i, f, g, o  <- our gates i, f, g, o = 0, 1, 3, 2
    with torch.no_grad():
        cell.weight_ih.copy_(torch.cat([torch.cat(blocks[g], 1) for g in order], 0))
        cell.bias_ih.copy_(torch.cat([torch.tensor(bias[g]) for g in order]))
        cell.weight_hh.copy_(torch.cat([torch.diag(torch.tensor(w[g])) for g in order], 0))
        cell.bias_hh.zero_()
    return cell


def torch_unroll(inp, s0=None):
    """Sequential unroll with the torch library cell; returns [S][B][T][D] float64."""
    B, T, D = inp.B, inp.T, inp.D
    pre = [torch.tensor(p.astype(np.float64)) for p in inp.pre_f32()]
    w, bias = inp.w.astype(np.float64), inp.bias.astype(np.float64)
    if inp.cell == "gru":
        cell = torch_gru_cell(w, bias)
        h = torch.zeros(B, D) if s0 is None else torch.tensor(s0[0].astype(np.float64))
        out = []
        for t in range(T):
            h = cell(torch.cat([p[:, t, :] for p in pre], 1), h)
            out.append(h)
        return torch.stack(out, 1)[None].detach().numpy()
    cell = torch_lstm_cell(w, bias)
    c = torch.zeros(B, D) if s0 is None else torch.tensor(s0[0].astype(np.float64))
    h = torch.zeros(B, D) if s0 is None else torch.tensor(s0[1].astype(np.float64))
    cs, hs = [], []
    for t in range(T):
        h, c = cell(torch.cat([p[:, t, :] for p in pre], 1), (h, c))
        cs.append(c)
        hs.append(h)
    return np.stack([torch.stack(cs, 1).detach().numpy(), torch.stack(hs, 1).detach().numpy()])


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unroll_matches_torch_library_cell(cell, dtype):
    inp = synth.make_inputs(cell, 2, 37, 6, dtype=dtype, seed=1004)
    s0 = synth.random_state(inp.S, 2, 6, seed=77)
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, s0=s0,
                          dtype=oracle.BF16 if dtype == "bf16" else oracle.F32)
    got = oracle.unroll(prob)
    want = torch_unroll(inp, s0)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_gru_gate_roles_special_cases():
    # z -> 0 (b_z = -40): the state is carried unchanged;  z -> 1 with r -> 0: h_t = tanh(U_c + b_c)
    inp = synth.make_inputs("gru", 1, 20, 4, seed=5)
    s0 = np.full((1, 1, 4), 0.37, np.float32)
    bias = inp.bias.copy()
    bias[0] = -40.0
    h = oracle.unroll(oracle.Problem("gru", inp.pre, inp.w, bias, s0=s0))
    np.testing.assert_allclose(h[0, 0], np.full((20, 4), np.float32(0.37)), atol=1e-15)
    bias[0], bias[1] = 40.0, -40.0
    h = oracle.unroll(oracle.Problem("gru", inp.pre, inp.w, bias, s0=s0))
    want = np.tanh(inp.pre[2][0].astype(np.float64) + bias[2].astype(np.float64))
    np.testing.assert_allclose(h[0, 0], want, atol=1e-15)


def _fd(fun, x, eps=1e-6):
    cols = []
    for i in range(len(x)):
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        cols.append((fun(xp) - fun(xm)) / (2 * eps))
    return np.stack(cols, axis=-1)


@pytest.mark.parametrize("cell", ["linear", "gru", "lstm"])
def test_jacobian_and_gate_partials_finite_differences(cell):
    rng = np.random.default_rng(21)
    S, G = oracle.state_size(oracle.CELLS[cell]), oracle.gate_count(oracle.CELLS[cell])
    for _ in range(25):
        u = rng.standard_normal(G)
        w = rng.uniform(-0.5, 0.5, G) if cell != "linear" else np.zeros(G)
        b = rng.normal(0, 0.3, G) if cell != "linear" else np.zeros(G)
        s = rng.standard_normal(S) * 0.8
        sn, J, dfdu, wc = oracle.cell_step(cell, u, w, b, s)
        J_fd = _fd(lambda x: oracle.cell_step(cell, u, w, b, x)[0], s)
        U_fd = _fd(lambda x: oracle.cell_step(cell, x, w, b, s)[0], u)
        np.testing.assert_allclose(J, J_fd, atol=1e-8)
        np.testing.assert_allclose(dfdu, U_fd, atol=1e-8)
        if cell != "linear":
            W_fd = _fd(lambda x: oracle.cell_step(cell, u, x, b, s)[0], w)
            np.testing.assert_allclose(dfdu * wc[None, :], W_fd, atol=1e-8)
            B_fd = _fd(lambda x: oracle.cell_step(cell, u, w, x, s)[0], b)
            np.testing.assert_allclose(dfdu, B_fd, atol=1e-8)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_jacobian_matches_torch_autograd(cell):
    rng = np.random.default_rng(8)
    D = 3
    G = 3 if cell == "gru" else 4
    w = rng.uniform(-0.5, 0.5, (G, D))
    b = rng.normal(0, 0.1, (G, D))
    U = rng.standard_normal((G, D))
    s = rng.standard_normal((2 if cell == "lstm" else 1, D)) * 0.7
    x = torch.tensor(np.concatenate(list(U)))[None]
    if cell == "gru":
        tc = torch_gru_cell(w, b)
        Jt = torch.autograd.functional.jacobian(lambda h: tc(x, h[None])[0], torch.tensor(s[0])).numpy()
    else:
        tc = torch_lstm_cell(w, b)

        def f(v):
            h2, c2 = tc(x, (v[D:][None], v[:D][None]))
            return torch.cat([c2[0], h2[0]])
        Jt = torch.autograd.functional.jacobian(f, torch.tensor(np.concatenate([s[0], s[1]]))).numpy()
    S = s.shape[0]
    for d in range(D):
        _, J, _, _ = oracle.cell_step(cell, U[:, d], w[:, d], b[:, d], s[:, d])
        for i in range(S):
            for j in range(S):
                np.testing.assert_allclose(J[i, j], Jt[i * D + d, j * D + d], atol=1e-13)
