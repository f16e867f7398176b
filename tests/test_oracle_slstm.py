"""Pins for the oracle's diagonal sLSTM cell and its Picard sweeps.

The pages name the cell (pararnn-torch README: ParaSLSTM with mix="diag", "API overview" and
"Method") but print no equations; the oracle follows the published sLSTM (exponential input
gate, sigmoid forget gate, normaliser state n and log-domain stabiliser m) with diagonal recurrent
weights acting on h.  What pins it:
  * the stabiliser changes nothing: the unstabilised recurrence c~ = f c~ + i z, n~ = f n~ + i
    (no m, no max) gives the same h and c~ = c e^m, n~ = n e^m -- a different computation of the
    same cell, evaluated here in numpy;
  * the hand-derived Jacobian and gate partials against central differences, on both sides of
    the stabiliser's max;
  * Newton iterates against dense Newton on the stacked system (torch autograd Jacobian, numpy
    solve), and the VJP against torch autograd through the sequential unroll;
  * Picard sweeps: one sweep is the cell applied to the shifted iterate; after P sweeps from any
    guess the first P steps are exact; Picard sweeps followed by Newton reach the unroll.
"""
import numpy as np
import pytest
import torch

import oracle
from nonlinear_rnn_solve_amd import synth


@pytest.fixture(autouse=True)
def _fp64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def unstabilised(inp, s0=None):
    """h, c~, n~ of the sLSTM without the stabiliser, in float64 numpy (short sequences only)."""
    U = [p.astype(np.float64) for p in inp.pre_f32()]
    w, b = inp.w.astype(np.float64), inp.bias.astype(np.float64)
    B, T, D = inp.B, inp.T, inp.D
    c = np.zeros((B, D)) if s0 is None else s0[0] * np.exp(s0[2])
    n = np.zeros((B, D)) if s0 is None else s0[1] * np.exp(s0[2])
    h = np.zeros((B, D)) if s0 is None else s0[3].copy()
    hs, cs, ns = [], [], []
    for t in range(T):
        u = [U[g][:, t] + w[g] * h + b[g] for g in range(4)]
        z, i, f, o = np.tanh(u[0]), np.exp(u[1]), 1 / (1 + np.exp(-u[2])), 1 / (1 + np.exp(-u[3]))
        c = f * c + i * z
        n = f * n + i
        h = o * c / n
        hs.append(h); cs.append(c); ns.append(n)
    return np.stack(hs, 1), np.stack(cs, 1), np.stack(ns, 1)


def test_stabiliser_changes_nothing():
    inp = synth.make_inputs("slstm", 2, 30, 5, seed=1030)
    s0 = synth.random_state(4, 2, 5, seed=40)
    s0[1] = np.abs(s0[1]) + 0.5                     # a positive normaliser
    prob = oracle.Problem("slstm", inp.pre, inp.w, inp.bias, s0=s0)
    H = oracle.unroll(prob)
    h, c, n = unstabilised(inp, s0.astype(np.float64))
    np.testing.assert_allclose(H[3], h, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(H[0] * np.exp(H[2]), c, rtol=1e-11)
    np.testing.assert_allclose(H[1] * np.exp(H[2]), n, rtol=1e-11)
    # the stabiliser is the running maximum of the log-domain gates
    assert np.all(H[1] > 0) and np.all(np.isfinite(H))


@pytest.mark.parametrize("branch", ["forget", "input"])
def test_jacobian_and_gate_partials_by_central_differences(branch):
    rng = np.random.default_rng(1031)
    w = rng.uniform(-0.5, 0.5, 4)
    bias = rng.normal(0, 0.1, 4)
    for trial in range(20):
        u = rng.normal(0, 1, 4)
        s = np.array([rng.normal(), abs(rng.normal()) + 0.3, rng.normal(), rng.normal()])
        # put the max of the stabiliser clearly on one side
        lf = -np.log1p(np.exp(-(u[2] + w[2] * s[3] + bias[2])))
        ui = u[1] + w[1] * s[3] + bias[1]
        s[2] = ui - lf + (2.0 if branch == "forget" else -2.0)
        sn, J, dfdu, wc = oracle.cell_step("slstm", u, w, bias, s)
        eps = 1e-6
        for j in range(4):
            sp, sm = s.copy(), s.copy()
            sp[j] += eps
            sm[j] -= eps
            fd = (oracle.cell_step("slstm", u, w, bias, sp)[0] - oracle.cell_step("slstm", u, w, bias, sm)[0]) / (2 * eps)
            np.testing.assert_allclose(J[:, j], fd, rtol=1e-6, atol=1e-8)
        for g in range(4):
            up, um = u.copy(), u.copy()
            up[g] += eps
            um[g] -= eps
            fd = (oracle.cell_step("slstm", up, w, bias, s)[0] - oracle.cell_step("slstm", um, w, bias, s)[0]) / (2 * eps)
            np.testing.assert_allclose(dfdu[:, g], fd, rtol=1e-6, atol=1e-8)
        np.testing.assert_array_equal(wc, [s[3]] * 4)


def torch_slstm_step(w, b):
    """The stabilised cell in torch (float64), for autograd-based references."""
    w, b = torch.tensor(w), torch.tensor(b)

    def step(x, state):
        c, n, m, h = state
        D = h.shape[-1]
        u = [x[..., g * D:(g + 1) * D] + w[g] * h + b[g] for g in range(4)]
        z, o = torch.tanh(u[0]), torch.sigmoid(u[3])
        lf = torch.nn.functional.logsigmoid(u[2])
        m2 = torch.maximum(lf + m, u[1])
        ip, fp = torch.exp(u[1] - m2), torch.exp(lf + m - m2)
        c2 = fp * c + ip * z
        n2 = fp * n + ip
        return c2, n2, m2, o * c2 / n2
    return step


def dense_newton_slstm(inp, s0, K, picard=0):
    B, T, D, S = inp.B, inp.T, inp.D, 4
    pre = [torch.tensor(p.astype(np.float64)) for p in inp.pre_f32()]
    step = torch_slstm_step(inp.w.astype(np.float64), inp.bias.astype(np.float64))
    s0t = torch.tensor(s0.astype(np.float64))

    def F(flat):
        H = flat.reshape(S, B, T, D)
        out = []
        for t in range(T):
            prev = s0t if t == 0 else H[:, :, t - 1, :]
            f = torch.stack(step(torch.cat([p[:, t, :] for p in pre], 1), tuple(prev)))
            out.append(H[:, :, t, :] - f)
        return torch.stack(out, 2).reshape(-1)

    H = torch.zeros(S * B * T * D)
    for k in range(K):
        r = F(H).detach()
        if k < picard:
            H = H - r
        else:
            Jf = torch.autograd.functional.jacobian(F, H).numpy()
            H = H - torch.tensor(np.linalg.solve(Jf, r.numpy()))
    return H.reshape(S, B, T, D).numpy()


@pytest.mark.parametrize("K,picard", [(1, 0), (2, 0), (3, 1), (4, 2)])
def test_iterates_match_dense_newton(K, picard):
    inp = synth.make_inputs("slstm", 1, 6, 2, seed=1032)
    s0 = synth.random_state(4, 1, 2, seed=41)
    s0[1] = np.abs(s0[1]) + 0.5
    prob = oracle.Problem("slstm", inp.pre, inp.w, inp.bias, s0=s0)
    H = oracle.newton(prob, K, picard=picard)[0]
    np.testing.assert_allclose(H, dense_newton_slstm(inp, s0, K, picard), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("cell", ["gru", "lstm", "slstm"])
def test_picard_sweeps(cell):
    inp = synth.make_inputs(cell, 2, 40, 3, seed=1033)
    prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias)
    ref = oracle.unroll(prob)
    S = inp.S
    guess = np.random.default_rng(2).standard_normal((S, 2, 40, 3)).astype(np.float32)
    if cell == "slstm":
        guess[1] = np.abs(guess[1]) + 0.5
    # one sweep: the cell applied to the shifted guess (s0 = 0 before the first step)
    H1 = oracle.newton(prob, 1, init_guess=guess, picard=1)[0]
    g64 = guess.astype(np.float64)
    U = [p.astype(np.float64) for p in inp.pre_f32()]
    for b in range(2):
        for t in (0, 1, 17, 39):
            for d in range(3):
                prev = np.zeros(S) if t == 0 else g64[:, b, t - 1, d]
                u = np.array([U[g][b, t, d] for g in range(inp.G)])
                sn = oracle.cell_step(cell, u, inp.w[:, d], inp.bias[:, d], prev)[0]
                np.testing.assert_allclose(H1[:, b, t, d], sn, rtol=1e-13, atol=1e-14)
    # after P sweeps from any guess the first P steps are exact
    for P in (3, 7):
        HP = oracle.newton(prob, P, init_guess=guess, picard=P)[0]
        np.testing.assert_allclose(HP[:, :, :P], ref[:, :, :P], rtol=1e-12, atol=1e-13)
    # Picard sweeps, then Newton, reach the unroll
    H = oracle.newton(prob, 12, picard=4)[0]
    np.testing.assert_allclose(H, ref, rtol=1e-10, atol=1e-11)


def test_vjp_matches_autograd():
    inp = synth.make_inputs("slstm", 2, 17, 3, seed=1034, with_grad=True)
    s0 = synth.random_state(4, 2, 3, seed=42)
    s0[1] = np.abs(s0[1]) + 0.5
    prob = oracle.Problem("slstm", inp.pre, inp.w, inp.bias, s0=s0)
    traj = oracle.unroll(prob)
    got = oracle.vjp(prob, traj, inp.g)
    pre = [torch.tensor(p.astype(np.float64), requires_grad=True) for p in inp.pre_f32()]
    w = torch.tensor(inp.w.astype(np.float64), requires_grad=True)
    b = torch.tensor(inp.bias.astype(np.float64), requires_grad=True)
    s0t = torch.tensor(s0.astype(np.float64), requires_grad=True)
    state = tuple(s0t[k] for k in range(4))
    loss = 0.0
    hs = []
    for t in range(inp.T):
        c, n, m, h = state
        u = [pre[g][:, t] + w[g] * h + b[g] for g in range(4)]
        z, o = torch.tanh(u[0]), torch.sigmoid(u[3])
        lf = torch.nn.functional.logsigmoid(u[2])
        m2 = torch.maximum(lf + m, u[1])
        ip, fp = torch.exp(u[1] - m2), torch.exp(lf + m - m2)
        c2, n2 = fp * c + ip * z, fp * n + ip
        state = (c2, n2, m2, o * c2 / n2)
        state[3].retain_grad()
        hs.append(state[3])
        loss = loss + (state[3] * torch.tensor(inp.g[:, t].astype(np.float64))).sum()
    loss.backward()
    np.testing.assert_allclose(got["d_pre"], np.stack([p.grad.numpy() for p in pre]), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["d_w"], w.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["d_bias"], b.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["d_s0"], s0t.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["lam"][3], np.stack([x.grad.numpy() for x in hs], 1), rtol=1e-9, atol=1e-11)


def test_stabiliser_is_the_running_maximum_also_near_ties():
    # m' = max(log sig(u_f) + m, u_i) exactly, including within a hair of the tie (where only the
    # representation (c, n, m), not h, would notice a wrong branch)
    rng = np.random.default_rng(1035)
    w = np.zeros(4)
    bias = np.zeros(4)
    for trial in range(200):
        u = rng.normal(0, 1, 4)
        s = np.array([rng.normal(), abs(rng.normal()) + 0.3, rng.normal(), rng.normal()])
        lf = -np.log1p(np.exp(-u[2]))
        if trial % 2:
            u[1] = lf + s[2] + rng.choice([-1, 1]) * 10.0 ** rng.uniform(-9, -2)   # near the tie
        sn = oracle.cell_step("slstm", u, w, bias, s)[0]
        assert sn[2] == max(lf + s[2], u[1]) or abs(sn[2] - max(lf + s[2], u[1])) < 1e-14
        # exactly one of the two rescaled gates is 1
        ip, fp = np.exp(u[1] - sn[2]), np.exp(lf + s[2] - sn[2])
        assert max(ip, fp) == pytest.approx(1.0, abs=1e-14)
