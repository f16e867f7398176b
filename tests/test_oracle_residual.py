"""Pins for the oracle's residual maximum R = max |F(H)_t| and the divergence rule built on it.

F(H)_t = h_t - f(h_{t-1}, x_t) is the system the method solves (pararnn-torch README, "Method"); its
largest component, over every batch row, step, channel and state component, is what tolerance mode
compares with tol, what the report carries, and what a divergence error hands back with its history
(same page, "Evaluation").  The oracle computes R in two places (``oracle.residual`` and the history of
``oracle.newton``); both are checked here against F built outside the oracle: the torch library cells
(``torch.nn.GRUCell`` / ``LSTMCell`` under the diagonal mapping, a block-diagonal ``GRUCell`` for the
head GRU, a torch sLSTM step, plain tensor ops for the linear cell) applied to the shifted trajectory, at
trajectories that solve nothing, and at the iterates of dense Newton on the stacked system.
"""
import numpy as np
import pytest
import torch

import oracle
from nonlinear_rnn_solve_amd import synth
from test_oracle_cells import torch_gru_cell, torch_lstm_cell
from test_oracle_head_gru import head_inputs, torch_head_cell
from test_oracle_newton import dense_F, dense_newton
from test_oracle_slstm import torch_slstm_step


@pytest.fixture(autouse=True)
def _fp64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def F_torch(inp, H, s0=None, starts=()):
    """F(H) [S][B][T][D] from torch cells, step by step (the previous state of step 0 is s0, of a packed
    sequence's first step the zero state)."""
    S, B, T, D = inp.S, inp.B, inp.T, inp.D
    pre = [torch.tensor(p.astype(np.float64)) for p in inp.pre_f32()]
    Ht = torch.tensor(np.asarray(H, np.float64).reshape(S, B, T, D))
    s0t = torch.zeros(S, B, D) if s0 is None else torch.tensor(s0.astype(np.float64))
    w, bias = (None, None) if inp.w is None else (inp.w.astype(np.float64), inp.bias.astype(np.float64))
    if inp.cell == "gru":
        cell = torch_gru_cell(w, bias)
        step = lambda x, s: cell(x, s[0])[None]                                   # noqa: E731
    elif inp.cell == "lstm":
        cell = torch_lstm_cell(w, bias)

        def step(x, s):
            h2, c2 = cell(x, (s[1], s[0]))
            return torch.stack([c2, h2])
    elif inp.cell == "slstm":
        st = torch_slstm_step(w, bias)
        step = lambda x, s: torch.stack(st(x, tuple(s)))                          # noqa: E731
    elif inp.cell == "head_gru":
        cell = torch_head_cell(inp.w, inp.bias)
        step = lambda x, s: cell(x, s[0])[None]                                   # noqa: E731
    else:
        step = lambda x, s: (x[:, :D] * s[0] + x[:, D:])[None]                    # noqa: E731
    out = []
    with torch.no_grad():
        for t in range(T):
            prev = s0t if t == 0 else (torch.zeros_like(s0t) if t in starts else Ht[:, :, t - 1, :])
            x = torch.cat([p[:, t, :] for p in pre], 1)
            out.append(Ht[:, :, t, :] - step(x, prev))
    return torch.stack(out, 2).numpy()


def problem(inp, s0=None, cu_seqlens=None):
    return oracle.Problem(inp.cell, inp.pre, inp.w, inp.bias, s0=s0, cu_seqlens=cu_seqlens,
                          head_size=getattr(inp, "head_size", None),
                          dtype=oracle.BF16 if inp.dtype == "bf16" else oracle.F32)


def random_trajectory(inp, seed):
    rng = np.random.default_rng(seed)
    H = rng.normal(0.0, 0.7, (inp.S, inp.B, inp.T, inp.D))
    if inp.cell == "slstm":
        H[1] = np.abs(H[1]) + 0.5          # a positive normaliser n
    return H


@pytest.mark.parametrize("cell,dtype,hs", [("gru", "f32", None), ("gru", "bf16", None), ("lstm", "f32", None),
                                           ("slstm", "f32", None), ("linear", "f32", None),
                                           ("head_gru", "diag_c", 4), ("head_gru", "r_one", 4)])
def test_residual_is_the_largest_component_of_F(cell, dtype, hs):
    # head GRU: torch's GRUCell applies the reset gate after its recurrent matrix, so it is this cell where
    # the A_c blocks are diagonal (dense A_z, A_r) or where r == 1 (dense A_c)
    if cell == "head_gru":
        inp = head_inputs(dtype, 2, 29, 8, hs, seed=1060)
    else:
        inp = synth.make_inputs(cell, 2, 29, 8, dtype=dtype, seed=1060)
    s0 = synth.random_state(inp.S, 2, 8, seed=61)
    if cell == "slstm":
        s0[1] = np.abs(s0[1]) + 0.5
    prob = problem(inp, s0)
    for seed in (1, 2, 3):
        H = random_trajectory(inp, seed)
        want = np.abs(F_torch(inp, H, s0)).max()
        assert oracle.residual(prob, H) == pytest.approx(want, rel=1e-12)
    # at the sequential unroll F vanishes (to rounding) in every component
    assert oracle.residual(prob, oracle.unroll(prob)) <= 1e-12


def test_residual_covers_every_state_component_of_the_lstm():
    # the exact solution, spoiled in one component at one step: R is that component's deviation, and the
    # deviation of c must be seen as well as that of h (a residual over h alone would miss the first case)
    inp = synth.make_inputs("lstm", 2, 40, 6, seed=1061)
    prob = problem(inp)
    ref = oracle.unroll(prob)
    for comp, amp in ((0, 3.0), (1, 0.25)):
        H = ref.copy()
        H[comp, 1, 17, 4] += amp
        F = F_torch(inp, H)
        got = oracle.residual(prob, H)
        assert got == pytest.approx(np.abs(F).max(), rel=1e-12)
        assert got >= amp * (1 - 1e-12)
        # the largest term of F sits in the spoiled component at the spoiled step
        assert np.unravel_index(np.abs(F).argmax(), F.shape)[0] == comp


def test_residual_with_packed_sequences():
    inp = synth.make_inputs("gru", 2, 50, 4, seed=1062)
    cu = np.array([0, 13, 13, 30, 50], np.int32)
    s0 = synth.random_state(1, 2, 4, seed=62)
    prob = problem(inp, s0, cu_seqlens=cu)
    H = random_trajectory(inp, 4)
    assert oracle.residual(prob, H) == pytest.approx(np.abs(F_torch(inp, H, s0, starts=(13, 30))).max(), rel=1e-12)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_newton_history_is_the_residual_of_each_dense_newton_iterate(cell):
    inp = synth.make_inputs(cell, 1, 9, 3, seed=1063)
    s0 = synth.random_state(inp.S, 1, 3, seed=63)
    prob = problem(inp, s0)
    K = 4
    _, res, iters, _, rc = oracle.newton(prob, K)
    assert iters == K and rc == oracle.OK
    F = dense_F(inp, s0)
    for k in range(K):
        Hk = dense_newton(inp, s0, k) if k else np.zeros(prob.traj_shape())
        want = float(torch.abs(F(torch.tensor(Hk).reshape(-1))).max().detach())
        assert res[k] == pytest.approx(want, rel=1e-9, abs=1e-15), k


# ------------------------------------------------------------------------------------------------
# divergence: a solve that spends its budget and ends above the residual it started from
# ------------------------------------------------------------------------------------------------
def large_weights(cell, T, D, scale, seed):
    inp = synth.make_inputs(cell, 1, T, D, seed=seed)
    rng = np.random.default_rng(seed + 1)
    inp.w[:] = (rng.choice([-1.0, 1.0], inp.w.shape) * scale).astype(np.float32)
    return inp


def test_large_recurrent_weights_diverge_with_the_history():
    # recurrent weights of +-4: the Jacobians reach ~ |w|/4 > 1, the first update overshoots and, within a
    # budget of 6, the residual never comes back below where it started
    inp = large_weights("gru", 12, 4, 4.0, 1072)
    prob = problem(inp)
    H, res, iters, conv, rc = oracle.newton(prob, 6, tol=1e-5)
    assert rc == oracle.DIVERGED and iters == 6 and not conv
    assert res[-1] > res[0] and np.all(np.isfinite(res))
    # the history is the residual of dense Newton's iterates (built from the torch library cell)
    s0 = np.zeros((1, 1, 4), np.float32)
    F = dense_F(inp, s0)
    for k in range(6):
        Hk = dense_newton(inp, s0, k) if k else np.zeros(prob.traj_shape())
        assert res[k] == pytest.approx(float(torch.abs(F(torch.tensor(Hk).reshape(-1))).max().detach()), rel=1e-8), k
    # the same budget without a tolerance runs to the end and reports nothing
    _, res0, it0, _, rc0 = oracle.newton(prob, 6)
    assert rc0 == oracle.OK and it0 == 6
    np.testing.assert_array_equal(res0, res)


def test_weights_of_fifty_diverge():
    inp = large_weights("gru", 256, 8, 50.0, 1065)
    prob = problem(inp)
    _, res, iters, conv, rc = oracle.newton(prob, 6, tol=1e-5)
    assert rc == oracle.DIVERGED and not conv
    assert (not np.isfinite(res[-1])) or res[-1] > 1e30 * res[0]


def test_a_transient_rise_that_converges_is_not_divergence():
    # an LSTM solve from the zero guess whose first update raises the max residual (0.909 -> 1.16) and
    # which then converges: tolerance mode ends converged, with the rise in its history
    inp = synth.make_inputs("lstm", 1, 1024, 8, seed=1057)
    prob = problem(inp)
    _, res, iters, conv, rc = oracle.newton(prob, 8, tol=1e-5)
    assert rc == oracle.OK and conv and res[1] > res[0]


def test_a_budget_that_ends_below_the_start_is_not_divergence():
    inp = large_weights("gru", 12, 4, 4.0, 1064)
    prob = problem(inp)
    _, full, *_ = oracle.newton(prob, 6)
    K = int(np.argmax(full[1:] > full[0])) + 1           # an iteration above the start ...
    K_end = next(k for k in range(K, 6) if full[k] < full[0]) + 1   # ... and a later one below it
    _, res, iters, conv, rc = oracle.newton(prob, K_end, tol=1e-12)
    assert rc == oracle.OK and not conv and iters == K_end and max(res) > res[0] > res[-1]
    _, res2, iters2, _, rc2 = oracle.newton(prob, K + 1, tol=1e-12)
    assert rc2 == oracle.DIVERGED and iters2 == K + 1 and res2[-1] > res2[0]


def test_picard_sweeps_are_not_judged():
    # sLSTM: the divergence test compares with the residual at the first Newton iteration, after the sweeps
    inp = synth.make_inputs("slstm", 1, 1024, 8, seed=1067)
    prob = problem(inp)
    _, res, iters, conv, rc = oracle.newton(prob, 24, tol=1e-5, picard=8)
    assert rc == oracle.OK and conv
