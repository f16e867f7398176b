"""Pins for the oracle's head-wise block GRU (pararnn-torch README, "Usage": the Dreamer-style
ParaGRU in its head-wise mixing mode, whose recurrent matrices are block-diagonal; "News": its
factorized Newton).

The oracle's cell applies the reset gate before the candidate's matrix, c = tanh(U_c + A_c (r*h) + b_c),
with one dense block per head.  torch.nn.GRUCell applies it after, r * (W_hn h); the two agree
exactly when A_c's blocks are diagonal or when r == 1.  The library-cell pins use those two cases:
the first covers the dense A_z and A_r blocks, the second the dense A_c blocks.  The general cell is
covered by central differences of the step, by two reductions to the diagonal GRU (head size 1;
diagonal blocks), whose oracle is pinned to torch on its own, and by what any correct Newton solve
does (dense Newton on the stacked system, triangular exactness, agreement with the unroll).
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


def head_inputs(config, B, T, D, hs, seed, with_grad=False, dtype="f32"):
    """Seeded head-GRU inputs.  config: "general" (as drawn), "diag_c" (A_c blocks made diagonal) or
    "r_one" (U_r raised by 60 so that r == 1 in fp64 whatever A_r h is)."""
    inp = synth.make_inputs("head_gru", B, T, D, dtype=dtype, seed=seed, with_grad=with_grad, head_size=hs)
    if config == "diag_c":
        eye = np.eye(hs, dtype=np.float32)
        inp.w[2] = inp.w[2] * eye[None]
    elif config == "r_one":
        assert dtype == "f32"
        inp.pre[1] = (inp.pre[1] + np.float32(60.0)).astype(np.float32)
    return inp


def problem(inp, s0=None, cu_seqlens=None):
    return oracle.Problem("head_gru", inp.pre, inp.w, inp.bias, s0=s0, head_size=inp.head_size,
                          dtype=oracle.BF16 if inp.dtype == "bf16" else oracle.F32, cu_seqlens=cu_seqlens)


def torch_head_cell(w, bias):
    """torch.nn.GRUCell with block-diagonal recurrent weights; input x_t = [U_z, U_r, U_c].  torch's
    update gate is 1 - z here, so its z rows carry -U_z, -A_z and -b_z."""
    G, H, hs, _ = w.shape
    D = H * hs
    cell = torch.nn.GRUCell(3 * D, D, bias=True)
    I, Z = torch.eye(D), torch.zeros(D, D)
    Az, Ar, Ac = [torch.block_diag(*[torch.tensor(w[g, h].astype(np.float64)) for h in range(H)]) for g in range(3)]
    b = torch.tensor(bias.astype(np.float64))
    with torch.no_grad():
        # rows [r; z; n], columns [U_z, U_r, U_c]
        cell.weight_ih.copy_(torch.cat([torch.cat([Z, I, Z], 1), torch.cat([-I, Z, Z], 1), torch.cat([Z, Z, I], 1)], 0))
        cell.bias_ih.copy_(torch.cat([b[1], -b[0], b[2]]))
        cell.weight_hh.copy_(torch.cat([Ar, -Az, Ac], 0))
        cell.bias_hh.zero_()
    return cell


def torch_unroll(inp, s0=None, starts=(), grad=False):
    """Sequential unroll with the torch cell; returns (h [B][T][D] tensor list, pre leaves, s0 leaf, cell)."""
    B, T, D = inp.B, inp.T, inp.D
    pre = [torch.tensor(p.astype(np.float64), requires_grad=grad) for p in inp.pre_f32()]
    s0t = torch.tensor((np.zeros((1, B, D)) if s0 is None else s0).astype(np.float64), requires_grad=grad)
    cell = torch_head_cell(inp.w, inp.bias)
    h = s0t[0]
    hs = []
    for t in range(T):
        if t in starts:
            h = torch.zeros_like(h)
        h = cell(torch.cat([p[:, t, :] for p in pre], 1), h)
        if grad:
            h.retain_grad()
        hs.append(h)
    return hs, pre, s0t, cell


def to_blocks(M, H, hs):
    """[D][D] block-diagonal matrix -> its diagonal blocks [H][hs][hs]."""
    return np.stack([M[h * hs:(h + 1) * hs, h * hs:(h + 1) * hs] for h in range(H)])


# ------------------------------------------------------------------------------------------------
# the cell
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("config", ["diag_c", "r_one"])
def test_unroll_matches_torch_gru_cell(config):
    inp = head_inputs(config, 2, 9, 12, 4, seed=2001)
    s0 = synth.random_state(1, 2, 12, seed=11)
    ref = torch.stack(torch_unroll(inp, s0)[0], 1).detach().numpy()
    got = oracle.unroll(problem(inp, s0))[0]
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("config", ["diag_c", "r_one"])
def test_the_library_pin_sees_a_transposed_block(config):
    # the comparison above is sensitive to the orientation of the dense blocks it covers
    inp = head_inputs(config, 1, 6, 8, 4, seed=2002)
    ref = torch.stack(torch_unroll(inp)[0], 1).detach().numpy()
    g = 0 if config == "diag_c" else 2       # a block that is dense in this configuration
    inp.w[g] = np.ascontiguousarray(np.swapaxes(inp.w[g], 1, 2))
    assert np.abs(oracle.unroll(problem(inp))[0] - ref).max() > 1e-4


def test_head_size_one_is_the_diagonal_gru():
    diag = synth.make_inputs("gru", 2, 30, 6, seed=2003, with_grad=True)
    s0 = synth.random_state(1, 2, 6, seed=12)
    w = diag.w.reshape(3, 6, 1, 1)
    hp = oracle.Problem("head_gru", diag.pre, w, diag.bias, s0=s0, head_size=1)
    dp = oracle.Problem("gru", diag.pre, diag.w, diag.bias, s0=s0)
    np.testing.assert_allclose(oracle.unroll(hp), oracle.unroll(dp), rtol=0, atol=1e-15)
    for warm in (False, True):
        Hh, rh, *_ = oracle.newton(hp, 3, warm=warm)
        Hd, rd, *_ = oracle.newton(dp, 3, warm=warm)
        np.testing.assert_allclose(Hh, Hd, rtol=0, atol=1e-14)
        np.testing.assert_allclose(rh, rd, rtol=1e-13)
    traj = oracle.unroll(dp)
    vh, vd = oracle.vjp(hp, traj, diag.g), oracle.vjp(dp, traj, diag.g)
    for k in ("d_pre", "d_bias", "d_s0", "lam"):
        np.testing.assert_allclose(vh[k], vd[k], rtol=1e-13, atol=1e-14, err_msg=k)
    np.testing.assert_allclose(vh["d_w"].reshape(3, 6), vd["d_w"], rtol=1e-13, atol=1e-14)


def test_diagonal_blocks_are_the_diagonal_gru():
    # pins which channels a head owns and where its block sits in w
    D, hs = 12, 4
    diag = synth.make_inputs("gru", 1, 25, D, seed=2004, with_grad=True)
    w = np.zeros((3, D // hs, hs, hs), np.float32)
    for g in range(3):
        for h in range(D // hs):
            w[g, h] = np.diag(diag.w[g, h * hs:(h + 1) * hs])
    hp = oracle.Problem("head_gru", diag.pre, w, diag.bias, head_size=hs)
    dp = oracle.Problem("gru", diag.pre, diag.w, diag.bias)
    np.testing.assert_allclose(oracle.unroll(hp), oracle.unroll(dp), rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.newton(hp, 2)[0], oracle.newton(dp, 2)[0], rtol=0, atol=1e-14)
    traj = oracle.unroll(dp)
    vh, vd = oracle.vjp(hp, traj, diag.g), oracle.vjp(dp, traj, diag.g)
    np.testing.assert_allclose(vh["d_pre"], vd["d_pre"], rtol=1e-13, atol=1e-14)
    got_diag = np.stack([np.concatenate([np.diag(vh["d_w"][g, h]) for h in range(D // hs)]) for g in range(3)])
    np.testing.assert_allclose(got_diag, vd["d_w"], rtol=1e-13, atol=1e-14)


def test_step_derivatives_by_central_differences():
    rng = np.random.default_rng(7)
    hs = 5
    A = rng.uniform(-0.6, 0.6, (3, hs, hs))
    u, bias, h = rng.standard_normal((3, hs)), 0.1 * rng.standard_normal((3, hs)), 0.7 * rng.standard_normal(hs)
    hn, J, dz, dc, dr, rh = oracle.hgru_step(u, A, bias, h)
    eps = 1e-6

    def f(u_=u, A_=A, h_=h):
        return oracle.hgru_step(u_, A_, bias, h_)[0]

    Jfd = np.stack([(f(h_=h + eps * e) - f(h_=h - eps * e)) / (2 * eps) for e in np.eye(hs)], 1)
    np.testing.assert_allclose(J, Jfd, atol=1e-9)
    for g, want in ((0, np.diag(dz)), (1, dr), (2, np.diag(dc))):
        cols = []
        for k in range(hs):
            up, um = u.copy(), u.copy()
            up[g, k] += eps
            um[g, k] -= eps
            cols.append((f(u_=up) - f(u_=um)) / (2 * eps))
        np.testing.assert_allclose(np.stack(cols, 1), want, atol=1e-9, err_msg="gate %d" % g)
    # rh is the vector A_c multiplies: d h'_i / d A_c[i][j] = dc_i rh_j
    for i, j in ((0, 3), (4, 1), (2, 2)):
        Ap, Am = A.copy(), A.copy()
        Ap[2, i, j] += eps
        Am[2, i, j] -= eps
        np.testing.assert_allclose((f(A_=Ap)[i] - f(A_=Am)[i]) / (2 * eps), dc[i] * rh[j], atol=1e-9)


@pytest.mark.parametrize("config", ["diag_c", "r_one"])
def test_step_jacobian_matches_autograd_of_the_library_cell(config):
    inp = head_inputs(config, 1, 1, 8, 4, seed=2005)
    cell = torch_head_cell(inp.w, inp.bias)
    x = torch.cat([torch.tensor(p[:, 0, :].astype(np.float64)) for p in inp.pre_f32()], 1)
    h = torch.tensor(np.random.default_rng(3).standard_normal((1, 8)) * 0.6)
    Jt = torch.autograd.functional.jacobian(lambda v: cell(x, v[None])[0], h[0]).numpy()
    for head in range(2):
        sl = slice(4 * head, 4 * head + 4)
        u = np.stack([p[0, 0, sl] for p in inp.pre_f32()])
        _, J, *_ = oracle.hgru_step(u, inp.w[:, head], inp.bias[:, sl], h[0, sl].numpy())
        np.testing.assert_allclose(J, Jt[sl, sl], rtol=1e-12, atol=1e-13)
        other = np.delete(np.arange(8), np.arange(4 * head, 4 * head + 4))
        assert np.abs(Jt[sl][:, other]).max() == 0.0     # heads do not interact


# ------------------------------------------------------------------------------------------------
# Newton
# ------------------------------------------------------------------------------------------------
def dense_newton(inp, s0, K, starts=()):
    """Newton on the stacked system, F from the torch cell, its Jacobian by autograd, each step by
    numpy.linalg.solve; returns the K-th iterate [1][B][T][D]."""
    B, T, D = inp.B, inp.T, inp.D
    pre = [torch.tensor(p.astype(np.float64)) for p in inp.pre_f32()]
    s0t = torch.tensor(s0.astype(np.float64))
    cell = torch_head_cell(inp.w, inp.bias)

    def F(flat):
        Hm = flat.reshape(B, T, D)
        out = []
        for t in range(T):
            prev = s0t[0] if t == 0 else (torch.zeros_like(s0t[0]) if t in starts else Hm[:, t - 1])
            out.append(Hm[:, t] - cell(torch.cat([p[:, t, :] for p in pre], 1), prev))
        return torch.stack(out, 1).reshape(-1)

    Hv = torch.zeros(B * T * D)
    for _ in range(K):
        Jf = torch.autograd.functional.jacobian(F, Hv).numpy()
        Hv = Hv - torch.tensor(np.linalg.solve(Jf, F(Hv).detach().numpy()))
    return Hv.reshape(1, B, T, D).numpy()


@pytest.mark.parametrize("K", [1, 2, 3])
def test_newton_iterates_match_dense_newton(K):
    inp = head_inputs("diag_c", 1, 5, 8, 4, seed=2006)
    s0 = synth.random_state(1, 1, 8, seed=13)
    H, res, iters, conv, rc = oracle.newton(problem(inp, s0), K)
    assert iters == K and rc == oracle.OK
    np.testing.assert_allclose(H, dense_newton(inp, s0, K), rtol=1e-11, atol=1e-12)


def test_newton_iterates_match_dense_newton_across_sequence_starts():
    inp = head_inputs("diag_c", 1, 7, 8, 4, seed=2007)
    s0 = synth.random_state(1, 1, 8, seed=14)
    cu = np.array([0, 3, 7], np.int32)
    H = oracle.newton(problem(inp, s0, cu_seqlens=cu), 2)[0]
    np.testing.assert_allclose(H, dense_newton(inp, s0, 2, starts=(3,)), rtol=1e-11, atol=1e-12)


def test_newton_triangular_exactness_general_cell():
    inp = head_inputs("general", 2, 10, 16, 8, seed=2008)
    prob = problem(inp, synth.random_state(1, 2, 16, seed=15))
    ref = oracle.unroll(prob)
    for k in (1, 4):
        H = oracle.newton(prob, k)[0]
        np.testing.assert_allclose(H[:, :, :k], ref[:, :, :k], atol=1e-13)
        if k == 1:
            assert np.abs(H[:, :, k:] - ref[:, :, k:]).max() > 1e-6   # not yet exact further on
    np.testing.assert_allclose(oracle.newton(prob, 10)[0], ref, atol=1e-13)
    # from a random first iterate as well
    guess = np.random.default_rng(2).standard_normal(prob.traj_shape()).astype(np.float32)
    np.testing.assert_allclose(oracle.newton(prob, 3, init_guess=guess)[0][:, :, :3], ref[:, :, :3], atol=1e-13)


def test_newton_converges_quadratically_to_the_unroll():
    inp = head_inputs("general", 2, 64, 128, 32, seed=2009)
    prob = problem(inp)
    H, res, iters, conv, rc = oracle.newton(prob, 12, tol=1e-12)
    assert conv and rc == oracle.OK and iters <= 7, res
    small = [k for k in range(len(res) - 1) if res[k] < 0.05 and res[k + 1] > 1e-14]
    assert small and all(res[k + 1] < 20.0 * res[k] ** 2 for k in small), res
    np.testing.assert_allclose(H, oracle.unroll(prob), atol=1e-11)
    assert oracle.residual(prob, H) < 1e-12


def test_warm_start_is_the_cell_at_a_zero_state():
    inp = head_inputs("diag_c", 2, 12, 8, 4, seed=2010)
    cell = torch_head_cell(inp.w, inp.bias)
    x = torch.cat([torch.tensor(p.astype(np.float64)) for p in inp.pre_f32()], 2).reshape(24, -1)
    f0 = cell(x, torch.zeros(24, 8)).detach().numpy().reshape(1, 2, 12, 8).astype(np.float32)
    prob = problem(inp)
    for K in (1, 2):
        np.testing.assert_allclose(oracle.newton(prob, K, warm=True)[0], oracle.newton(prob, K, init_guess=f0)[0],
                                   atol=1e-6)


def test_tolerance_rule_and_divergence():
    inp = head_inputs("general", 1, 40, 16, 8, seed=2011)
    prob = problem(inp)
    _, full, *_ = oracle.newton(prob, 8)
    tol = 1e-6
    H, res, iters, conv, rc = oracle.newton(prob, 8, tol=tol)
    assert conv and iters == int(np.argmax(full < tol)) + 1
    np.testing.assert_array_equal(H, oracle.newton(prob, iters)[0])
    inp.pre[2][0, 7, 3] = np.nan
    _, res, iters, conv, rc = oracle.newton(problem(inp), 5, tol=1e-5)
    assert rc == oracle.DIVERGED and iters == 1 and np.isnan(res[0])


# ------------------------------------------------------------------------------------------------
# VJP
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("config", ["diag_c", "r_one"])
def test_vjp_matches_autograd_of_the_library_unroll(config):
    B, T, D, hs = 2, 11, 8, 4
    inp = head_inputs(config, B, T, D, hs, seed=2012, with_grad=True)
    s0 = synth.random_state(1, B, D, seed=16)
    hs_list, pre, s0t, cell = torch_unroll(inp, s0, grad=True)
    gt = torch.tensor(inp.g.astype(np.float64))
    (torch.stack(hs_list, 1) * gt).sum().backward()
    prob = problem(inp, s0)
    traj = oracle.unroll(prob)
    got = oracle.vjp(prob, traj, inp.g)
    np.testing.assert_allclose(got["d_pre"], np.stack([p.grad.numpy() for p in pre]), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["d_s0"], s0t.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["lam"][0], np.stack([h.grad.numpy() for h in hs_list], 1), rtol=1e-11, atol=1e-12)
    Wg, bg = cell.weight_hh.grad.numpy(), cell.bias_ih.grad.numpy()
    H = D // hs
    np.testing.assert_allclose(got["d_w"][0], to_blocks(-Wg[D:2 * D], H, hs), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["d_w"][1], to_blocks(Wg[0:D], H, hs), rtol=1e-11, atol=1e-12)
    dAc = to_blocks(Wg[2 * D:], H, hs)
    if config == "r_one":
        np.testing.assert_allclose(got["d_w"][2], dAc, rtol=1e-11, atol=1e-12)
    else:   # torch's r * (W h) and A_c (r * h) share only the diagonal's derivative
        np.testing.assert_allclose(np.diagonal(got["d_w"][2], axis1=1, axis2=2),
                                   np.diagonal(dAc, axis1=1, axis2=2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["d_bias"], np.stack([-bg[D:2 * D], bg[:D], bg[2 * D:]]), rtol=1e-11, atol=1e-12)


def test_vjp_matches_autograd_across_sequence_starts():
    B, T, D, hs = 1, 12, 8, 4
    inp = head_inputs("diag_c", B, T, D, hs, seed=2013, with_grad=True)
    s0 = synth.random_state(1, B, D, seed=17)
    cu = np.array([0, 4, 4, 9, 12], np.int32)
    hs_list, pre, s0t, cell = torch_unroll(inp, s0, starts=(4, 9), grad=True)
    (torch.stack(hs_list, 1) * torch.tensor(inp.g.astype(np.float64))).sum().backward()
    prob = problem(inp, s0, cu_seqlens=cu)
    got = oracle.vjp(prob, oracle.unroll(prob), inp.g)
    np.testing.assert_allclose(got["d_pre"], np.stack([p.grad.numpy() for p in pre]), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["d_s0"], s0t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_vjp_central_differences_general_cell():
    B, T, D, hs = 1, 7, 6, 3
    inp = head_inputs("general", B, T, D, hs, seed=2014, with_grad=True)
    s0 = synth.random_state(1, B, D, seed=18)
    g64 = inp.g.astype(np.float64)

    def loss(pre=None, w=None, bias=None, s0v=None):
        pr = oracle.Problem("head_gru", inp.pre if pre is None else pre, inp.w if w is None else w,
                            inp.bias if bias is None else bias, s0=s0 if s0v is None else s0v, head_size=hs)
        return float((oracle.unroll(pr)[0] * g64).sum())

    got = oracle.vjp(problem(inp, s0), oracle.unroll(problem(inp, s0)), inp.g)
    eps = 1e-3   # float32 inputs: perturb by a representable step, divide by the actual step

    def fd(arr, idx, kw):
        ap, am = arr.copy(), arr.copy()
        ap[idx] += eps
        am[idx] -= eps
        return (loss(**{kw: ap}) - loss(**{kw: am})) / (float(ap[idx]) - float(am[idx]))

    for g in range(3):
        for (t, d) in ((0, 1), (3, 5), (6, 2)):
            pre = [p.copy() for p in inp.pre]
            pp, pm = [p.copy() for p in pre], [p.copy() for p in pre]
            pp[g][0, t, d] += eps
            pm[g][0, t, d] -= eps
            want = (loss(pre=pp) - loss(pre=pm)) / (float(pp[g][0, t, d]) - float(pm[g][0, t, d]))
            assert abs(want - got["d_pre"][g, 0, t, d]) < 1e-5 * max(1.0, abs(want)), (g, t, d)
        for idx in ((g, 0, 0, 2), (g, 1, 2, 0), (g, 1, 1, 1)):
            want = fd(inp.w, idx, "w")
            assert abs(want - got["d_w"][idx]) < 1e-5 * max(1.0, abs(want)), idx
        want = fd(inp.bias, (g, 4), "bias")
        assert abs(want - got["d_bias"][g, 4]) < 1e-5 * max(1.0, abs(want))
    for d in (0, 5):
        want = fd(s0, (0, 0, d), "s0v")
        assert abs(want - got["d_s0"][0, 0, d]) < 1e-5 * max(1.0, abs(want))


def test_lambda_solves_the_stacked_adjoint_system_general_cell():
    # (dF/dH)^T lambda = g with dF/dH = I - (sub-diagonal blocks J_t), the blocks from the (pinned)
    # step Jacobian
    B, T, D, hs = 1, 6, 8, 4
    inp = head_inputs("general", B, T, D, hs, seed=2015, with_grad=True)
    prob = problem(inp)
    H = oracle.unroll(prob)[0, 0]
    n = T * D
    M = np.eye(n)
    for t in range(1, T):
        for head in range(D // hs):
            sl = slice(head * hs, (head + 1) * hs)
            u = np.stack([p[0, t, sl] for p in inp.pre_f32()])
            _, J, *_ = oracle.hgru_step(u, inp.w[:, head], inp.bias[:, sl], H[t - 1, sl])
            M[t * D + head * hs: t * D + (head + 1) * hs, (t - 1) * D + head * hs: (t - 1) * D + (head + 1) * hs] -= J
    lam = np.linalg.solve(M.T, inp.g.astype(np.float64).reshape(-1)).reshape(T, D)
    got = oracle.vjp(prob, oracle.unroll(prob), inp.g)["lam"][0, 0]
    np.testing.assert_allclose(got, lam, rtol=1e-11, atol=1e-12)


def test_packed_unroll_is_the_separate_unrolls():
    B, T, D, hs = 2, 20, 8, 4
    inp = head_inputs("general", B, T, D, hs, seed=2016)
    s0 = synth.random_state(1, B, D, seed=19)
    cu = np.array([0, 6, 6, 13, 20], np.int32)
    got = oracle.unroll(problem(inp, s0, cu_seqlens=cu))
    for j, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if a == b:
            continue
        sub = synth.Inputs("head_gru", B, int(b - a), D, "f32", [p[:, a:b].copy() for p in inp.pre], inp.w, inp.bias,
                           None, hs)
        want = oracle.unroll(problem(sub, s0 if a == 0 else None))
        np.testing.assert_allclose(got[:, :, a:b], want, rtol=0, atol=1e-15)
