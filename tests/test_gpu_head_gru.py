"""GPU parity of the head-wise block GRU's Newton solve against the fp64 oracle, element by element.

Tolerance: max |got - ref| / max(1, |ref|) <= 1e-5, the fp32 bar of the other parity tests.  Each
Jacobian entry is an fp32 sum of up to 2 * 64 products (typical rounding ~sqrt(64) u |terms|,
u = 6e-8), and a chunk composes 16 such blocks whose norms are below 1, so an iterate carries a few
1e-7 of fp32 rounding (measured: <= 5e-7 on every case here); bf16 storage uses the same input bits
on both sides and so has the same bar.  Converged solves are also compared with the sequential
unroll at the same bar.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu
TOL = 1e-5


def announce(*a):
    print("[case]", *a, flush=True)


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def inputs(B, T, heads, hs, dtype="f32", seed=3000, with_grad=False):
    return synth.make_inputs("head_gru", B, T, heads * hs, dtype=dtype, seed=seed, with_grad=with_grad, head_size=hs)


def oprob(inp, s0=None, cu=None):
    return oracle.Problem("head_gru", inp.pre, inp.w, inp.bias, s0=s0, head_size=inp.head_size,
                          dtype=oracle.BF16 if inp.dtype == "bf16" else oracle.F32, cu_seqlens=cu)


def solve(inp, s0=None, **kw):
    return api.newton_solve("head_gru", dev_pre(inp), dev(inp.w), dev(inp.bias), s0=dev(s0), **kw)


SHAPES = [(2, 53, 2), (1, 16, 1), (3, 1, 3), (1, 200, 4)]   # (B, T, heads): tail, one chunk, T = 1, longer


@pytest.mark.parametrize("hs", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_newton_iterates(hs, dtype, shape):
    B, T, heads = shape
    announce("head newton", hs, dtype, shape)
    inp = inputs(B, T, heads, hs, dtype, seed=3000 + T + hs)
    s0 = synth.random_state(1, B, heads * hs, seed=31)
    for K in (1, 3):
        h, rep = solve(inp, s0, max_iters=K)
        H, res, iters, conv, rc = oracle.newton(oprob(inp, s0), K)
        err = rel_err(h.cpu().numpy(), H)
        print("  K=%d max rel err %.3e" % (K, err))
        assert err <= TOL
        assert rep.iters == K
        np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


@pytest.mark.parametrize("option", ["warm", "guess", "picard", "packed", "zero_s0"])
def test_newton_options(option):
    B, T, heads, hs = 2, 77, 2, 32
    announce("head newton option", option)
    inp = inputs(B, T, heads, hs, seed=3100)
    s0 = None if option == "zero_s0" else synth.random_state(1, B, heads * hs, seed=32)
    kw, okw, cu = {}, {}, None
    if option == "warm":
        kw, okw = {"warm_start": True}, {"warm": True}
    elif option == "guess":
        g = np.random.default_rng(4).standard_normal((1, B, T, heads * hs)).astype(np.float32) * 0.3
        kw, okw = {"init_guess": dev(g)}, {"init_guess": g}
    elif option == "picard":
        kw, okw = {"picard_iters": 1}, {"picard": 1}
    elif option == "packed":
        cu = synth.packed_offsets(T, seed=5, mean_len=20, forced=(16, 17, 48))
        kw = {"cu_seqlens": torch.from_numpy(cu).cuda()}
    h, rep = solve(inp, s0, max_iters=3, **kw)
    H, res, *_ = oracle.newton(oprob(inp, s0, cu), 3, **okw)
    err = rel_err(h.cpu().numpy(), H)
    print("  max rel err %.3e" % err)
    assert err <= TOL
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


def test_tolerance_mode_report_and_final_residual():
    B, T, heads, hs = 2, 150, 2, 64
    announce("head newton tol")
    inp = inputs(B, T, heads, hs, seed=3200)
    prob = oprob(inp)
    H, res, iters, conv, rc = oracle.newton(prob, 10, tol=1e-5)
    h, rep = solve(inp, max_iters=10, tol=1e-5, final_residual=True)
    assert conv and rep.converged and rep.iters == iters, (rep, res)
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)
    err = rel_err(h.cpu().numpy(), oracle.unroll(prob))
    print("  iters %d, err vs unroll %.3e, final residual %.3e" % (rep.iters, err, rep.final_residual))
    assert err <= TOL
    assert rep.final_residual is not None and rep.final_residual < 1e-5
    ref_final = oracle.residual(prob, h.cpu().numpy().astype(np.float64))
    assert abs(rep.final_residual - ref_final) <= 1e-6 + 1e-3 * ref_final


def test_example_shape_of_the_pages():
    # the pararnn-torch README's example ("Usage"): a head GRU of width 512 with 8 heads on 4 sequences of 64 steps
    B, T, heads, hs = 4, 64, 8, 64
    announce("head newton example shape")
    inp = inputs(B, T, heads, hs, seed=3300)
    prob = oprob(inp)
    h3, _ = solve(inp, max_iters=3)
    assert rel_err(h3.cpu().numpy(), oracle.newton(prob, 3)[0]) <= TOL
    H, res, iters, conv, rc = oracle.newton(prob, 8, tol=1e-5)
    h, rep = solve(inp, max_iters=8, tol=1e-5)
    print("  iters %d (oracle %d), residuals %s" % (rep.iters, iters, rep.residuals))
    assert rep.converged and rep.iters == iters
    assert rel_err(h.cpu().numpy(), oracle.unroll(prob)) <= TOL


def test_longer_sequence_many_chunks():
    B, T, heads, hs = 2, 1500, 4, 64
    announce("head newton long")
    inp = inputs(B, T, heads, hs, "bf16", seed=3400)
    s0 = synth.random_state(1, B, heads * hs, seed=33)
    h, rep = solve(inp, s0, max_iters=3)
    H, res, *_ = oracle.newton(oprob(inp, s0), 3)
    err = rel_err(h.cpu().numpy(), H)
    print("  max rel err %.3e" % err)
    assert err <= TOL


def test_nan_input_reports_divergence():
    announce("head newton nan")
    inp = inputs(1, 40, 2, 16, seed=3500)
    inp.pre[2][0, 9, 5] = np.nan
    with pytest.raises(api.NewtonDivergenceError) as e:
        solve(inp, max_iters=5, tol=1e-5)
    assert e.value.report.iters == 1 and np.isnan(e.value.report.residuals[0])


# ------------------------------------------------------------------------------------------------
# VJP.  lambda, dL/dU and dL/ds0 relative to max(1, |ref|) <= 1e-4 (as for the diagonal cells: the
# adjoint recurrence amplifies fp32 rounding).  A parameter entry is a sum over rows n of dU_n x_n,
# so its error is bounded by the gate gradients' own absolute errors times |x_n| plus the fp32
# summation: dA and dbias are checked against 1e-5 * sum_n max(1, |dU_n|) |x_n| (1e-5 is the absolute
# error allowed per gate gradient here; factors such as (c - h) cancel, so a small dU carries an
# absolute, not a relative, fp32 error).  The bounds come from the oracle's fp64 gate gradients.
# ------------------------------------------------------------------------------------------------
def prev_states(traj, s0, cu, T):
    """[B][T][D] state each step starts from: s0, zero at a sequence start, else s_{t-1}."""
    prev = np.zeros_like(traj)
    prev[:, 1:] = traj[:, :-1]
    prev[:, 0] = 0.0 if s0 is None else s0[0]
    if cu is not None:
        for c in cu:
            if 0 < c < T:
                prev[:, c] = 0.0
    return prev


def param_bounds(ref, traj, s0, inp, cu):
    """sum_n max(1, |dU_n|) |x_n| of every dA and dbias entry."""
    B, T, D, hs = inp.B, inp.T, inp.D, inp.head_size
    H = D // hs
    prev = prev_states(traj, s0, cu, T).reshape(B * T, H, hs)
    dU = np.maximum(1.0, np.abs(ref["d_pre"])).reshape(3, B * T, H, hs)
    # x of gate c is r_t * s_{t-1}; |r| <= 1, so |s_{t-1}| bounds it
    x = np.abs(prev)
    bw = np.einsum("gnhi,nhj->ghij", dU, x)
    bb = dU.sum(axis=1).reshape(3, D)
    return bw, bb


def vjp_case(inp, s0=None, cu=None, want_lambda=True):
    prob = oprob(inp, s0, cu)
    traj = oracle.unroll(prob).astype(np.float32)
    ref = oracle.vjp(prob, traj.astype(np.float64), inp.g)
    kw = {"cu_seqlens": torch.from_numpy(cu).cuda()} if cu is not None else {}
    got = api.scan_vjp("head_gru", dev_pre(inp), dev(traj), dev(inp.g), dev(inp.w), dev(inp.bias), s0=dev(s0),
                       want_lambda=want_lambda, **kw)
    got = {k: (v.cpu().numpy() if v is not None else None) for k, v in got.items()}
    for k in ("d_pre", "lam", "d_s0"):
        if got.get(k) is not None:
            err = rel_err(got[k], ref[k])
            print("  %s max rel err %.3e" % (k, err))
            assert err <= 1e-4, k
    bw, bb = param_bounds(ref, traj[0].astype(np.float64), s0, inp, cu)
    ew = float(np.max(np.abs(got["d_w"] - ref["d_w"]) / np.maximum(bw, 1e-30)))
    eb = float(np.max(np.abs(got["d_bias"] - ref["d_bias"]) / np.maximum(bb, 1e-30)))
    print("  d_w err / bound %.3e, d_bias %.3e" % (ew, eb))
    assert ew <= 1e-5 and eb <= 1e-5
    return got


@pytest.mark.parametrize("hs", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_vjp(hs, dtype, shape):
    B, T, heads = shape
    announce("head vjp", hs, dtype, shape)
    inp = inputs(B, T, heads, hs, dtype, seed=3600 + T + hs, with_grad=True)
    s0 = synth.random_state(1, B, heads * hs, seed=34)
    vjp_case(inp, s0)


def test_vjp_packed_sequences_and_zero_state():
    announce("head vjp packed")
    B, T, heads, hs = 2, 90, 2, 32
    inp = inputs(B, T, heads, hs, seed=3700, with_grad=True)
    cu = synth.packed_offsets(T, seed=6, mean_len=18, forced=(16, 17, 33, 89))
    vjp_case(inp, None, cu)


def test_vjp_example_shape_and_reproducible():
    announce("head vjp example shape")
    B, T, heads, hs = 4, 64, 8, 64
    inp = inputs(B, T, heads, hs, seed=3800, with_grad=True)
    got = vjp_case(inp, want_lambda=False)
    again = api.scan_vjp("head_gru", dev_pre(inp), dev(oracle.unroll(oprob(inp)).astype(np.float32)), dev(inp.g),
                         dev(inp.w), dev(inp.bias))
    for k in ("d_pre", "d_w", "d_bias", "d_s0"):
        assert np.array_equal(again[k].cpu().numpy(), got[k]), k    # fixed-order sums: bitwise equal


def test_vjp_long_sequence():
    announce("head vjp long")
    B, T, heads, hs = 2, 1500, 4, 64
    inp = inputs(B, T, heads, hs, "bf16", seed=3900, with_grad=True)
    vjp_case(inp, synth.random_state(1, B, heads * hs, seed=35), want_lambda=False)


def test_empty_problems_are_no_ops():
    announce("head empty")
    for B, T in ((0, 10), (2, 0)):
        inp = inputs(max(B, 1), max(T, 1), 2, 16, seed=4000)
        pre = [torch.empty((B, T, 32), device="cuda") for _ in range(3)]
        h, rep = api.newton_solve("head_gru", pre, dev(inp.w), dev(inp.bias), max_iters=3, tol=1e-5)
        assert h.shape == (1, B, T, 32) and rep.iters == 0 and rep.converged
        gr = api.scan_vjp("head_gru", pre, h, torch.empty((B, T, 32), device="cuda"), dev(inp.w), dev(inp.bias))
        assert gr["d_pre"].shape == (3, B, T, 32)
