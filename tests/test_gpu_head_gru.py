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
    # ParaGRU(512, 512, mix="head", n_heads=8) applied to a (4, 64, 512) batch (pararnn-torch README, "Usage")
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
