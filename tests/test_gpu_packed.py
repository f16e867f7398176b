"""GPU parity for packed variable-length sequences (cu_seqlens): the HIP library against the fp64
oracle on the same seeded inputs and offsets.

Offsets mix geometric lengths with forced boundaries on the kernels' structural edges: a lane's
8 or 16 steps, a wave's slices, a workgroup chunk (128 steps for the GRU Newton tile, 256 for the
scalar scan), the first and last step, empty and length-1 sequences.  Tolerances as in
test_gpu_parity: fp32-level errors (1e-5 fixed-K iterates and scans, 1e-4 relative for the VJP).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre, max_abs, oracle_problem, sample_channels, take_channels
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu

EDGES = (1, 7, 8, 9, 16, 64, 127, 128, 129, 255, 256, 257, 511, 512)


def announce(*a):
    print("[case]", *a, flush=True)


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def offsets(T, seed, mean_len):
    cu = synth.packed_offsets(T, seed, mean_len, forced=[e for e in EDGES if e < T] + [T - 1])
    return cu, torch.from_numpy(cu).cuda()


@pytest.mark.parametrize("S,dtype,shape,reverse", [(1, "f32", (2, 1000, 100), False), (1, "f32", (2, 1000, 100), True),
                                                   (1, "bf16", (1, 4096, 64), False), (2, "f32", (3, 700, 6), False),
                                                   (2, "bf16", (1, 1500, 34), True), (1, "f32", (1, 2, 2), False)])
def test_packed_linear_scan(S, dtype, shape, reverse):
    B, T, D = shape
    announce("packed scan", S, dtype, shape, reverse)
    rng = np.random.default_rng(2000 + T)
    A = rng.uniform(-0.95, 0.95, ((4,) if S == 2 else ()) + (B, T, D)).astype(np.float32)
    if S == 2:
        A[1:3] *= 0.1
    b = rng.standard_normal(((2,) if S == 2 else ()) + (B, T, D)).astype(np.float32)
    if dtype == "bf16":
        A, b = synth.f32_to_bf16_bits(A), synth.f32_to_bf16_bits(b)
        ta = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
        tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        ta, tb = dev(A), dev(b)
    s0 = synth.random_state(S, B, D, seed=30)
    cu, tcu = offsets(T, 2100 + T, 60)
    ref = oracle.linear_scan(A, b, s0=s0, reverse=reverse, S=S, dtype=oracle.BF16 if dtype == "bf16" else oracle.F32,
                             cu_seqlens=cu)
    got = api.linear_scan(ta, tb, s0=dev(s0), reverse=reverse, cu_seqlens=tcu).cpu().numpy()
    err = rel_err(got, ref)
    print("  n_seqs", len(cu) - 1, "max rel err", err)
    assert err <= 1e-5


NEWTON_CASES = [("gru", "f32", (2, 1000, 200), 3, False), ("gru", "bf16", (1, 3000, 64), 3, True),
                ("lstm", "f32", (2, 1000, 66), 3, False), ("lstm", "bf16", (1, 777, 8), 2, True),
                ("linear", "f32", (2, 600, 16), 1, False), ("gru", "f32", (3, 129, 6), 4, False)]


@pytest.mark.parametrize("cell,dtype,shape,K,warm", NEWTON_CASES)
def test_packed_newton(cell, dtype, shape, K, warm):
    B, T, D = shape
    announce("packed newton", cell, dtype, shape, K, "warm" if warm else "zero")
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=2200 + T + D)
    s0 = synth.random_state(inp.S, B, D, seed=31)
    cu, tcu = offsets(T, 2300 + T, 90)
    H, res, *_ = oracle.newton(oracle_problem(inp, s0, cu_seqlens=cu), K, warm=warm)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0),
                                warm_start=warm, cu_seqlens=tcu, final_residual=True)
    err = max_abs(got.cpu().numpy(), H)
    print("  n_seqs", len(cu) - 1, "max abs err", err, "residuals", rep.residuals, "oracle", list(res))
    assert err <= (1e-5 if dtype == "f32" else 1e-4)
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)
    # the final residual pass honours the boundaries too
    assert abs(rep.final_residual - oracle.residual(oracle_problem(inp, s0, cu_seqlens=cu), got.cpu().numpy())) <= 1e-5


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_packed_newton_tolerance_mode_reaches_the_unroll(cell):
    B, T, D = 2, 2500, 32
    inp = synth.make_inputs(cell, B, T, D, seed=2400)
    cu, tcu = offsets(T, 2401, 300)
    prob = oracle_problem(inp, cu_seqlens=cu)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=10, tol=1e-5,
                                cu_seqlens=tcu)
    _, ores, oit, oconv, _ = oracle.newton(prob, 10, tol=1e-5)
    print("  gpu iters", rep.iters, rep.residuals, "oracle", oit, list(ores))
    assert rep.converged and abs(rep.iters - oit) <= 1
    assert max_abs(got.cpu().numpy(), oracle.unroll(prob)) <= 1e-4


def test_unpacked_offsets_match_the_plain_solve():
    inp = synth.make_inputs("gru", 2, 900, 32, dtype="bf16", seed=2402)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    plain, _ = api.newton_solve("gru", pre, w, b, max_iters=3)
    for cu in ([0, 900], [0, 0, 900, 900]):
        packed, _ = api.newton_solve("gru", pre, w, b, max_iters=3, cu_seqlens=torch.tensor(cu, dtype=torch.int32).cuda())
        assert torch.equal(plain, packed)


VJP_CASES = [("gru", "f32", (2, 1000, 100)), ("gru", "bf16", (1, 1500, 64)), ("lstm", "f32", (2, 700, 66)),
             ("linear", "f32", (2, 1000, 64)), ("lstm", "bf16", (1, 300, 8))]


@pytest.mark.parametrize("cell,dtype,shape", VJP_CASES)
def test_packed_vjp(cell, dtype, shape):
    B, T, D = shape
    announce("packed vjp", cell, dtype, shape)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=2500 + T, with_grad=True)
    s0 = synth.random_state(inp.S, B, D, seed=32)
    cu, tcu = offsets(T, 2600 + T, 80)
    prob = oracle_problem(inp, s0, cu_seqlens=cu)
    traj = oracle.unroll(prob).astype(np.float32)
    ref = oracle.vjp(prob, traj.astype(np.float64), inp.g)
    got = api.scan_vjp(cell, dev_pre(inp), dev(traj), dev(inp.g), dev(inp.w), dev(inp.bias), s0=dev(s0),
                       want_lambda=True, cu_seqlens=tcu)
    e_lam = rel_err(got["lam"].cpu().numpy(), ref["lam"])
    e_dp = rel_err(got["d_pre"].cpu().numpy(), ref["d_pre"])
    e_s0 = rel_err(got["d_s0"].cpu().numpy(), ref["d_s0"])
    print("  n_seqs", len(cu) - 1, "lambda", e_lam, "d_pre", e_dp, "d_s0", e_s0)
    assert e_lam <= 1e-4 and e_dp <= 1e-4 and e_s0 <= 1e-4
    if cell != "linear":
        scale_b = np.abs(ref["d_pre"]).sum(axis=(1, 2)) + 1.0
        e_b = np.max(np.abs(got["d_bias"].cpu().numpy() - ref["d_bias"]) / scale_b)
        e_w = np.max(np.abs(got["d_w"].cpu().numpy() - ref["d_w"]) / (scale_b * max(1.0, np.abs(traj).max())))
        print("  d_w", e_w, "d_bias", e_b)
        assert e_w <= 1e-5 and e_b <= 1e-5


def test_packed_long_sequence_newton_and_vjp_sampled():
    # the long-sequence GRU workload (B=1, T=131072, D=1024, bf16 gate inputs) packed into sequences
    # of mean length 2048, tolerance mode, then the VJP; checked on sampled channels
    B, T, D = 1, 131072, 1024
    announce("packed long", B, T, D)
    inp = synth.make_inputs("gru", B, T, D, dtype="bf16", seed=4, with_grad=True)
    cu, tcu = offsets(T, 2700, 2048)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    got, rep = api.newton_solve("gru", pre, w, b, max_iters=8, tol=1e-5, cu_seqlens=tcu, final_residual=True)
    print("  n_seqs", len(cu) - 1, "iters", rep.iters, rep.residuals, "final", rep.final_residual)
    assert rep.converged and rep.final_residual < 1e-5
    ch = sample_channels(B, D, 12, seed=7)
    prob = oracle_problem(inp, channels=ch, cu_seqlens=cu)
    unroll = oracle.unroll(prob)
    g_s = take_channels(got.cpu().numpy(), ch)
    print("  vs unroll", max_abs(g_s, unroll))
    assert max_abs(g_s, unroll) <= 1e-4
    gr = api.scan_vjp("gru", pre, got, dev(inp.g), w, b, want_lambda=True, cu_seqlens=tcu)
    ref = oracle.vjp(prob, unroll, take_channels(inp.g, ch))
    e_lam = rel_err(take_channels(gr["lam"].cpu().numpy(), ch), ref["lam"])
    e_dp = rel_err(take_channels(gr["d_pre"].cpu().numpy(), ch), ref["d_pre"])
    print("  vjp lambda", e_lam, "d_pre", e_dp)
    assert e_lam <= 2e-2 and e_dp <= 2e-2
