"""The fused Newton pass (several iterations in one launch, the trajectory kept in registers between
them) against one launch per iteration (fuse_iters = 1): the same trajectory bit for bit and the same
report, for the diagonal GRU and LSTM in fp32 and bf16 storage.  Cases: fixed budgets below, at and above
the longest fused launch (so a solve takes several fused launches), s0, the warm start, a first iterate
in a separate buffer and in the output itself, packed sequences, lengths that end inside a lane's steps,
channel counts that leave lanes of a tile idle, and tolerance mode whose speculative first launch is too
long (the re-run recomputes it), exact, or too short (single launches follow).  The re-run and the single
launches after the first take tickets in a loop on a grid of what is resident; the tolerance cases make them
compute (launch lengths 2 and 3 leave iterations to them, 8 runs past the stop), in the masked and packed
variants too.  The fused solve is also held to the oracle directly, since a solve now runs fused by default."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre, oracle_problem
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[fused]", *a, flush=True)


def _inputs(cell, dtype, shape, seed, s0=False, guess=False, seqs=False):
    B, T, D = shape
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=seed)
    kw = {}
    if s0:
        kw["s0"] = dev(synth.random_state(inp.S, B, D, seed=seed + 1))
    if guess:
        rng = np.random.default_rng(seed + 2)
        kw["init_guess"] = dev((0.2 * rng.standard_normal((inp.S, B, T, D))).astype(np.float32))
    if seqs:
        rng = np.random.default_rng(seed + 3)
        cuts = sorted(set([0, T] + [int(x) for x in rng.integers(1, T, size=5)]))
        kw["cu_seqlens"] = torch.tensor(cuts, dtype=torch.int32, device="cuda")
    return inp, kw


def _solve(cell, inp, kw, fuse, in_place=False, **opts):
    args = dict(kw)
    if in_place:
        # the first iterate is the output buffer itself (resume)
        buf = kw["init_guess"].clone()
        args["init_guess"] = buf
        args["out"] = buf
    out, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), fuse_iters=fuse, **args, **opts)
    torch.cuda.synchronize()
    return out.clone(), rep


def _same(a, b):
    ra, rb = a[1], b[1]
    return (torch.equal(a[0], b[0]) and ra.iters == rb.iters and ra.converged == rb.converged
            and ra.residuals == rb.residuals)


CASES = [
    # cell, dtype, (B, T, D), options
    ("gru", "f32", (3, 1000, 100), dict(max_iters=5)),
    ("gru", "bf16", (2, 1300, 130), dict(max_iters=10, s0=True)),            # two fused launches (8 + 2)
    ("gru", "f32", (1, 3000, 64), dict(max_iters=4, warm_start=True)),
    ("gru", "f32", (2, 777, 66), dict(max_iters=3, guess=True)),
    ("gru", "f32", (2, 777, 66), dict(max_iters=3, guess=True, in_place=True)),
    ("gru", "bf16", (2, 2000, 64), dict(max_iters=4, seqs=True)),
    ("gru", "f32", (1, 5, 2), dict(max_iters=4)),                             # one lane, mostly idle
    ("gru", "f32", (1, 3000, 64), dict(max_iters=0)),                        # the measured budget
    ("lstm", "f32", (2, 1500, 70), dict(max_iters=6, s0=True)),
    ("lstm", "bf16", (2, 900, 64), dict(max_iters=3, warm_start=True, seqs=True)),
    ("lstm", "f32", (1, 129, 66), dict(max_iters=9)),
    ("gru", "f32", (2, 5000, 64), dict(max_iters=8, tol=1e-5)),
    ("gru", "bf16", (2, 5000, 64), dict(max_iters=8, tol=1e-5, warm_start=True)),
    ("lstm", "f32", (2, 3000, 64), dict(max_iters=8, tol=1e-5)),
    ("gru", "f32", (1, 2000, 64), dict(max_iters=8, tol=1e-5, guess=True)),
    ("gru", "f32", (1, 2000, 64), dict(max_iters=8, tol=1e-5, guess=True, in_place=True)),
    ("gru", "bf16", (2, 3000, 64), dict(max_iters=8, tol=1e-5, seqs=True)),
    ("lstm", "bf16", (2, 2500, 64), dict(max_iters=8, tol=1e-5, seqs=True)),
    ("gru", "f32", (1, 2000, 64), dict(max_iters=8, tol=1e-1)),              # stops after few iterations
    ("gru", "f32", (1, 2000, 64), dict(max_iters=8, tol=1e-30)),             # never stops: the budget
]


@pytest.mark.parametrize("cell,dtype,shape,opts", CASES)
def test_fused_equals_one_launch_per_iteration(cell, dtype, shape, opts):
    opts = dict(opts)
    flags = {k: opts.pop(k, False) for k in ("s0", "guess", "seqs", "in_place")}
    inp, kw = _inputs(cell, dtype, shape, seed=4000 + shape[1] + shape[2], s0=flags["s0"], guess=flags["guess"],
                      seqs=flags["seqs"])
    ref = _solve(cell, inp, kw, 1, in_place=flags["in_place"], **opts)
    for fuse in (0, 2, 3, 5, api.MAX_FUSE):
        announce(cell, dtype, shape, opts, flags, "fuse", fuse)
        got = _solve(cell, inp, kw, fuse, in_place=flags["in_place"], **opts)
        assert _same(got, ref), (fuse, float((got[0] - ref[0]).abs().max()), got[1], ref[1])


def test_tolerance_speculation_too_short_exact_too_long():
    # a solve that needs n iterations: a first launch of n - 2, n and n + 2 iterations (the last is re-run)
    inp, kw = _inputs("gru", "bf16", (2, 4096, 256), seed=4100)
    ref = _solve("gru", inp, kw, 1, max_iters=8, tol=1e-5)
    n = ref[1].iters
    announce("tolerance needs", n, ref[1].residuals)
    assert ref[1].converged and 3 <= n <= 6
    for fuse in (n - 2, n, n + 2):
        got = _solve("gru", inp, kw, fuse, max_iters=8, tol=1e-5)
        assert _same(got, ref), fuse


def test_divergence_inside_a_fused_launch():
    # a NaN gate input: iteration 0's residual is NaN, so the solve stops after it; the speculative launch
    # of 4 iterations is re-run with one
    inp = synth.make_inputs("gru", 1, 300, 8, seed=4200)
    inp.pre[0][0, 100, 3] = np.nan
    outs = []
    for fuse in (1, 4):
        buf = torch.zeros((1, 1, 300, 8), device="cuda")
        with pytest.raises(api.NewtonDivergenceError) as ei:
            api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=6, tol=1e-5,
                             fuse_iters=fuse, out=buf)
        assert ei.value.report.iters == 1 and np.isnan(ei.value.report.residuals[0])
        outs.append(buf.view(torch.int32).clone())   # bit patterns: NaNs compare equal
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("cell,dtype,shape,K", [("gru", "bf16", (2, 3000, 200), 10), ("lstm", "f32", (2, 1000, 70), 8),
                                                ("gru", "f32", (3, 129, 6), 5)])
def test_fused_solve_against_the_oracle(cell, dtype, shape, K):
    B, T, D = shape
    announce("oracle", cell, dtype, shape, K)
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=4300 + T)
    s0 = synth.random_state(inp.S, B, D, seed=12)
    H, res, _, _, _ = oracle.newton(oracle_problem(inp, s0), K)
    got, rep = api.newton_solve(cell, dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=K, s0=dev(s0),
                                fuse_iters=api.MAX_FUSE)
    err = float(np.max(np.abs(got.cpu().numpy() - H)))
    print("  max abs err", err)
    assert rep.iters == K
    assert err <= (1e-5 if dtype == "f32" else 2e-2) and err <= 1e-4
    np.testing.assert_allclose(rep.residuals, res, rtol=1e-3, atol=1e-5)


@pytest.mark.parametrize("cell,dtype,shape", [("gru", "bf16", (1, 65536, 512)), ("lstm", "f32", (2, 16384, 256))])
def test_looping_launches_with_several_tiles_per_workgroup(cell, dtype, shape):
    # thousands of tiles against ~1000 resident workgroups: the looping re-run (speculation too long) and the
    # looping single launches (too short) each take several tiles per workgroup, in ticket order
    inp, kw = _inputs(cell, dtype, shape, seed=4500 + shape[1])
    ref = _solve(cell, inp, kw, 1, max_iters=8, tol=1e-5)
    n = ref[1].iters
    announce("looping launches", cell, dtype, shape, "needs", n)
    assert ref[1].converged and 4 <= n <= 7
    for fuse in (2, api.MAX_FUSE):
        got = _solve(cell, inp, kw, fuse, max_iters=8, tol=1e-5)
        assert _same(got, ref), (fuse, float((got[0] - ref[0]).abs().max()), got[1], ref[1])
