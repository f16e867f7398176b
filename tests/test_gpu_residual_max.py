"""The max residual that the Newton kernels reduce over a wave (lane pairs, quads, half rows, rows, then the
row broadcasts) and over a tile's waves, pinned lane by lane.  The first iterate is the sequential unroll
with one spike, so the largest residual sits at a chosen step and channel: with the GRU tiles of 32
channels x 256 steps (each wave two time slices of 16 steps, lane = 32 slice + channel in the group), the
positions below land on lanes 0..63 of every pattern the reduction pairs up, on all eight waves, on both
tiles and both channel groups.  Iteration 0's reported residual is the max |h_t - f(h_{t-1}, x_t)| of that
iterate, which the oracle evaluates in fp64; a NaN or an infinite spike at the same places must come back
as a NaN (the solve stops as diverged).  Run through the one-launch-per-iteration kernel and the fused pass.
The final-residual pass (its own kernel, the same wave reduction) is held to the oracle too."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_pre, oracle_problem
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu

B, T, D = 1, 512, 64
LANES = [0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 16, 17, 31, 32, 33, 46, 47, 48, 63]


def _position(lane):
    """(t, d) of a step inside lane `lane` of wave lane % 8, tile lane % 2, channel group (lane // 2) % 2"""
    wave, tile, group = lane % 8, lane % 2, (lane // 2) % 2
    slice_, q = divmod(lane, 32)
    return tile * 256 + wave * 32 + slice_ * 16 + 5, group * 32 + q


@pytest.fixture(scope="module")
def problem():
    inp = synth.make_inputs("gru", B, T, D, seed=4400)
    prob = oracle_problem(inp)
    H = oracle.unroll(prob).astype(np.float32)    # [1][B][T][D]
    return inp, prob, H


def _solve(inp, H, fuse, **kw):
    iters = 1 if fuse == 1 else 2
    return api.newton_solve("gru", dev_pre(inp), dev(inp.w), dev(inp.bias), max_iters=iters, fuse_iters=fuse,
                            init_guess=dev(H), **kw)


@pytest.mark.parametrize("fuse", [1, 2])
def test_spike_on_every_lane_pattern(problem, fuse):
    inp, prob, H0 = problem
    for k, lane in enumerate(LANES):
        t, d = _position(lane)
        H = H0.copy()
        H[0, 0, t, d] += 0.25 + 0.01 * k        # a different maximum for every case
        want = oracle.residual(prob, H)
        _, rep = _solve(inp, H, fuse)
        got = rep.residuals[0]
        print("[resmax] fuse", fuse, "lane", lane, "t", t, "d", d, "got", got, "want", want, flush=True)
        assert want > 0.2
        assert abs(got - want) <= 1e-5 * want, (lane, got, want)


@pytest.mark.parametrize("fuse", [1, 2])
@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_non_finite_spike_on_every_lane_pattern(problem, fuse, bad):
    inp, _, H0 = problem
    for lane in LANES:
        t, d = _position(lane)
        H = H0.copy()
        H[0, 0, t, d] = bad
        print("[resmax] fuse", fuse, "lane", lane, "spike", bad, flush=True)
        with pytest.raises(api.NewtonDivergenceError) as ei:
            _solve(inp, H, fuse, tol=1e-5)
        rep = ei.value.report
        assert rep.iters == 1 and np.isnan(rep.residuals[0]), (lane, rep)


def test_final_residual_pass(problem):
    inp, prob, H0 = problem
    H = H0.copy()
    t, d = _position(37)
    H[0, 0, t, d] += 0.5
    out, rep = _solve(inp, H, 1, final_residual=True)
    torch.cuda.synchronize()
    want = oracle.residual(prob, out.cpu().numpy())
    print("[resmax] final residual", rep.final_residual, "oracle on the returned trajectory", want, flush=True)
    assert rep.final_residual is not None
    assert abs(rep.final_residual - want) <= 1e-3 * want + 1e-6
