"""Look-back race stress: the library built with -DPR_LB_STRESS=1 (libpararnn_stress.so) pauses tiles for
pseudo-random times around the publication of their look-back words, so that tiles find their predecessor
with only its aggregate published and take the other path to their carry (that aggregate applied to the
state of the tile before it).  Every scan of the method (the Newton update's linear solve, the plain linear
scan, the adjoint's reverse scan; pararnn-torch README, "Method") joins its time chunks this way, and the
carry must not depend on which path a tile took: each result of the stress build must equal the plain
library's bit for bit, run after run, while the aggregate path is really taken.  The first mismatch ends the
test (the loops assert as they go).
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_pre
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu

RUNS = 3


def announce(*a):
    print("[case]", *a, flush=True)


def _both(fn):
    """fn() with the plain library, then RUNS times with the stress build: the plain result and the deepest
    walk the stress runs saw (>= 1: some carry came from an aggregate); every stress result is compared with the
    plain one bit for bit."""
    ref = fn()
    with api.using_library(api.STRESS_LIB_PATH):
        api.lookback_depth(reset=True)
        for run in range(RUNS):
            got = fn()
            for k in ref:
                if ref[k] is None:
                    continue
                assert torch.equal(got[k], ref[k]), (k, run)
        depth = api.lookback_depth(reset=True)
    print("  deepest walk:", depth, "aggregate(s)", flush=True)
    return ref, depth


@pytest.mark.parametrize("S,reverse,dtype", [(1, False, "f32"), (1, True, "bf16"), (2, False, "f32"), (2, True, "f32")])
def test_linear_scan_stress(S, reverse, dtype):
    announce("scan stress", S, reverse, dtype)
    B, T, D = 2, 40000, 64
    if S == 1:
        inp = synth.make_inputs("linear", B, T, D, dtype=dtype, seed=2100)
        a, b = dev_pre(inp)
    else:
        rng = np.random.default_rng(2101)
        A = np.empty((4, B, T, D), np.float32)
        A[0] = rng.uniform(0.3, 0.99, (B, T, D))
        A[3] = rng.uniform(0.3, 0.99, (B, T, D))
        A[1] = rng.uniform(-0.05, 0.05, (B, T, D))
        A[2] = rng.uniform(-0.05, 0.05, (B, T, D))
        a, b = dev(A), dev(rng.standard_normal((2, B, T, D)).astype(np.float32))
    s0 = dev(synth.random_state(S, B, D, seed=21))
    _, depth = _both(lambda: {"h": api.linear_scan(a, b, s0=s0, reverse=reverse).clone()})
    assert depth >= 1


@pytest.mark.parametrize("cell,dtype,fuse", [("gru", "bf16", 1), ("gru", "bf16", 0), ("gru", "f32", 3),
                                             ("lstm", "f32", 1), ("lstm", "f32", 0)])
def test_newton_stress(cell, dtype, fuse):
    announce("newton stress", cell, dtype, "fuse", fuse)
    B, T, D = 1, 32768, 64
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=2200, with_grad=True)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    s0 = dev(synth.random_state(inp.S, B, D, seed=22))

    def run():
        h, rep = api.newton_solve(cell, pre, w, b, max_iters=4, s0=s0, fuse_iters=fuse)
        return {"h": h.clone(), "res": torch.tensor(rep.residuals)}
    ref, depth = _both(run)
    assert depth >= 1

    def vjp():
        g = api.scan_vjp(cell, pre, ref["h"], dev(inp.g), w, b, s0=s0, want_lambda=True)
        return {k: (None if v is None else v.clone()) for k, v in g.items()}
    _, depth = _both(vjp)
    assert depth >= 1


def test_slstm_newton_walk_stress():
    """The sLSTM Newton iteration takes its carry by the walk (any depth, the passed aggregates re-read and
    applied in order); its VJP by the wait at most one aggregate deep."""
    announce("slstm newton + vjp stress")
    B, T, D = 1, 32768, 64
    inp = synth.make_inputs("slstm", B, T, D, dtype="f32", seed=2400, with_grad=True)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    s0 = synth.random_state(4, B, D, seed=24)
    s0[1] = np.abs(s0[1]) + 0.5     # the normaliser n is positive
    s0 = dev(s0)

    def run():
        h, rep = api.newton_solve("slstm", pre, w, b, max_iters=6, picard_iters=2, s0=s0)
        return {"h": h.clone(), "res": torch.tensor(rep.residuals)}
    ref, depth = _both(run)
    assert depth >= 2     # the walk passed several aggregates and re-read them

    def vjp():
        g = api.scan_vjp("slstm", pre, ref["h"], dev(inp.g), w, b, s0=s0, want_lambda=True)
        return {k: (None if v is None else v.clone()) for k, v in g.items()}
    _, depth = _both(vjp)
    assert depth >= 1


def test_tolerance_mode_and_packed_stress():
    announce("tolerance + packed stress")
    B, T, D = 1, 32768, 64
    inp = synth.make_inputs("gru", B, T, D, dtype="bf16", seed=2300)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    cu = torch.tensor(synth.packed_offsets(T, 23, 3000), dtype=torch.int32, device="cuda")

    def run():
        h, rep = api.newton_solve("gru", pre, w, b, max_iters=8, tol=1e-5, cu_seqlens=cu)
        return {"h": h.clone(), "res": torch.tensor(rep.residuals + [rep.iters])}
    _, depth = _both(run)
    assert depth >= 1
