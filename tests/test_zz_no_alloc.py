"""pararnn_newton_solve_noalloc (the solve for callers that cannot allocate: its workspace is the library's
static device array) against pararnn_newton_solve with a caller workspace: the same trajectory and report,
bit for bit, on two calls in a row, the second with a smaller input; a problem that does not fit the array
is rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_pre
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20   # PARARNN_NOALLOC_SCRATCH_BYTES


def announce(*a):
    print("[case]", *a, flush=True)


def _solve_both(cell, dtype, B, T, D, seed, **opts):
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=seed)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    ref, rep_ref = api.newton_solve(cell, pre, w, b, **opts)
    out = torch.full_like(ref, float("nan"))
    got, rep = api.newton_solve(cell, pre, w, b, out=out, noalloc=True, **opts)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, ref)
    assert (rep.iters, rep.converged, rep.residuals, rep.final_residual) == \
        (rep_ref.iters, rep_ref.converged, rep_ref.residuals, rep_ref.final_residual)
    return rep


def test_noalloc_equals_the_workspace_solve_on_two_calls_in_a_row():
    # 1: the LSTM at the long workload's size, whose default launch length needs 200 MiB of look-back words:
    #    the call shortens it to fit the 128 MiB array
    announce("noalloc lstm f32 (4, 8192, 2048) tol 1e-5")
    rep = _solve_both("lstm", "f32", 4, 8192, 2048, 3, max_iters=8, tol=1e-5, final_residual=True)
    assert rep.converged
    # 2: a smaller GRU problem right after, which finds the first call's words in the array
    announce("noalloc gru bf16 (2, 3000, 96) K=3")
    rep = _solve_both("gru", "bf16", 2, 3000, 96, 5, max_iters=3)
    assert rep.iters == 3


def test_noalloc_rejects_what_does_not_fit():
    inp = synth.make_inputs("lstm", 4, 8192, 2048, dtype="f32", seed=3)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    ws = api.newton_workspace_bytes("lstm", pre, w, b)      # the size that fits every option: 8 launches
    assert ws > SCRATCH
    with pytest.raises(api.PararnnError) as ei:
        api.newton_solve("lstm", pre, w, b, max_iters=8, fuse_iters=8, noalloc=True)
    assert ei.value.status == -3
