"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph): every launch of a solve,
scan and VJP is asynchronous and allocation-free once the workspace exists, and each call clears
its workspace with a kernel (not a memset node), so replays are independent.  Each replay is checked
bitwise against the eager result, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_pre
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cell,dtype,shape,tol,fuse", [("gru", "bf16", (1, 5000, 64), 1e-5, 0),
                                                       ("gru", "bf16", (1, 5000, 64), 1e-5, 6),   # speculation re-run
                                                       ("lstm", "f32", (2, 700, 34), 0.0, 0),
                                                       ("head_gru", "f32", (2, 300, 128), 1e-5, 0)])
def test_captured_solve_and_vjp_replay_like_eager(cell, dtype, shape, tol, fuse):
    B, T, D = shape
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=3100 + T, with_grad=True,
                            head_size=64 if cell == "head_gru" else None)
    pre, w, b, g = dev_pre(inp), dev(inp.w), dev(inp.bias), dev(inp.g)
    lin = synth.make_inputs("linear", B, T, D, seed=3101)
    a_, b_ = dev(lin.pre[0]), dev(lin.pre[1])
    out = torch.empty((inp.S, B, T, D), device="cuda")
    scan_out = torch.empty((B, T, D), device="cuda")
    # eager reference (also creates the cached workspaces)
    kw = {"fuse_iters": fuse} if fuse else {}
    ref_h, ref_rep = api.newton_solve(cell, pre, w, b, max_iters=6, tol=tol, out=out.clone(), **kw)
    if fuse:
        assert ref_rep.iters < fuse   # the speculative launch ran past the stop: the re-run launch does the work
    ref_g = api.scan_vjp(cell, pre, ref_h, g, w, b)
    ref_s = api.linear_scan(a_, b_)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        api.newton_solve(cell, pre, w, b, max_iters=6, tol=tol, out=out, report=False, **kw)   # warm the workspace
        api.linear_scan(a_, b_, out=scan_out)
        gr0 = api.scan_vjp(cell, pre, out, g, w, b)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        api.newton_solve(cell, pre, w, b, max_iters=6, tol=tol, out=out, report=False, **kw)
        api.linear_scan(a_, b_, out=scan_out)
        grads = api.scan_vjp(cell, pre, out, g, w, b)
    for rep in range(3):
        out.zero_()
        scan_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_h), rep
        assert torch.equal(scan_out, ref_s), rep
        for k in ("d_pre", "d_w", "d_bias", "d_s0"):
            assert torch.equal(grads[k], ref_g[k]), (rep, k)
        # eager work between replays
        api.newton_solve(cell, pre, w, b, max_iters=2)
        torch.cuda.synchronize()
    del gr0


def test_each_stream_has_its_own_workspace():
    # solves on two streams may overlap, so the binding gives each stream its own workspace: a side stream's
    # solve equals the default stream's, and the two cached buffers are distinct
    inp = synth.make_inputs("gru", 2, 3000, 64, dtype="bf16", seed=3150)
    pre, w, b = dev_pre(inp), dev(inp.w), dev(inp.bias)
    ref, _ = api.newton_solve("gru", pre, w, b, max_iters=8, tol=1e-5)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got, rep = api.newton_solve("gru", pre, w, b, max_iters=8, tol=1e-5)
        ws_side = api._workspace(1, pre[0].device, "newton")
    torch.cuda.synchronize()
    ws_default = api._workspace(1, pre[0].device, "newton")
    assert ws_side.data_ptr() != ws_default.data_ptr()
    assert torch.equal(got, ref) and rep.converged
