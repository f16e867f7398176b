"""Solves on two streams at once.  Every scan of the library orders its tiles by atomic tickets and a tile waits
only on smaller tickets of its own launch, which running or finished workgroups hold, so launches that share the
chip (including the ones that loop over tiles on a grid of what is resident) can neither deadlock nor change each
other's results: each result must equal the same call run alone, bit for bit.  The binding gives each stream its
own workspace (pararnn-torch README, "Compatibility": determinism)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_pre
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[streams]", *a, flush=True)


def _problem(cell, dtype, shape, seed):
    B, T, D = shape
    inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=seed, with_grad=True)
    return cell, dev_pre(inp), dev(inp.w), dev(inp.bias), dev(inp.g), (inp.S, B, T, D)


def _run(p, fuse):
    cell, pre, w, b, g, shp = p
    out = torch.empty(shp, dtype=torch.float32, device="cuda")
    api.newton_solve(cell, pre, w, b, max_iters=8, tol=1e-5, out=out, report=False, fuse_iters=fuse)
    grads = api.scan_vjp(cell, pre, out, g, w, b, want_s0=False)
    return [out] + [grads[k] for k in sorted(grads) if grads[k] is not None]


def test_two_streams_equal_each_call_alone():
    probs = [(_problem("gru", "bf16", (1, 65536, 512), 4700), 0),
             (_problem("lstm", "f32", (2, 16384, 256), 4701), 0),
             (_problem("gru", "bf16", (1, 65536, 512), 4702), 2)]   # launch length 2: looping launches do work
    torch.cuda.synchronize()
    alone = []
    for p, fuse in probs:
        r = _run(p, fuse)
        torch.cuda.synchronize()
        alone.append([x.clone() for x in r])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(2):
        announce("round", rnd)
        got = [None] * len(probs)
        for i, (p, fuse) in enumerate(probs):
            with torch.cuda.stream(streams[(i + rnd) % 2]):
                got[i] = _run(p, fuse)
        torch.cuda.synchronize()
        for i in range(len(probs)):
            for j, (x, y) in enumerate(zip(got[i], alone[i])):
                assert torch.equal(x, y), (rnd, i, j)
