"""GPU parity at a maximum size: more than 2^30 elements in one [B][T][D] plane, so that a lane's
offset no longer fits 32 bits and the kernels take their 64-bit addressing path (the full-tile
buffer-load path is only used below that size).  Checked on sampled channels against the oracle.

B=1, T=1100 (ragged against the 128-step chunk), D=2^20: 1.15e9 elements, bf16 gate inputs
(6.9 GB on the host, 2.3 GB per plane on the GPU), fp32 trajectory and gradients (4.6 GB per plane).
The inputs are drawn plane by plane with the benchmark distributions (U ~ N(0, 1) rounded to bf16,
w ~ U(-0.5, 0.5), biases ~ N(0, 0.01)) from one seeded stream, in chunks to bound host memory.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import max_abs
from nonlinear_rnn_solve_amd import api, synth

pytestmark = pytest.mark.gpu

B, T, D = 1, 1100, 1 << 20


def draw_bf16_plane(rng, n, chunk=1 << 26):
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = synth.f32_to_bf16_bits(rng.standard_normal(size=m, dtype=np.float32))
    return out


def test_newton_and_vjp_beyond_32_bit_offsets():
    print("[case] max size", B, T, D, flush=True)
    rng = np.random.Generator(np.random.PCG64(2900))
    N = B * T * D
    pre_bits = [draw_bf16_plane(rng, N).reshape(B, T, D) for _ in range(3)]
    w = rng.uniform(-0.5, 0.5, size=(3, D)).astype(np.float32)
    bias = (rng.standard_normal(size=(3, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    g_sample_seed = 2901
    pre = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).cuda() for p in pre_bits]
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda()
    K = 3
    H, rep = api.newton_solve("gru", pre, wt, bt, max_iters=K)
    ds = np.array([0, 1, 63, 64, 777777, D - 65, D - 2, D - 1])
    idx = torch.from_numpy(ds).cuda()
    got = H[0, 0][:, idx].cpu().numpy()                           # [T, n]
    sub = [np.ascontiguousarray(p[0][:, ds][None]) for p in pre_bits]
    prob = oracle.Problem("gru", sub, w[:, ds], bias[:, ds], dtype=oracle.BF16)
    ref, res, *_ = oracle.newton(prob, K)
    err = max_abs(got, ref[0, 0])
    print("  newton max abs err", err, "residuals", rep.residuals, "oracle", list(res), flush=True)
    assert err <= 1e-4
    # the GPU's residual is the maximum over all channels, the oracle's over the sampled ones
    assert all(r >= q * (1 - 1e-3) for r, q in zip(rep.residuals, res))
    # the VJP at the GPU's trajectory, with an upstream gradient that is nonzero on the sampled channels
    g = torch.zeros((B, T, D), device="cuda")
    gs = np.random.default_rng(g_sample_seed).standard_normal((T, len(ds))).astype(np.float32)
    g[0][:, idx] = torch.from_numpy(gs).cuda()
    out = api.scan_vjp("gru", pre, H, g, wt, bt, want_lambda=True)
    traj = H[0, 0][:, idx].cpu().numpy().astype(np.float64)[None, None]
    vref = oracle.vjp(prob, traj, gs[None])
    lam = out["lam"][0, 0][:, idx].cpu().numpy()
    dpre = torch.stack([out["d_pre"][k, 0][:, idx] for k in range(3)]).cpu().numpy()
    e_lam = float(np.max(np.abs(lam - vref["lam"][0, 0]) / np.maximum(1, np.abs(vref["lam"][0, 0]))))
    e_dp = float(np.max(np.abs(dpre - vref["d_pre"][:, 0]) / np.maximum(1, np.abs(vref["d_pre"][:, 0]))))
    dw = out["d_w"].cpu().numpy()[:, ds]
    e_dw = float(np.max(np.abs(dw - vref["d_w"]) / (1 + np.abs(vref["d_w"]))))
    print("  vjp lambda", e_lam, "d_pre", e_dp, "d_w", e_dw, flush=True)
    assert e_lam <= 1e-4 and e_dp <= 1e-4 and e_dw <= 1e-4


def test_head_gru_beyond_32_bit_element_offsets():
    """The head-wise block GRU with more than 2^31 elements per plane (B=4200, T=1000, D=512: 2.15e9), so
    that element offsets of the later batch rows exceed 32 bits; fp32 gate inputs tiled from a seeded pool of
    2^26 + 7 draws (the period is prime to every stride, so rows differ).  The Newton iterate and the VJP are
    checked on sampled batch rows (all heads) against the oracle; the last row's offsets exceed 2^31."""
    Bh, Th, Dh, hs = 4200, 1000, 512, 64
    print("[case] head max size", Bh, Th, Dh, flush=True)
    rng = np.random.Generator(np.random.PCG64(2950))
    N = Bh * Th * Dh
    assert N > (1 << 31)
    pool = rng.standard_normal(size=(1 << 26) + 7, dtype=np.float32)
    planes = [np.resize(np.roll(pool, 977 * g), N).reshape(Bh, Th, Dh) for g in range(3)]
    w = ((rng.random(size=(3, Dh // hs, hs, hs), dtype=np.float32) - np.float32(0.5)) *
         np.float32(2.0 / np.sqrt(hs))).astype(np.float32)
    bias = (rng.standard_normal(size=(3, Dh), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    pre = [torch.from_numpy(p).cuda() for p in planes]
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda()
    K = 2
    H, rep = api.newton_solve("head_gru", pre, wt, bt, max_iters=K)
    rows = [0, 2049, Bh - 1]
    sub = [np.ascontiguousarray(p[rows]) for p in planes]
    prob = oracle.Problem("head_gru", sub, w, bias, head_size=hs)
    ref, res, *_ = oracle.newton(prob, K)
    got = H[0][torch.tensor(rows, device="cuda")].cpu().numpy()
    err = max_abs(got, ref[0])
    print("  newton max abs err", err, "residuals", rep.residuals, "oracle", list(res), flush=True)
    assert err <= 1e-5
    assert all(r >= q * (1 - 1e-3) for r, q in zip(rep.residuals, res))
    api._ws_cache.clear()           # release the Newton workspace (86 GB) before the VJP's
    torch.cuda.empty_cache()
    g = torch.zeros((Bh, Th, Dh), device="cuda")
    gs = np.random.default_rng(2951).standard_normal((len(rows), Th, Dh)).astype(np.float32)
    g[torch.tensor(rows, device="cuda")] = torch.from_numpy(gs).cuda()
    out = api.scan_vjp("head_gru", pre, H, g, wt, bt, want_s0=False)
    traj = got.astype(np.float64)[None]
    vref = oracle.vjp(prob, traj, gs)
    dpre = out["d_pre"][:, torch.tensor(rows, device="cuda")].cpu().numpy()
    e_dp = float(np.max(np.abs(dpre - vref["d_pre"]) / np.maximum(1, np.abs(vref["d_pre"]))))
    # only the sampled rows carry a gradient, so the parameter sums are the oracle's over those rows
    dw = out["d_w"].cpu().numpy()
    e_dw = float(np.max(np.abs(dw - vref["d_w"]) / (1 + np.abs(vref["d_w"]))))
    print("  vjp d_pre", e_dp, "d_w", e_dw, flush=True)
    assert e_dp <= 1e-4 and e_dw <= 1e-4
    del pre, H, g, out
    api._ws_cache.clear()
    torch.cuda.empty_cache()
