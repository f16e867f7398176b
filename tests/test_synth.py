"""The seeded input generator: bf16 rounding, determinism, distributions."""
import numpy as np
import torch

from nonlinear_rnn_solve_amd import synth


def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = synth.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (mine.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
        (rng.standard_normal(10000) * 1e-38).astype(np.float32),
        # exact ties: low 16 bits = 0x8000, both parities of the kept bit
        (np.arange(1000, dtype=np.uint32) * np.uint32(0x20000) + np.uint32(0x3F808000)).view(np.float32),
        (np.arange(1000, dtype=np.uint32) * np.uint32(0x20000) + np.uint32(0x3F818000)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38], np.float32),
    ])
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_inputs_are_deterministic_and_seed_dependent():
    a = synth.make_inputs("gru", 1, 64, 8, "bf16", seed=5, with_grad=True)
    b = synth.make_inputs("gru", 1, 64, 8, "bf16", seed=5, with_grad=True)
    c = synth.make_inputs("gru", 1, 64, 8, "bf16", seed=6, with_grad=True)
    for x, y in zip(a.pre + [a.w, a.bias, a.g], b.pre + [b.w, b.bias, b.g]):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.pre[0], c.pre[0])


def test_distributions():
    inp = synth.make_inputs("lstm", 2, 2048, 64, seed=1)
    for p in inp.pre:
        assert abs(p.mean()) < 0.01 and abs(p.std() - 1) < 0.01
    assert inp.w.min() >= -0.5 and inp.w.max() < 0.5
    assert np.all(inp.bias[1] == 1.0)
    assert abs(inp.bias[[0, 2, 3]].std() - 0.1) < 0.02
    lin = synth.make_inputs("linear", 1, 4096, 64, seed=2)
    a, b = lin.pre
    assert a.min() > 0 and a.max() < 1 and abs(a.mean() - 0.5) < 0.01
    assert abs(b.std() - 1) < 0.01


def test_workload_table():
    assert [w.index for w in synth.WORKLOADS] == [0, 1, 2, 3, 4]
    wl = synth.WORKLOADS[4]
    assert (wl.B, wl.T, wl.D, wl.dtype, wl.tol, wl.max_iters, wl.vjp) == (1, 131072, 1024, "bf16", 1e-5, 8, True)
    small = synth.workload_inputs(synth.WORKLOADS[0])
    assert small.pre[0].shape == (1, 256, 16) and small.pre[0].dtype == np.float32
