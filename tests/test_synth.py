"""The seeded generators: determinism, shapes, and bf16 rounding equal to torch's RNE cast."""

import numpy as np
import torch

import synth


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.bf16_round(x), ref)
    bits = synth.bf16_bits(synth.bf16_round(x))
    np.testing.assert_array_equal(torch.from_numpy(bits).view(torch.bfloat16).float().numpy(), ref)


def test_generators_are_deterministic_and_shaped():
    a = synth.causal_inputs(B=1, T=8, H=2, d=16)
    b = synth.causal_inputs(B=1, T=8, H=2, d=16)
    for n in ("q", "k", "v", "dout"):
        np.testing.assert_array_equal(a[n], b[n])
        assert a[n].shape == (1, 8, 2, 16) and a[n].dtype == np.float32
        np.testing.assert_array_equal(a[n], synth.bf16_round(a[n]))
    t = synth.tiny_inputs()
    assert t["q"].shape == (1, 1, 1, 64) and t["k"].shape == (1, 16, 1, 64)
    assert 0.5 <= t["rms_gamma"].min() and t["rms_gamma"].max() <= 1.5
    l0 = synth.layer_inputs(0, T=4, H=2, d=8)
    l1 = synth.layer_inputs(1, T=4, H=2, d=8)
    assert not np.array_equal(l0["h"], l1["h"])
    assert abs(float(np.std(synth.layer_inputs(2, T=4, H=20, d=128)["W"])) - 0.02) < 1e-3
