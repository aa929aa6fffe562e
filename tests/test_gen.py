"""The synthetic input generator: bf16 rounding, determinism, distribution."""
import numpy as np
import torch

from sparse_decode_attention_amd import gen
from sparse_decode_attention_amd.configs import WORKLOADS


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 1e3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact halfway cases
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_seeded():
    w = WORKLOADS["tiny_s1k"].with_(S=64)
    a = gen.numpy_layer(w, seed=3, steps=2)
    b = gen.numpy_layer(w, seed=3, steps=2)
    c = gen.numpy_layer(w, seed=4, steps=2)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert a["q_win"].shape == (1, 32, 32, 128) and a["k"].shape == (1, 8, 64, 128)
    assert a["q_dec"].shape == (2, 1, 32, 128)


def test_channel_cv_closed_form():
    """|k| = |z| s_c e_tc: the per-channel CV over tokens is
    sqrt(E[z^2]E[e^2] / (E|z|^2 E[e]^2) - 1) = sqrt(pi e / 2 - 1) ~ 1.808 (> 1)."""
    w = WORKLOADS["tiny_s1k"].with_(S=65536)
    k = gen.bf16_bits_to_f32(gen.numpy_tensor(0, w.cfg_id, gen.T_K, 0, 0, 1, 8, w.S, 128)).astype(np.float64)
    s = gen.channel_scales(0, w.cfg_id, gen.T_K, 0, 8, 128).astype(np.float64)
    x = np.abs(k[0]) / s[:, None, :]
    m1, m2 = x.mean(), (x * x).mean()
    cv = np.sqrt(m2 / m1 ** 2 - 1)
    assert abs(cv - np.sqrt(np.pi * np.e / 2 - 1)) < 0.03, cv
