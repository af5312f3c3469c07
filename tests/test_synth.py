"""The seeded generators: recipe checks (no method arithmetic involved)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(20000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -1.5, 1.00390625, 1.01171875], np.float32)])
    bits = synth.round_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits),
                                  torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_workload_recipes():
    s3 = synth.WORKLOADS["gmpo_kl_bf16_b8_t2048"]
    a = synth.advantages(s3)
    assert (a == 0).sum() == 2
    P = synth.prompt_lengths(s3)
    assert P.min() >= 64 and P.max() <= 512
    m = synth.completion_mask(s3).reshape(s3.B, s3.T)
    assert all(m[i].sum() == s3.T - P[i] for i in range(s3.B))
    s1 = synth.WORKLOADS["tiny_gmpo_f32"]
    assert set(synth.advantages(s1).tolist()) <= {1.0, -1.0, 0.0}
    assert synth.completion_mask(s1).reshape(2, 16)[:, :4].sum() == 0
    y = synth.targets(synth.WORKLOADS["gmpo_bf16_b1_t512"])
    assert y.min() >= 0 and y.max() < 151936 and y.dtype == np.int64


def test_hidden_row_subset_consistent():
    s = synth.small(B=3, T=3000, H=16, V=50)
    h, raw = synth.hidden(s)
    rows = np.array([0, 5, 4095, 4096, 8999, 4097])
    hs, raws = synth.hidden(s, rows)
    np.testing.assert_array_equal(hs, h[rows])
    np.testing.assert_array_equal(raws, raw[rows])
