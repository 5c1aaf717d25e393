"""Checks of the seeded input generators (shapes, bf16 rounding, row addressability)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100000), rng.standard_t(3, 1000) * 1e3,
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40]]).astype(np.float32)
    mine = workloads.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f32(mine),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_rows_are_addressable():
    p, q = workloads.verify_logits("qwen", seqs=[3, 5], V=4096)
    p2, q2 = workloads.verify_logits("qwen", seqs=[5], V=4096)
    np.testing.assert_array_equal(p[1], p2[0])
    np.testing.assert_array_equal(q[1], q2[0])
    assert p.dtype == np.uint16 and p.shape == (2, 16, 4096)


def test_tiny_shapes_and_distribution():
    p, q = workloads.verify_logits("tiny")
    assert p.shape == (1, 8, 1024) and p.dtype == np.float32
    assert 1.7 < p.std() < 2.3
    assert 0.4 < (q - p).std() < 0.6


def test_noise_mask_layout():
    m = workloads.noise_row_mask(3, 4)
    np.testing.assert_array_equal(m, [0, 1, 1, 1] * 3)


def test_response_mask():
    m = workloads.tv_response_mask(2, 8, 3)
    np.testing.assert_array_equal(m, [0] * 5 + [1] * 3 + [0] * 5 + [1] * 3)
