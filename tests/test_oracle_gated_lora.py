"""Pins of the oracle's row-gated LoRA linear layer.

* Exact rational triple loops on tiny shapes.
* Noise rows equal the merged-weight form X (W + s B A)^T; seed rows equal X W^T
  exactly; the delta is linear in the scale.
"""
from fractions import Fraction

import numpy as np

import workloads
from oracle.gated_lora import bf16_bits_to_f64, gated_lora_linear, lora_delta


def test_exact_rational_triple_loop():
    M, K, N, r = 3, 8, 5, 2
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=3, tag=7)
    mask = np.array([0, 1, 1], np.uint8)
    s = 16.0
    Y = gated_lora_linear(X, W, A, B, mask, s)
    x, w, a, bb = (bf16_bits_to_f64(v) for v in (X, W, A, B))
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(x[m, k]) * Fraction(w[n, k]) for k in range(K))
            if mask[m]:
                for j in range(r):
                    t = sum(Fraction(x[m, k]) * Fraction(a[j, k]) for k in range(K))
                    acc += Fraction(s) * t * Fraction(bb[n, j])
            assert abs(float(acc) - Y[m, n]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_merged_weight_form_and_seed_rows():
    M, K, N, r = 8, 256, 256, 16
    X, W, A, B = workloads.gemm_inputs(M, K, N, r)
    mask = workloads.noise_row_mask(1, 8)
    for s in (1.0, 16.0):
        Y = gated_lora_linear(X, W, A, B, mask, s)
        x, w, a, bb = (bf16_bits_to_f64(v) for v in (X, W, A, B))
        merged = x @ (w + s * bb @ a).T
        np.testing.assert_allclose(Y[1:], merged[1:], rtol=1e-10, atol=1e-12)
        Y0 = gated_lora_linear(X, W, A, B, np.zeros(M, np.uint8), s)
        np.testing.assert_array_equal(Y[0], Y0[0])
        # the delta is what separates noise rows from seed rows
        np.testing.assert_allclose(Y[1:] - Y0[1:], lora_delta(X, A, B, s)[1:], rtol=1e-9, atol=1e-13)


def test_delta_linear_in_scale():
    X, W, A, B = workloads.gemm_inputs(4, 64, 32, 8, seed=1)
    mask = np.ones(4, np.uint8)
    y1 = gated_lora_linear(X, W, A, B, mask, 1.0)
    y0 = gated_lora_linear(X, W, A, B, mask, 0.0)
    y16 = gated_lora_linear(X, W, A, B, mask, 16.0)
    np.testing.assert_allclose(y16 - y0, 16 * (y1 - y0), rtol=1e-9, atol=1e-14)
