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


# --- backward ------------------------------------------------------------------

from oracle.gated_lora import gated_lora_linear_bwd  # noqa: E402


def test_backward_matches_torch_autograd():
    """The oracle's gradients equal torch.autograd's on the fp64 forward."""
    import torch
    M, K, N, r = 6, 32, 24, 8
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=5, tag=2)
    G = workloads.gemm_grad(M, N, seed=5)
    mask = np.array([0, 1, 1, 0, 1, 1], np.uint8)
    s = 16.0
    dx, da, db = gated_lora_linear_bwd(X, W, A, B, mask, s, G)
    x, w, a, bb, g = (torch.tensor(bf16_bits_to_f64(v), dtype=torch.float64) for v in (X, W, A, B, G))
    x.requires_grad_(True)
    a.requires_grad_(True)
    bb.requires_grad_(True)
    w.requires_grad_(True)
    m = torch.tensor(mask, dtype=torch.float64)[:, None]
    y = torch.nn.functional.linear(x, w) + s * m * torch.nn.functional.linear(torch.nn.functional.linear(x, a), bb)
    (y * g).sum().backward()
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(da, a.grad.numpy(), rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(db, bb.grad.numpy(), rtol=1e-12, atol=1e-16)


def test_backward_exact_rational_adapter_gradients():
    M, K, N, r = 3, 4, 5, 2
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=9, tag=1)
    G = workloads.gemm_grad(M, N, seed=9)
    mask = np.array([1, 0, 1], np.uint8)
    s = 2.0
    _, da, db = gated_lora_linear_bwd(X, W, A, B, mask, s, G)
    x, a, bb, g = (bf16_bits_to_f64(v) for v in (X, A, B, G))
    F = Fraction
    for j in range(r):
        for k in range(K):
            # dL/dA[j,k] = s * sum_m mask_m * (sum_n g[m,n] B[n,j]) * X[m,k]
            acc = sum(F(s) * F(int(mask[m])) * sum(F(g[m, n]) * F(bb[n, j]) for n in range(N)) * F(x[m, k])
                      for m in range(M))
            assert abs(float(acc) - da[j, k]) <= 1e-13 * max(1e-30, abs(float(acc)))
    for n in range(N):
        for j in range(r):
            # dL/dB[n,j] = s * sum_m mask_m * g[m,n] * (sum_k X[m,k] A[j,k])
            acc = sum(F(s) * F(int(mask[m])) * F(g[m, n]) * sum(F(x[m, k]) * F(a[j, k]) for k in range(K))
                      for m in range(M))
            assert abs(float(acc) - db[n, j]) <= 1e-13 * max(1e-30, abs(float(acc)))


def test_backward_seed_rows_and_linearity():
    M, K, N, r = 8, 64, 48, 8
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=2)
    G = workloads.gemm_grad(M, N, seed=2)
    zero = np.zeros(M, np.uint8)
    dx, da, db = gated_lora_linear_bwd(X, W, A, B, zero, 16.0, G)
    # no noise rows: the adapter gets no gradient and dX is the plain dY W
    assert np.all(da == 0.0) and np.all(db == 0.0)
    np.testing.assert_allclose(dx, bf16_bits_to_f64(G) @ bf16_bits_to_f64(W), rtol=1e-12, atol=1e-16)
    # gradients are linear in the scale's adapter part and in the mask rows
    mask = workloads.noise_row_mask(1, 8)
    dx1, da1, db1 = gated_lora_linear_bwd(X, W, A, B, mask, 1.0, G)
    dx2, da2, db2 = gated_lora_linear_bwd(X, W, A, B, mask, 2.0, G)
    np.testing.assert_allclose(da2, 2 * da1, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(db2, 2 * db1, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(dx2 - dx, 2 * (dx1 - dx), rtol=1e-9, atol=1e-18)
