"""Pins of the oracle's TV self-distillation loss and its gradient.

* torch.autograd (fp64, CPU) of the loss written as 1 - sum min(p, q) gives the
  gradient the oracle computes in closed form.
* Central finite differences.
* Shift invariance: each gradient row sums to zero.
* TV(p, p) = 0 with zero gradient; disjoint supports give TV -> 1; TV in [0, 1].
* 1 - TV equals the verifier's exact acceptance probability with the filters off
  (the page's identity between the loss and lossless acceptance).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle.sampling import filter_logits
from oracle.tv import tv_loss_fwd_bwd


def _f32_rows(rng, R, V, s1=3.0, s2=1.0):
    t = (s1 * rng.standard_normal((R, V))).astype(np.float32)
    s = (t + s2 * rng.standard_normal((R, V))).astype(np.float32)
    return t, s


@pytest.mark.parametrize("T", [1.0, 0.7, 2.0])
def test_gradient_matches_autograd(T):
    rng = np.random.default_rng(21)
    R, V = 6, 40
    t, s = _f32_rows(rng, R, V)
    mask = np.array([1, 0, 1, 1, 0, 1], np.uint8)
    loss, tv, grad = tv_loss_fwd_bwd(t, s, mask, T, dtype="f32")
    tt = torch.tensor(t, dtype=torch.float64)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(tt / T, dim=-1)
    q = torch.softmax(st / T, dim=-1)
    tv_t = 1.0 - torch.minimum(p, q).sum(dim=-1)
    m = torch.tensor(mask, dtype=torch.float64)
    L = (tv_t * m).sum() / m.sum()
    L.backward()
    assert abs(loss - L.item()) < 1e-14
    np.testing.assert_allclose(tv[mask == 1], tv_t.detach().numpy()[mask == 1], rtol=1e-12)
    assert np.all(tv[mask == 0] == 0)
    np.testing.assert_allclose(grad, st.grad.numpy(), rtol=1e-10, atol=1e-16)


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(22)
    R, V = 2, 25
    t, s = _f32_rows(rng, R, V)
    t64, s64 = t.astype(np.float64), s.astype(np.float64)
    mask = np.ones(R, np.uint8)

    def loss_of(s_):
        p = np.exp(t64 - t64.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
        q = np.exp(s_ - s_.max(-1, keepdims=True)); q /= q.sum(-1, keepdims=True)
        return 0.5 * np.abs(p - q).sum() / R

    _, _, grad = tv_loss_fwd_bwd(t, s, mask, 1.0, dtype="f32")
    h = 1e-6
    for r in range(R):
        for j in range(V):
            sp, sm = s64.copy(), s64.copy()
            sp[r, j] += h
            sm[r, j] -= h
            fd = (loss_of(sp) - loss_of(sm)) / (2 * h)
            assert abs(fd - grad[r, j]) < 1e-7 + 1e-5 * abs(grad[r, j])


def test_rows_sum_to_zero_and_range():
    rng = np.random.default_rng(23)
    t, s = _f32_rows(rng, 16, 500)
    mask = (rng.random(16) < 0.7).astype(np.uint8)
    mask[0] = 1
    loss, tv, grad = tv_loss_fwd_bwd(t, s, mask, 1.0, dtype="f32")
    assert np.all(np.abs(grad.sum(-1)) < 1e-15)
    assert np.all((tv >= 0) & (tv <= 1))
    assert np.all(grad[mask == 0] == 0)
    assert 0 <= loss <= 1


def test_identical_and_disjoint():
    rng = np.random.default_rng(24)
    t, _ = _f32_rows(rng, 3, 100)
    loss, tv, grad = tv_loss_fwd_bwd(t, t, np.ones(3, np.uint8), 1.0, dtype="f32")
    assert loss == 0 and np.all(tv == 0) and np.all(grad == 0)
    a = np.full((1, 10), -200.0, np.float32)
    b = a.copy()
    a[0, 0] = 200.0
    b[0, 1] = 200.0
    loss, tv, _ = tv_loss_fwd_bwd(a, b, np.ones(1, np.uint8), 1.0, dtype="f32")
    assert abs(tv[0] - 1.0) < 1e-15


def test_empty_mask_gives_zero_loss_and_gradient():
    rng = np.random.default_rng(25)
    t, s = _f32_rows(rng, 4, 50)
    loss, tv, grad = tv_loss_fwd_bwd(t, s, np.zeros(4, np.uint8), 1.0, dtype="f32")
    assert loss == 0.0 and np.all(tv == 0) and np.all(grad == 0)


def test_bf16_decoding_and_workload_rows():
    t, s = workloads.tv_rows([0, 1], 2000)
    loss, tv, grad = tv_loss_fwd_bwd(t, s, np.ones(2, np.uint8), 1.0, dtype="bf16")
    tf = workloads.bf16_bits_to_f32(t).astype(np.float64)
    sf = workloads.bf16_bits_to_f32(s).astype(np.float64)
    loss2, tv2, _ = tv_loss_fwd_bwd(tf.astype(np.float32), sf.astype(np.float32),
                                    np.ones(2, np.uint8), 1.0, dtype="f32")
    assert loss == loss2
    assert 0.2 < loss < 0.6


def test_one_minus_tv_is_exact_acceptance_with_filters_off():
    from test_oracle_verify_exact import _count_accept, N
    rng = np.random.default_rng(26)
    for _ in range(10):
        V = int(rng.integers(2, 8))
        t, s = _f32_rows(rng, 1, V, 1.5, 1.0)
        _, tv, _ = tv_loss_fwd_bwd(t, s, np.ones(1, np.uint8), 1.0, dtype="f32")
        pf = filter_logits(t[0].astype(np.float64), 1.0, 0, 1.0)
        qf = filter_logits(s[0].astype(np.float64), 1.0, 0, 1.0)
        acc = sum(float(qd) * _count_accept(pf, qf, int(d)) / N for d, qd in zip(qf.ids, qf.probs))
        assert abs(acc - (1.0 - tv[0])) < 2 * V * 2.0 ** -24
