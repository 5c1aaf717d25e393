"""Pins of the decode-step oracle (oracle/step.py) to library routines, exact
arithmetic and closed forms: no GPU needed.

* rmsnorm, SiLU and the one-token-context attention against torch's own
  rms_norm, silu and scaled_dot_product_attention (with grouped kv heads);
* the noise token against exact rational arithmetic on numpy's Philox words, and
  its uniformity over the vocabulary;
* the forward against structure the reading fixes: loops share weights (two loops
  equal a stack with its layers listed twice), rows are independent (a row
  permutation permutes the logits), and a stack with zero projection weights
  gives rmsnorm(embed[token]) lm_head^T exactly;
* the whole step against a closed form: for a model whose greedy output repeats
  its input token, every draft is kept, so a greedy step commits the seed followed
  by the block's noise tokens, and the AR step returns its input token.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import step as ostep

SMALL = dict(hidden=256, kv_width=64, head_dim=32, ffn=512, vocab=1000, layers=2, rank=32, b=8, S=3, loops=1)


def test_rmsnorm_matches_torch():
    x = np.random.default_rng(0).normal(0, 3, (7, 96))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), eps=ostep.NORM_EPS).numpy()
    np.testing.assert_allclose(ostep.rmsnorm(x), ref, rtol=1e-13, atol=0)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(ostep.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("hidden,kv_width,head_dim", [(256, 64, 32), (384, 384, 64), (512, 128, 128)])
def test_one_token_attention_matches_sdpa(hidden, kv_width, head_dim):
    """Each row attends over a context of itself alone (grouped kv heads)."""
    rng = np.random.default_rng(1)
    M = 5
    q = torch.from_numpy(rng.normal(size=(M, hidden // head_dim, 1, head_dim)))
    k = torch.from_numpy(rng.normal(size=(M, kv_width // head_dim, 1, head_dim)))
    v_np = rng.normal(size=(M, kv_width))
    v = torch.from_numpy(v_np).reshape(M, kv_width // head_dim, 1, head_dim)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, enable_gqa=True)
    ref = ref.reshape(M, hidden).numpy()
    np.testing.assert_allclose(ostep.one_token_attention(v_np, hidden, head_dim), ref, rtol=1e-12, atol=1e-12)


def test_noise_token_is_the_exact_scaled_uniform():
    """floor(u * V) with u = (w >> 40) / 2^24 for numpy's Philox word (numpy
    pre-increments its counter, so it starts at counter - 1)."""
    for seq, pos, V in [(0, 0, 151936), (3, 17, 166144), (2**40 + 5, 999, 7), (11, 2**33, 1)]:
        key = np.array([123, seq], dtype=np.uint64)
        ctr = np.array([(pos - 1) % 2**64, 2, 0, 0], dtype=np.uint64) if pos > 0 else \
            np.array([2**64 - 1, 1, 0, 0], dtype=np.uint64)
        w = int(np.random.Philox(key=key, counter=ctr).random_raw(4)[0])
        assert oracle.noise_token(123, seq, pos, V) == math.floor(Fraction(w >> 40, 2**24) * V)


def test_noise_tokens_are_uniform():
    from scipy import stats
    V, n = 13, 26000
    counts = np.bincount([oracle.noise_token(5, s, 100 + s % 7, V) for s in range(n)], minlength=V)
    assert counts.sum() == n and counts.shape == (V,)
    assert stats.chisquare(counts).pvalue > 1e-4


def _model(cfg=SMALL, seed=0):
    return workloads.step_model_host(cfg, seed=seed)


def test_two_loops_equal_the_layers_listed_twice():
    m = _model()
    rng = np.random.default_rng(2)
    toks = rng.integers(0, SMALL["vocab"], 6)
    mask = np.array([0, 1, 1, 0, 1, 1], np.uint8)
    twice = dict(m, weights=m["weights"] * 2, lora_a=m["lora_a"] * 2, lora_b=m["lora_b"] * 2)
    np.testing.assert_array_equal(ostep.forward(m, toks, mask, loops=2), ostep.forward(twice, toks, mask, loops=1))


def test_rows_are_independent():
    m = _model()
    rng = np.random.default_rng(3)
    toks = rng.integers(0, SMALL["vocab"], 8)
    mask = (rng.random(8) < 0.5).astype(np.uint8)
    perm = rng.permutation(8)
    a = ostep.forward(m, toks, mask)
    b = ostep.forward(m, toks[perm], mask[perm])
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_zero_projections_leave_the_embedding():
    m = _model()
    zero = [[np.zeros_like(w) for w in layer] for layer in m["weights"]]
    mz = dict(m, weights=zero, rank=0)
    toks = np.array([0, 5, 999, 5])
    h = oracle.bf16_bits_to_f64(m["embed"][toks])
    x = oracle.bf16_bits_to_f64(ostep.to_bf16_bits(h / np.sqrt((h * h).mean(1, keepdims=True) + 1e-6)))
    ref = x @ oracle.bf16_bits_to_f64(m["lm_head"]).T
    np.testing.assert_allclose(ostep.forward(mz, toks, None, loops=2), ref, rtol=1e-12, atol=1e-12)


def identity_model(cfg=SMALL, seed=4):
    """Zero projection weights and lm_head = embed: logits rmsnorm(e_t) . e_v peak at
    v = t (|e_t|^2 ~ H against cross terms ~ sqrt(H) for random rows)."""
    m = _model(cfg, seed)
    return dict(m, weights=[[np.zeros_like(w) for w in layer] for layer in m["weights"]],
                lm_head=m["embed"].copy())


def test_identity_model_keeps_every_draft():
    m = identity_model()
    S, b, V = 3, 8, SMALL["vocab"]
    seed_tok = np.array([7, 500, 999])
    seq = np.array([0, 1, 2**40], dtype=np.int64)
    pos = np.array([10, 0, 12345], dtype=np.int64)
    r = ostep.decode_step(m, seed_tok, seq, pos, b, 0.0, 50, 0.95, seed=9, draft_loops=1, verify_loops=2)
    assert np.all(r["accept_len"] == b) and np.all(r["resampled"] == -1)
    for s in range(S):
        expect = [seed_tok[s]] + [oracle.noise_token(9, seq[s], pos[s] + i, V) for i in range(1, b)]
        np.testing.assert_array_equal(r["out_tokens"][s], expect)
        np.testing.assert_array_equal(r["drafts"][s, 1:], expect[1:])
    tok, _ = ostep.ar_step(m, seed_tok, seq, pos, 0.0, 50, 0.95, seed=9, loops=2)
    np.testing.assert_array_equal(tok, seed_tok)


def test_step_slot0_is_the_ar_step():
    """The first position of a step is the AR token of the same seed, sequence and
    position (sampled decoding, a random stack)."""
    m = _model()
    seed_tok = np.array([1, 2, 3])
    seq = np.arange(3, dtype=np.int64)
    pos = np.array([5, 6, 7], dtype=np.int64)
    r = ostep.decode_step(m, seed_tok, seq, pos, 4, 1.0, 50, 0.95, seed=3)
    tok, _ = ostep.ar_step(m, seed_tok, seq, pos, 1.0, 50, 0.95, seed=3)
    np.testing.assert_array_equal(r["out_tokens"][:, 0], tok)
    assert np.all((r["accept_len"] >= 1) & (r["accept_len"] <= 4))
