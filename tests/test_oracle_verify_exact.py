"""Pins of the oracle's lossless verifier.

* Exact rational enumeration: the accept / residual rule reproduces p~ exactly.
* The implemented sampler, counted over the whole 2^24-point grid of its 24-bit
  uniforms, reproduces p~ within V * 2^-24 (a wrong comparison direction, a wrong
  residual sign or an off-by-one inverse CDF fails this).
* Acceptance probability equals sum min(p~, q~) = 1 - TV (closed form).
* Statistical checks through verify_block with Philox draws: slot marginals,
  acceptance rate, E[accept_len] = 1 + sum_j prod_{i<=j}(1 - TV_i), slot 0 = AR.
* The page's plateau statement (0.54 acceptance at block 8 ~ 2.1-2.2 tokens per
  step) fixes accept_len as the TPF numerator.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

from oracle.sampling import (EVENT_Q_ZERO, TIE_MASK, draft_sample, expected_accept_len,
                             filter_logits, verify_block, verify_slot)

N = 1 << 24
HERE = os.path.dirname(os.path.abspath(__file__))


def _frac_dist(f, V):
    d = [Fraction(0)] * V
    for i, p in zip(f.ids, f.probs):
        d[int(i)] = Fraction(float(p))
    s = sum(d)
    return [x / s for x in d]


def _random_pair(rng, V):
    zp = rng.normal(0, 1.5, V)
    zq = zp + rng.normal(0, 1.0, V)
    T = float(rng.choice([0.7, 1.0, 1.5]))
    k = int(rng.integers(0, V + 1))
    top_p = float(rng.choice([0.6, 0.9, 1.0]))
    return filter_logits(zp, T, k, top_p), filter_logits(zq, T, k, top_p)


def test_rule_is_exactly_lossless_in_rationals():
    rng = np.random.default_rng(11)
    for _ in range(60):
        V = int(rng.integers(2, 9))
        pf, qf = _random_pair(rng, V)
        p, q = _frac_dist(pf, V), _frac_dist(qf, V)
        res = [max(Fraction(0), p[x] - q[x]) for x in range(V)]
        rs = sum(res)
        marg = [Fraction(0)] * V
        for d in range(V):
            if q[d] == 0:
                continue
            a = min(Fraction(1), p[d] / q[d])
            marg[d] += q[d] * a
            for x in range(V):
                if rs:
                    marg[x] += q[d] * (1 - a) * res[x] / rs
        assert marg == p
        acc = sum(q[d] * min(Fraction(1), p[d] / q[d]) for d in range(V) if q[d])
        tv = sum(abs(p[x] - q[x]) for x in range(V)) / 2
        assert acc == 1 - tv == sum(min(p[x], q[x]) for x in range(V))


def _count_accept(pf, qf, d):
    """#grid points u_acc = j/2^24 the implemented rule accepts (monotone in j)."""
    lo, hi = 0, N            # accepted for j < lo, rejected for j >= hi
    if not verify_slot(pf, qf, d, 0.0, 0.0)[0]:
        return 0
    if verify_slot(pf, qf, d, (N - 1) / N, 0.0)[0]:
        return N
    lo, hi = 0, N - 1        # accept(lo) True, accept(hi) False
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if verify_slot(pf, qf, d, mid / N, 0.0)[0]:
            lo = mid
        else:
            hi = mid
    return hi


def _count_residual(pf, qf, d):
    """{token: #grid points u_res} of the rejection branch (token is monotone in u)."""
    tok = lambda j: verify_slot(pf, qf, d, (N - 1) / N, j / N)[1]
    counts = {}
    j = 0
    while j < N:
        x = tok(j)
        lo, hi = j, N        # tok(lo) == x; find first index with a different token
        if tok(N - 1) == x:
            hi = N
        else:
            hi = N - 1
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if tok(mid) == x:
                    lo = mid
                else:
                    hi = mid
        counts[x] = counts.get(x, 0) + (hi - j)
        j = hi
    return counts


def test_implemented_sampler_marginal_on_the_uniform_grid():
    rng = np.random.default_rng(12)
    for _ in range(25):
        V = int(rng.integers(2, 9))
        pf, qf = _random_pair(rng, V)
        p = _frac_dist(pf, V)
        marg = [Fraction(0)] * V
        res_counts = None
        for d, qd in zip(qf.ids, qf.probs):
            d = int(d)
            qd = Fraction(float(qd))
            na = _count_accept(pf, qf, d)
            marg[d] += qd * Fraction(na, N)
            if na < N:
                if res_counts is None:
                    # the residual does not depend on d as long as d is rejected
                    res_counts = _count_residual(pf, qf, d)
                for x, c in res_counts.items():
                    marg[x] += qd * Fraction(N - na, N) * Fraction(c, N)
        err = max(abs(float(marg[x] - p[x])) for x in range(V))
        assert err <= V * 2.0 ** -24, err


def test_acceptance_probability_is_one_minus_tv_on_the_grid():
    rng = np.random.default_rng(13)
    for _ in range(20):
        V = int(rng.integers(2, 9))
        pf, qf = _random_pair(rng, V)
        p, q = _frac_dist(pf, V), _frac_dist(qf, V)
        acc = sum(Fraction(float(qd)) * Fraction(_count_accept(pf, qf, int(d)), N)
                  for d, qd in zip(qf.ids, qf.probs))
        tv = sum(abs(p[x] - q[x]) for x in range(V)) / 2
        assert abs(float(acc - (1 - tv))) <= 2 * V * 2.0 ** -24


def _broadcast_block(rows_p, rows_q, S):
    p = np.broadcast_to(np.asarray(rows_p, np.float32), (S,) + np.shape(rows_p)).copy()
    q = np.broadcast_to(np.asarray(rows_q, np.float32), (S,) + np.shape(rows_q)).copy()
    return p, q


def _tv(a, b, V):
    pa, pb = np.zeros(V), np.zeros(V)
    pa[a.ids] = a.probs
    pb[b.ids] = b.probs
    return 0.5 * np.abs(pa - pb).sum()


def test_statistics_through_verify_block():
    rng = np.random.default_rng(14)
    V, b, S = 6, 4, 12000
    T, k, top_p = 1.0, 5, 0.95
    zp = rng.normal(0, 1.2, (b, V)).astype(np.float32)
    zq = (zp + rng.normal(0, 0.8, (b, V))).astype(np.float32)
    p, q = _broadcast_block(zp, zq, S)
    seq = np.arange(S, dtype=np.int64)
    pos = np.zeros(S, dtype=np.int64)
    d, _ = draft_sample(q, seq, pos, T, k, top_p, 5, dtype="f32")
    r = verify_block(p, q, d, seq, pos, T, k, top_p, 5, dtype="f32")
    pfs = [filter_logits(zp[i].astype(np.float64), T, k, top_p) for i in range(b)]
    qfs = [filter_logits(zq[i].astype(np.float64), T, k, top_p) for i in range(b)]
    # slot 0 is the AR sample: marginal p~_0, never rejected
    assert np.all(r["slot_accept"][:, 0] == 1) and np.all(r["accept_len"] >= 1)
    assert np.all(r["out_tokens"][:, 0] >= 0)
    for i in range(b):
        expect = np.zeros(V)
        expect[pfs[i].ids] = pfs[i].probs
        obs = np.bincount(r["slot_token"][:, i], minlength=V)
        sup = expect > 0
        assert obs[~sup].sum() == 0
        chi = stats.chisquare(obs[sup], expect[sup] * S)
        assert chi.pvalue > 1e-4, (i, chi)
    tvs = [0.0] + [_tv(pfs[i], qfs[i], V) for i in range(1, b)]
    for i in range(1, b):
        a = r["slot_accept"][:, i].mean()
        sd = math.sqrt((1 - tvs[i]) * tvs[i] / S)
        assert abs(a - (1 - tvs[i])) < 4 * sd + 1e-12
    e = expected_accept_len(tvs)
    L = r["accept_len"].astype(np.float64)
    assert abs(L.mean() - e) < 4 * L.std() / math.sqrt(S)
    # prefix structure of out_tokens
    for s in range(S):
        n = r["accept_len"][s]
        assert np.all(r["slot_accept"][s, 1:n] == 1)
        if n < b:
            assert r["slot_accept"][s, n] == 0
            assert r["out_tokens"][s, n] == r["resampled"][s]
            assert np.all(r["out_tokens"][s, n + 1:] == -1)
            assert np.all(r["out_tokens"][s, 1:n] == d[s, 1:n])
        else:
            assert r["resampled"][s] == -1


def test_identical_distributions_always_accept():
    rng = np.random.default_rng(15)
    z = rng.normal(0, 3, (2, 8, 300)).astype(np.float32)
    seq = np.arange(2)
    pos = np.array([0, 1000])
    d, _ = draft_sample(z, seq, pos, 1.0, 50, 0.95, 0, dtype="f32")
    r = verify_block(z, z, d, seq, pos, 1.0, 50, 0.95, 0, dtype="f32")
    assert np.all(r["accept_len"] == 8)
    assert np.all(r["out_tokens"][:, 1:] == d[:, 1:])


def test_greedy_accepts_iff_draft_is_base_argmax():
    rng = np.random.default_rng(16)
    zp = rng.normal(0, 3, (1, 6, 50)).astype(np.float32)
    zq = zp.copy()
    zq[0, 3] = rng.normal(0, 3, 50)        # slot 3's draft model disagrees
    d, _ = draft_sample(zq, [0], [0], 0.0, 0, 1.0, 0, dtype="f32")
    assert np.all(d[0] == np.argmax(zq[0], axis=-1))
    r = verify_block(zp, zq, d, [0], [0], 0.0, 0, 1.0, 0, dtype="f32")
    am = np.argmax(zp[0], axis=-1)
    assert r["out_tokens"][0, 0] == am[0]
    agree = [i for i in range(1, 6) if am[i] != d[0, i]]
    n = agree[0] if agree else 6
    assert r["accept_len"][0] == n
    if n < 6:
        assert r["resampled"][0] == am[n]


def test_draft_outside_support_is_rejected_and_counted():
    z = np.broadcast_to(-np.arange(100, dtype=np.float32) / 10, (1, 2, 100)).copy()
    z[0, :, 7] = 10.0
    z[0, :, 8] = 9.0
    d = np.array([[0, 50]], np.int32)     # token 50 is outside the top-k 5 set
    r = verify_block(z, z, d, [0], [0], 1.0, 5, 1.0, 0, dtype="f32")
    assert r["accept_len"][0] == 1
    assert int(r["diag"][0, 1, 3]) & EVENT_Q_ZERO
    assert r["resampled"][0] in (7, 8)


def test_page_plateau_fixes_the_tpf_numerator():
    with open(os.path.join(HERE, "golden", "tpf_plateau.json")) as f:
        g = json.load(f)
    alpha, b = g["per_position_acceptance"], g["block"]
    tpf = expected_accept_len([0.0] + [1.0 - alpha] * (b - 1))
    assert g["tpf_low"] <= tpf <= g["tpf_high"]
    # counting the resampled token as well would leave the stated range
    assert tpf + (1 - alpha ** (b - 1)) > g["tpf_high"] + 0.5


def test_no_near_ties_on_tiny_workload():
    import workloads
    p, q = workloads.verify_logits("tiny")
    sp = workloads.SAMPLING
    seq, pos = np.arange(1), np.zeros(1, np.int64)
    d, dflags = draft_sample(q, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], "f32")
    r = verify_block(p, q, d, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], "f32")
    assert r["accept_len"][0] >= 1
    assert not np.any(r["diag"][..., 3].astype(int) & TIE_MASK)
