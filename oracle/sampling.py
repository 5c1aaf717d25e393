"""Plain fp64 CPU oracle of the Uno (Psi-Spec) lossless block verifier.

TEST INFRASTRUCTURE ONLY. Nothing in the product library imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP path.

What it follows (page titles as headed on the pages):

* "LoopUno: Turning Agentic Looped LLMs into Diffusion LLMs in One Hour",
  section "How it works" -> "The model drafts with noise and verifies with itself":
  a block of positions is drafted in one forward, the unmodified model verifies
  them and the longest correct prefix is kept; the first position is always the
  exact autoregressive token, so a step never moves backward.
* Same page, "How it works" -> "Training is self-distillation": under lossless
  verification the acceptance probability of a position is exactly 1 - TV(p, q).
  The rule that has this property and keeps the output distribution equal to the
  base model's is: accept a draft d with probability min(1, p(d)/q(d)); at the
  first rejection draw from normalise(max(0, p - q)).
* "Uno Qwen3-8B" model card, "Evaluation protocol" table: temperature 1.0,
  top-p 0.95, top-k 50, block size 16, one sample per problem.

Readings taken where the pages are silent (each is listed in the design notes):

* Filter order: temperature -> top-k -> top-p on the renormalised top-k set ->
  renormalise; applied to the base logits (p) and draft logits (q) alike.
* Top-k is tie-inclusive: keep v iff z_v >= the k-th largest logit counted with
  multiplicity (selected on raw logits; T > 0 is monotone). top_k <= 0 or
  top_k >= V switches it off.
* Top-p is tie-grouped: keep v iff the mass of tokens with strictly larger
  probability is < top_p; the top group is always kept. top_p >= 1 switches it
  off.
* temperature <= 0 is greedy: one-hot at the argmax, lowest id on ties.
* Slot 0 is the AR token: inverse CDF of p~_0 at u_res. Slots i >= 1 accept iff
  u_acc < p~(d)/q~(d) (strict; u in [0,1)). q~(d) == 0 rejects (counted). A
  zero residual mass after a rejection draws from p~ instead (counted).
* accept_len = index of the first rejected slot (b if none); out_tokens holds the
  kept tokens, then the resampled token, then -1.
* Inverse CDF: tokens in ascending id order, weights w, C_j their sequential
  fp64 prefix sums, Z = C_last; return the first j with u*Z < C_j.
* All arithmetic on the filtered sets is fp64; sums run sequentially in the
  stated order.
"""

import math

import numpy as np

from .philox import STREAM_DRAFT, STREAM_VERIFY, slot_uniforms

NEAR_TIE = 1e-6

# Bits of the per-slot flag word (diag[..., 3]).
TIE_ACCEPT = 1        # |u_acc - p~(d)/q~(d)| < 1e-6
TIE_TOPP_P = 2        # base row: a top-p group boundary lies within 1e-6 of top_p
TIE_TOPP_Q = 4        # draft row: same
TIE_ICDF = 8          # the inverse-CDF draw that made the token is within 1e-6*Z of a boundary
EVENT_Q_ZERO = 16     # draft token outside supp(q~): rejected
EVENT_RES_ZERO = 32   # residual mass zero after a rejection: drew from p~
TIE_MASK = TIE_ACCEPT | TIE_TOPP_P | TIE_TOPP_Q | TIE_ICDF


def decode_logits(x, dtype):
    """Logits as fp64. dtype 'bf16' takes uint16 bit patterns, 'f32' float32 values."""
    x = np.asarray(x)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 logits are passed as uint16 bit patterns")
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def seq_sum(w):
    """Sequential left-to-right fp64 sum (numpy's accumulate is a plain loop)."""
    if len(w) == 0:
        return 0.0
    return float(np.cumsum(np.asarray(w, dtype=np.float64))[-1])


class Filtered:
    """A filtered distribution: support ids (ascending) and fp64 probabilities."""

    def __init__(self, ids, probs, topp_gap=math.inf):
        self.ids = np.asarray(ids, dtype=np.int64)
        self.probs = np.asarray(probs, dtype=np.float64)
        self.topp_gap = topp_gap

    def prob_of(self, tok):
        j = np.searchsorted(self.ids, tok)
        if j < len(self.ids) and self.ids[j] == tok:
            return float(self.probs[j])
        return 0.0

    def probs_at(self, toks):
        toks = np.asarray(toks, dtype=np.int64)
        j = np.searchsorted(self.ids, toks)
        j = np.minimum(j, len(self.ids) - 1)
        hit = self.ids[j] == toks
        return np.where(hit, self.probs[j], 0.0)


def filter_logits(z, temperature, top_k, top_p):
    """Temperature / top-k / top-p filtering of one logit row (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.size
    if V == 0:
        raise ValueError("empty vocabulary")
    if temperature <= 0:
        # Greedy: np.argmax returns the first maximum, i.e. the lowest id on ties.
        return Filtered([int(np.argmax(z))], [1.0])
    if 0 < top_k < V:
        kth = np.partition(z, V - top_k)[V - top_k]   # k-th largest, with multiplicity
        ids = np.flatnonzero(z >= kth)
    else:
        ids = np.arange(V)
    zk = z[ids]
    m = zk.max()
    w = np.exp((zk - m) / temperature)
    gap = math.inf
    if top_p < 1:
        z_top = seq_sum(w)
        # Groups of equal logit in descending order; inside a group ascending id.
        order = np.lexsort((ids, -zk))
        keep = np.zeros(len(ids), dtype=bool)
        above = 0.0          # sum of w over strictly larger groups, sequential
        g0 = 0
        n = len(order)
        first = True
        while g0 < n:
            g1 = g0
            while g1 + 1 < n and zk[order[g1 + 1]] == zk[order[g0]]:
                g1 += 1
            mass_above = above / z_top
            if not first:       # the top group is kept unconditionally: not a decision
                gap = min(gap, abs(mass_above - top_p))
            if first or mass_above < top_p:
                keep[order[g0:g1 + 1]] = True
            else:
                break
            first = False
            for j in range(g0, g1 + 1):
                above += w[order[j]]
            g0 = g1 + 1
        ids = ids[keep]
        w = w[keep]
    total = seq_sum(w)
    return Filtered(ids, w / total, gap)


def inverse_cdf(ids, weights, u):
    """First token whose sequential prefix sum exceeds u*Z; returns (token, near_tie)."""
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    z = float(c[-1])
    t = u * z
    j = int(np.searchsorted(c, t, side="right"))   # first j with c[j] > t
    if j >= len(ids):
        j = int(np.flatnonzero(w > 0)[-1])
    gap = math.inf
    if j < len(ids) - 1:
        gap = min(gap, abs(t - c[j]))
    if j > 0:
        gap = min(gap, abs(t - c[j - 1]))
    return int(ids[j]), gap < NEAR_TIE * z


def verify_slot(pf, qf, d, u_acc, u_res):
    """Accept / resample decision of one draft slot given filtered p~ (pf), q~ (qf).

    Returns (accepted, token, ratio, flag bits).
    """
    flags = 0
    pd = pf.prob_of(d)
    qd = qf.prob_of(d)
    if qd == 0.0:
        acc = False
        ratio = 0.0
        flags |= EVENT_Q_ZERO
    else:
        ratio = pd / qd
        acc = u_acc < ratio
        if abs(u_acc - ratio) < NEAR_TIE:
            flags |= TIE_ACCEPT
    if acc:
        return True, d, ratio, flags
    res = np.maximum(0.0, pf.probs - qf.probs_at(pf.ids))
    if seq_sum(res) == 0.0:
        flags |= EVENT_RES_ZERO
        tok, tie = inverse_cdf(pf.ids, pf.probs, u_res)
    else:
        tok, tie = inverse_cdf(pf.ids, res, u_res)
    flags |= TIE_ICDF if tie else 0
    return False, tok, ratio, flags


def verify_block(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets,
                 temperature, top_k, top_p, seed, dtype="bf16"):
    """Lossless block verification of S sequences x b slots.

    Returns a dict with out_tokens [S,b], accept_len [S], resampled [S],
    slot_accept [S,b] (raw per-slot decisions, slot 0 = 1), slot_token [S,b]
    (the token each slot would emit: AR token / kept draft / its resample) and
    diag [S,b,4] = (u_acc, ratio, u_res, flag bits).
    """
    p_logits = np.asarray(p_logits)
    S, b, V = p_logits.shape
    out = np.full((S, b), -1, dtype=np.int32)
    accept_len = np.zeros(S, dtype=np.int32)
    resampled = np.full(S, -1, dtype=np.int32)
    slot_accept = np.zeros((S, b), dtype=np.uint8)
    slot_token = np.full((S, b), -1, dtype=np.int32)
    diag = np.zeros((S, b, 4), dtype=np.float64)
    for s in range(S):
        for i in range(b):
            u_acc, u_res = slot_uniforms(seed, seq_ids[s], int(pos_offsets[s]) + i, STREAM_VERIFY)
            pf = filter_logits(decode_logits(p_logits[s, i], dtype), temperature, top_k, top_p)
            flags = TIE_TOPP_P if pf.topp_gap < NEAR_TIE else 0
            ratio = 1.0
            if i == 0:
                tok, tie = inverse_cdf(pf.ids, pf.probs, u_res)
                acc = True
                flags |= TIE_ICDF if tie else 0
            else:
                qf = filter_logits(decode_logits(q_logits[s, i], dtype), temperature, top_k, top_p)
                flags |= TIE_TOPP_Q if qf.topp_gap < NEAR_TIE else 0
                acc, tok, ratio, f = verify_slot(pf, qf, int(draft_tokens[s, i]), u_acc, u_res)
                flags |= f
            slot_accept[s, i] = 1 if acc else 0
            slot_token[s, i] = tok
            diag[s, i] = (u_acc, ratio, u_res, flags)
        n = b
        for i in range(1, b):
            if not slot_accept[s, i]:
                n = i
                break
        accept_len[s] = n
        out[s, :n] = slot_token[s, :n]
        if n < b:
            out[s, n] = slot_token[s, n]
            resampled[s] = slot_token[s, n]
    return dict(out_tokens=out, accept_len=accept_len, resampled=resampled,
                slot_accept=slot_accept, slot_token=slot_token, diag=diag)


def draft_sample(q_logits, seq_ids, pos_offsets, temperature, top_k, top_p, seed,
                 dtype="bf16"):
    """Draft tokens d[s,i] ~ q~[s,i] by inverse CDF at Philox stream 1 (word 0).

    Returns (tokens [S,b] int32, flags [S,b] int32 with TIE_TOPP_Q / TIE_ICDF).
    """
    q_logits = np.asarray(q_logits)
    S, b, V = q_logits.shape
    toks = np.zeros((S, b), dtype=np.int32)
    flags = np.zeros((S, b), dtype=np.int32)
    for s in range(S):
        for i in range(b):
            u, _ = slot_uniforms(seed, seq_ids[s], int(pos_offsets[s]) + i, STREAM_DRAFT)
            qf = filter_logits(decode_logits(q_logits[s, i], dtype), temperature, top_k, top_p)
            tok, tie = inverse_cdf(qf.ids, qf.probs, u)
            toks[s, i] = tok
            flags[s, i] = (TIE_TOPP_Q if qf.topp_gap < NEAR_TIE else 0) | (TIE_ICDF if tie else 0)
    return toks, flags


def expected_accept_len(tv_per_slot):
    """E[accept_len] = 1 + sum_{j>=1} prod_{i<=j} (1 - TV_i) for one block."""
    tv = np.asarray(tv_per_slot, dtype=np.float64)
    e, run = 1.0, 1.0
    for j in range(1, len(tv)):
        run *= 1.0 - tv[j]
        e += run
    return e
