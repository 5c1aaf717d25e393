"""GPU parity of the HIP verifier and draft sampler against the CPU oracle.

Token ids, accept lengths and resampled tokens must be bit-exact given the same
Philox stream; a difference is tolerated only from the first decisive slot (slot
0, an accepted slot or the first rejected one) where either side flags a near-tie
(|u - p~/q~| < 1e-6, a top-p boundary within 1e-6 of top_p, or an inverse-CDF draw
within 1e-6*Z of a boundary); the tokens before it must still agree, and every
other slot's raw accept decision must agree. Excused sequences are counted and
printed, and each test bounds their number. Draft tokens given to both sides come
from the oracle's draft sampler; the full-size workloads compare every sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_mostly_exact, compare_verify, dtype_name, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SP = workloads.SAMPLING


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import lossless_diffusion_drafted_amd as uno
    uno.load()


def _uno():
    import lossless_diffusion_drafted_amd as uno
    return uno


def _gpu_verify(p, q, d, seq, pos, sp):
    uno = _uno()
    r = uno.uno_verify_block(to_device(p, DEV), to_device(q, DEV), to_device(d.astype(np.int32), DEV),
                             to_device(seq, DEV), to_device(pos, DEV),
                             temperature=sp["temperature"], top_k=sp["top_k"], top_p=sp["top_p"],
                             seed=sp["seed"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def _run_full(p, q, sp, seq=None, pos=None):
    S, b, V = p.shape
    seq = np.arange(S, dtype=np.int64) if seq is None else seq
    pos = np.zeros(S, dtype=np.int64) if pos is None else pos
    dt = dtype_name(p)
    d, _ = oracle.draft_sample(q, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], dt)
    ref = oracle.verify_block(p, q, d, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], dt)
    gpu = _gpu_verify(p, q, d, seq, pos, sp)
    return compare_verify(gpu, ref, b), gpu, ref


def test_draft_sampler_matches_oracle_tiny():
    uno = _uno()
    p, q = workloads.verify_logits("tiny")
    S, b, V = q.shape
    seq, pos = np.arange(S, dtype=np.int64), np.zeros(S, dtype=np.int64)
    ref, rflags = oracle.draft_sample(q, seq, pos, SP["temperature"], SP["top_k"], SP["top_p"], SP["seed"], "f32")
    d, flags = uno.uno_draft_sample(to_device(q, DEV), to_device(seq, DEV), to_device(pos, DEV), **SP)
    torch.cuda.synchronize()
    d, flags = d.cpu().numpy(), flags.cpu().numpy()
    tie = (flags | rflags) & oracle.TIE_MASK
    np.testing.assert_array_equal(d[tie == 0], ref[tie == 0])


def test_verify_tiny():
    p, q = workloads.verify_logits("tiny")
    st, gpu, ref = _run_full(p, q, SP)
    print("tiny", st, "accept_len", gpu["accept_len"])
    assert st["exact"] == 1


@pytest.mark.parametrize("V,S,b,seed", [(4096, 8, 16, 1), (32000, 4, 8, 2), (151936, 2, 16, 3)])
def test_verify_qwen_distribution_reduced(V, S, b, seed):
    cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=S, b=b)
    p, q = workloads.verify_logits(cfg, seed=seed, V=V)
    rng = np.random.default_rng(seed)
    seq = rng.integers(0, 2**62, S, dtype=np.int64)
    pos = rng.integers(0, 100000, S, dtype=np.int64)
    st, gpu, ref = _run_full(p, q, SP, seq, pos)
    print(V, S, b, st)
    assert_mostly_exact(st, S)


@pytest.mark.parametrize("V,b,k,top_p,T", [
    (1, 4, 50, 0.95, 1.0), (7, 3, 50, 0.95, 1.0), (50, 8, 50, 0.95, 1.0), (51, 8, 50, 0.9, 1.0),
    (1000, 1, 50, 0.95, 1.0), (4099, 5, 50, 0.95, 1.0), (2051, 64, 50, 0.5, 0.7),
    (300, 6, 0, 1.0, 1.0), (2048, 4, 0, 0.95, 1.3),              # top-k off: full-row path
    (3000, 4, 1, 0.95, 1.0), (3000, 4, 50, 1e-9, 1.0),
    (3000, 6, 256, 0.99, 2.0), (3000, 6, 200, 0.99, 2.0), (3000, 6, 128, 0.9, 1.0),
    (5000, 6, 50, 0.95, 0.0),
    (40000, 3, 50, 0.95, 1.0), (70001, 2, 7, 0.9, 0.8),
])
def test_verify_ragged_and_settings(V, b, k, top_p, T):
    S = 3
    cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=S, b=b)
    p, q = workloads.verify_logits(cfg, seed=V + b, V=V)
    sp = dict(temperature=T, top_k=k, top_p=top_p, seed=11)
    st, gpu, ref = _run_full(p, q, sp)
    print(V, b, k, top_p, T, st)
    assert_mostly_exact(st, S)


def test_verify_fp32_unaligned_rows():
    cfg = dict(workloads.VERIFY_CONFIGS["tiny"], S=3, b=5)
    p, q = workloads.verify_logits(cfg, seed=4, V=1027)   # 1027*4 bytes: rows not 16-byte aligned
    st, _, _ = _run_full(p, q, SP)
    assert st["exact"] == 3


def test_verify_many_ties():
    rng = np.random.default_rng(5)
    S, b, V = 4, 8, 3000
    base = np.round(rng.normal(0, 3, (S, b, V)) * 2) / 2          # half-integer grid: heavy ties
    p = workloads.to_bf16_bits(base.astype(np.float32))
    q = workloads.to_bf16_bits((base + np.round(rng.normal(0, 1, (S, b, V)) * 2) / 2).astype(np.float32))
    st, _, _ = _run_full(p, q, dict(SP, top_k=20))
    print(st)
    assert_mostly_exact(st, S)


def _one_wave_rows(n_planted, S=2, b=4, V=151936, seed=11):
    """Rows whose largest values all sit in 16-byte chunks that the first wave of a
    workgroup reads (chunk c = 8 elements, read by thread c % 256): that wave flags
    far more chunks than the others."""
    rng = np.random.default_rng(seed)
    base = rng.normal(0.0, 1.0, (S, b, V))
    j = np.arange(n_planted)
    groups = -(-n_planted // 64)
    step = (V // 8 // 256 - 1) // groups             # spread the groups of 64 along the row
    chunks = 256 * (step * (j // 64)) + (j % 64)     # distinct chunks of lanes 0..63
    cols = chunks * 8 + (j % 8)
    assert cols.max() < V
    base[:, :, cols] = 8.0 + rng.random((S, b, n_planted))
    p = workloads.to_bf16_bits(base.astype(np.float32))
    q = workloads.to_bf16_bits((base + rng.normal(0.0, 0.5, (S, b, V))).astype(np.float32))
    return p, q


@pytest.mark.parametrize("n_planted", [140, 400])
def test_verify_one_wave_holds_the_top_values(n_planted):
    """140: the first wave's own chunk list fills and the shared spill area takes the
    rest; 400: the lists overflow and the slot takes the full-row path. Both match
    the oracle."""
    p, q = _one_wave_rows(n_planted)
    st, _, _ = _run_full(p, q, SP)
    print(n_planted, st)
    assert_mostly_exact(st, p.shape[0])


def test_verify_identical_rows_accept_everything():
    p, _ = workloads.verify_logits(dict(workloads.VERIFY_CONFIGS["qwen"], S=4, b=16), V=8192)
    st, gpu, _ = _run_full(p, p.copy(), SP)
    assert np.all(gpu["accept_len"] == 16)


def test_empty_batch_is_a_no_op():
    uno = _uno()
    z = torch.empty((0, 4, 100), dtype=torch.bfloat16, device=DEV)
    r = uno.uno_verify_block(z, z, torch.empty((0, 4), dtype=torch.int32, device=DEV),
                             torch.empty(0, dtype=torch.int64, device=DEV),
                             torch.empty(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert r["accept_len"].numel() == 0


GREEDY = dict(SP, temperature=0.0)
_FULL = {}


def _full_workload(name):
    """The whole verify workload (generated once per module) and the oracle's drafts."""
    if name not in _FULL:
        _FULL.clear()                   # keep one workload's host arrays at a time
        _FULL[name] = workloads.verify_logits(name)
    return _FULL[name]


@pytest.mark.parametrize("name,sp,b", [
    ("qwen", SP, None), ("looped", SP, None), ("stress", SP, None),
    ("qwen", GREEDY, None), ("looped", GREEDY, None), ("stress", GREEDY, None),
    ("qwen", SP, 8),                    # block 8 at the metric's shape
    ("qwen", GREEDY, 8),
])
def test_verify_full_size(name, sp, b):
    """The full workload in the benchmark's launch configuration, every sequence
    compared with the oracle: the HIP draft sampler against the oracle's drafts, then
    the verifier on the oracle's drafts."""
    uno = _uno()
    c = workloads.VERIFY_CONFIGS[name]
    S = c["S"]
    p, q = _full_workload(name)
    if b is not None:                   # the first b slots of each block
        p, q = np.ascontiguousarray(p[:, :b]), np.ascontiguousarray(q[:, :b])
    b = p.shape[1]
    seq, pos = np.arange(S, dtype=np.int64), np.zeros(S, dtype=np.int64)
    print(f"full-size verify {name} b={b} T={sp['temperature']}", flush=True)
    pd, qd = to_device(p, DEV), to_device(q, DEV)
    seqd, posd = to_device(seq, DEV), to_device(pos, DEV)
    dg, dflags = uno.uno_draft_sample(qd, seqd, posd, **sp)
    torch.cuda.synchronize()
    d_gpu, dflags = dg.cpu().numpy(), dflags.cpu().numpy()
    dref, rflags = oracle.draft_sample(q, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"],
                                       "bf16")
    dtie = (dflags | rflags) & oracle.TIE_MASK
    np.testing.assert_array_equal(d_gpu[dtie == 0], dref[dtie == 0])
    ref = oracle.verify_block(p, q, dref, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"],
                              "bf16")
    r = uno.uno_verify_block(pd, qd, to_device(dref.astype(np.int32), DEV), seqd, posd, **sp)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in r.items()}
    st = compare_verify(gpu, ref, b)
    flags = gpu["diag"][..., 3].astype(np.int64)
    print(name, b, st, "draft near-tie slots", int(np.count_nonzero(dtie)), "mean accept_len",
          gpu["accept_len"].mean(), "near-tie slots", int(np.sum(flags & oracle.TIE_MASK != 0)))
    assert np.count_nonzero(dtie) <= 2
    assert_mostly_exact(st, S, max_excused=2)
    assert not np.any(flags & 64)
    assert np.all((gpu["accept_len"] >= 1) & (gpu["accept_len"] <= b))
    del pd, qd


def test_repeat_runs_are_identical():
    uno = _uno()
    p, q = workloads.verify_logits(dict(workloads.VERIFY_CONFIGS["qwen"], S=16, b=16), V=151936)
    S = 16
    seq, pos = to_device(np.arange(S, dtype=np.int64), DEV), to_device(np.zeros(S, dtype=np.int64), DEV)
    pd, qd = to_device(p, DEV), to_device(q, DEV)
    d, _ = uno.uno_draft_sample(qd, seq, pos, **SP)
    first = None
    for _ in range(20):
        r = uno.uno_verify_block(pd, qd, d, seq, pos, **SP)
        cur = torch.cat([r["out_tokens"].flatten(), r["accept_len"], r["resampled"]]).cpu()
        if first is None:
            first = cur
        assert torch.equal(cur, first)


@pytest.mark.parametrize("V,b,k,top_p,T,dtype", [
    (40000, 4, 0, 0.95, 1.0, "bf16"),      # top-k off over a large vocabulary
    (40000, 4, 0, 1.0, 1.0, "bf16"),       # no filter at all
    (20000, 3, 1000, 0.9, 0.8, "bf16"),    # large top-k
    (20000, 3, 300, 1.0, 1.2, "f32"),      # large top-k, fp32 keys (four radix levels)
    (20001, 3, 0, 0.5, 1.0, "f32"),        # rows not 16-byte aligned
])
def test_verify_full_row_path(V, b, k, top_p, T, dtype):
    """Settings whose filtered support is large take the multi-pass full-row path;
    its tokens must agree with the oracle exactly outside near-ties."""
    S = 3
    cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=S, b=b, dtype=dtype)
    p, q = workloads.verify_logits(cfg, seed=V + k, V=V)
    sp = dict(temperature=T, top_k=k, top_p=top_p, seed=5)
    st, gpu, ref = _run_full(p, q, sp)
    print(V, b, k, top_p, T, dtype, st)
    assert_mostly_exact(st, S)


@pytest.mark.parametrize("V,k,top_p", [(40000, 0, 0.95), (20000, 500, 1.0)])
def test_draft_sampler_full_row_path(V, k, top_p):
    uno = _uno()
    cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=4, b=4)
    _, q = workloads.verify_logits(cfg, seed=V, V=V)
    S = q.shape[0]
    seq, pos = np.arange(S, dtype=np.int64), np.zeros(S, dtype=np.int64)
    sp = dict(temperature=1.0, top_k=k, top_p=top_p, seed=3)
    ref, rflags = oracle.draft_sample(q, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], "bf16")
    d, flags = uno.uno_draft_sample(to_device(q, DEV), to_device(seq, DEV), to_device(pos, DEV), **sp)
    torch.cuda.synchronize()
    d, flags = d.cpu().numpy(), flags.cpu().numpy()
    tie = (flags | rflags) & oracle.TIE_MASK
    np.testing.assert_array_equal(d[tie == 0], ref[tie == 0])
    assert np.count_nonzero(tie) <= 1


def test_massive_ties_take_the_full_row_path():
    """A row of identical logits keeps the whole vocabulary in its tie-inclusive
    top-k set, far beyond the single pass's capacity: the slot falls back to the
    full-row path and matches the oracle (uniform distribution, every draft kept)."""
    S, b, V = 2, 3, 5000
    z = np.zeros((S, b, V), np.float32)
    z[1, :, 17] = 1.0                                     # one sequence with a unique maximum
    st, gpu, ref = _run_full(z, z.copy(), SP)
    assert not np.any(gpu["diag"][..., 3].astype(np.int64) & 64)
    print(st)
    assert_mostly_exact(st, S)


def test_greedy_ties_take_the_lowest_id():
    """T = 0 with a maximum shared by more tokens than the single pass holds: the
    lowest id wins (through the full-row fallback)."""
    S, b, V = 1, 4, 3000
    z = np.zeros((S, b, V), np.float32)
    z[..., 500:] = 2.0                                    # 2500 tokens tie at the maximum
    st, gpu, ref = _run_full(z, z.copy(), dict(SP, temperature=0.0))
    assert st["exact"] == S
    assert gpu["out_tokens"][0, 0] == 500


def test_workspace_reuse_across_shapes():
    """Calls of different shapes share one workspace. A call with more sequences
    lays its per-sequence counters over what an earlier call used for slot
    records, so every call must leave the workspace clear."""
    sp = dict(SP)
    for S, b in [(8, 16), (96, 1), (8, 16), (40, 3)]:
        cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=S, b=b)
        p, q = workloads.verify_logits(cfg, seed=S * 100 + b, V=4096)
        st, gpu, ref = _run_full(p, q, sp)
        print(S, b, st)
        assert_mostly_exact(st, S)


def _chi2_ok(obs, expect_prob, n):
    """Chi-square goodness of fit with bins of expected count < 5 pooled; tokens
    outside the support must never appear."""
    from scipy import stats
    sup = expect_prob > 0
    assert obs[~sup].sum() == 0
    e = expect_prob[sup] * n
    o = obs[sup].astype(np.float64)
    small = e < 5
    if small.any():
        e = np.append(e[~small], e[small].sum())
        o = np.append(o[~small], o[small].sum())
    return stats.chisquare(o, e * o.sum() / e.sum()).pvalue


def test_sampling_statistics_end_to_end():
    """The HIP draft sampler and verifier over 10^5 blocks (the same filtered rows
    in every block, independent Philox streams): drafts follow q~, every slot's
    committed token follows p~ (lossless), the per-slot acceptance rate is
    1 - TV(p~, q~) and the mean accept length 1 + sum_j prod_{i<=j} (1 - TV_i),
    each within 4 standard deviations."""
    import math
    uno = _uno()
    rng = np.random.default_rng(31)
    S, b, V = 100000, 4, 64
    T, k, top_p = 1.0, 20, 0.9
    zp = workloads.to_bf16_bits(rng.normal(0, 1.5, (b, V)).astype(np.float32))
    zq = workloads.to_bf16_bits(workloads.bf16_bits_to_f32(zp) + rng.normal(0, 0.8, (b, V)).astype(np.float32))
    pf = [oracle.filter_logits(workloads.bf16_bits_to_f32(zp[i]), T, k, top_p) for i in range(b)]
    qf = [oracle.filter_logits(workloads.bf16_bits_to_f32(zq[i]), T, k, top_p) for i in range(b)]

    def dense(f):
        d = np.zeros(V)
        d[f.ids] = f.probs
        return d

    pd, qd = [dense(f) for f in pf], [dense(f) for f in qf]
    tvs = [0.0] + [0.5 * np.abs(pd[i] - qd[i]).sum() for i in range(1, b)]
    p = to_device(np.broadcast_to(zp, (S, b, V)).copy(), DEV)
    q = to_device(np.broadcast_to(zq, (S, b, V)).copy(), DEV)
    seq = to_device(np.arange(S, dtype=np.int64) + 7, DEV)
    pos = to_device(np.full(S, 11, dtype=np.int64), DEV)
    sp = dict(temperature=T, top_k=k, top_p=top_p, seed=2024)
    d, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    r = uno.uno_verify_block(p, q, d, seq, pos, **sp)
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    r = {key: v.cpu().numpy() for key, v in r.items()}
    for i in range(1, b):
        assert _chi2_ok(np.bincount(d[:, i], minlength=V), qd[i], S) > 1e-4, ("draft", i)
    L = r["accept_len"]
    assert np.all((L >= 1) & (L <= b))
    assert np.all(r["slot_accept"][:, 0] == 1)
    for i in range(b):
        reached = L >= i if i > 0 else np.ones(S, bool)
        tok = r["out_tokens"][reached, i]
        assert np.all(tok >= 0)
        assert _chi2_ok(np.bincount(tok, minlength=V), pd[i], reached.sum()) > 1e-4, ("committed", i)
    for i in range(1, b):
        a = r["slot_accept"][:, i].mean()
        sd = math.sqrt((1 - tvs[i]) * tvs[i] / S)
        assert abs(a - (1 - tvs[i])) < 4 * sd + 1e-12, (i, a, 1 - tvs[i])
    e = oracle.expected_accept_len(tvs)
    Lf = L.astype(np.float64)
    assert abs(Lf.mean() - e) < 4 * Lf.std() / math.sqrt(S), (Lf.mean(), e)
