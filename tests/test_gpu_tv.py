"""GPU parity of the fused TV self-distillation loss (forward + student gradient)
against the fp64 CPU oracle.

Tolerances: the loss and the per-row TV are fp32 results of fp32 exponentials
summed partly in fp64, so they must agree with the oracle to 1e-5 relative (with
a 2e-6 absolute floor for rows whose TV is near zero). The gradient is stored in
the logits' dtype; for bf16 its rounding alone is 2^-9 relative per element, so
the check is normwise: per row and over all compared rows,
||g - g_ref|| <= 2e-2 ||g_ref||. Rows outside the response mask must be exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import lossless_diffusion_drafted_amd as uno
    uno.load()


def _uno():
    import lossless_diffusion_drafted_amd as uno
    return uno


def _inputs(R, V, dtype, seed):
    if dtype == "bf16":
        return workloads.tv_rows(range(R), V, seed=seed)
    rng = np.random.default_rng([seed, R, V])
    t = (3.0 * rng.standard_normal((R, V))).astype(np.float32)
    s = (t + rng.standard_normal((R, V))).astype(np.float32)
    return t, s


def _run(t, s, mask, T, want_grad=True, want_rows=True):
    uno = _uno()
    loss, rows, grad = uno.uno_tv_loss_fwd_bwd(to_device(t, DEV), to_device(s, DEV), to_device(mask, DEV),
                                               temperature=T, want_grad=want_grad, want_rows=want_rows)
    torch.cuda.synchronize()
    out = {"loss": float(loss.item())}
    out["rows"] = rows.cpu().numpy().astype(np.float64) if rows is not None else None
    out["grad"] = grad.float().cpu().numpy().astype(np.float64) if grad is not None else None
    return out


def _check(gpu, ref_loss, ref_rows, ref_grad, mask, T=1.0):
    assert abs(gpu["loss"] - ref_loss) <= 1e-5 * abs(ref_loss) + 2e-6, (gpu["loss"], ref_loss)
    if gpu["rows"] is not None:
        np.testing.assert_allclose(gpu["rows"], ref_rows, rtol=1e-5, atol=2e-6)
        assert np.all(gpu["rows"][mask == 0] == 0.0)
    if gpu["grad"] is not None and ref_grad is not None:
        g, gr = gpu["grad"], ref_grad
        assert np.all(g[mask == 0] == 0.0)
        for r in np.flatnonzero(mask):
            nr = np.linalg.norm(gr[r])
            if nr > 0:
                assert np.linalg.norm(g[r] - gr[r]) <= 2e-2 * nr, r
            else:
                assert np.all(g[r] == 0.0), r
        nt = np.linalg.norm(gr)
        assert np.linalg.norm(g - gr) <= 2e-2 * nt + 1e-30
        # the loss is invariant to shifting a row's logits, so each gradient row sums
        # to 0 up to rounding: the terms q_j (s_j/2 - G) / (T N) cancel with an error of
        # about eps32 / (T N), and the bf16 rounding adds 2^-9 of sum |g| at most
        n = max(int(mask.sum()), 1)
        sums = np.abs(g.sum(axis=1))
        assert np.all(sums <= 2 ** -8 * np.abs(g).sum(axis=1) + 1e-6 / (T * n))


# A row is split over a team of workgroups. bf16 rows with 16-byte alignment take
# the pipelined kernel: ceil(V / 30720) members (960 data threads x 32 logits).
# fp32 rows and unaligned rows take the register kernel: ceil(V / 40960) members
# (1024 threads x 40 logits).
@pytest.mark.parametrize("R,V,dtype,T,mask_kind", [
    (5, 1000, "bf16", 1.0, "all"),        # one workgroup per row, ragged slice
    (16, 1000, "bf16", 1.0, "random"),
    (40, 50000, "bf16", 0.7, "random"),   # two-member teams, ragged last slice
    (13, 50000, "f32", 1.0, "random"),    # fp32 logits
    (9, 30001, "f32", 1.3, "all"),        # rows not 16-byte aligned
    (7, 4097, "bf16", 1.0, "random"),     # rows not 16-byte aligned
    (6, 151936, "bf16", 1.0, "all"),      # the full vocabulary: five-member teams
    (3, 153600, "bf16", 1.0, "all"),      # exactly fills five slices
    (4, 262144, "bf16", 1.0, "all"),      # nine-member teams
    (3, 1000000, "f32", 0.9, "random"),   # 25-member teams, fp32
    (2, 64 * 30720 - 8, "bf16", 1.0, "all"),    # the largest team (64 members), ragged
    (2, 64 * 30720 - 5, "bf16", 1.0, "all"),    # unaligned rows: 48-member teams
    (2, 64 * 40960 - 4, "f32", 1.0, "all"),     # the largest fp32 team (64 members)
])
def test_tv_matches_oracle(R, V, dtype, T, mask_kind):
    t, s = _inputs(R, V, dtype, seed=R * 7 + V)
    if mask_kind == "all":
        mask = np.ones(R, np.uint8)
    else:
        mask = (np.random.default_rng(R + V).random(R) < 0.7).astype(np.uint8)
        mask[0] = 1
    ref_loss, ref_rows, ref_grad = oracle.tv_loss_fwd_bwd(t, s, mask, T, dtype=dtype)
    gpu = _run(t, s, mask, T)
    _check(gpu, ref_loss, ref_rows, ref_grad, mask, T)


def test_tv_forward_only_and_optional_rows():
    t, s = _inputs(12, 20000, "bf16", seed=3)
    mask = np.ones(12, np.uint8)
    ref_loss, ref_rows, _ = oracle.tv_loss_fwd_bwd(t, s, mask, 1.0, dtype="bf16", want_grad=False)
    gpu = _run(t, s, mask, 1.0, want_grad=False, want_rows=True)
    _check(gpu, ref_loss, ref_rows, None, mask)
    gpu = _run(t, s, mask, 1.0, want_grad=True, want_rows=False)
    assert abs(gpu["loss"] - ref_loss) <= 1e-5 * ref_loss + 2e-6


def test_tv_vocabulary_beyond_the_largest_team_is_rejected():
    uno = _uno()
    V = 64 * 30720 + 8
    z = torch.zeros((1, V), dtype=torch.bfloat16, device=DEV)
    m = torch.ones((1,), dtype=torch.uint8, device=DEV)
    with pytest.raises(uno.UnoError) as e:
        uno.uno_tv_loss_fwd_bwd(z, z, m)
    assert e.value.status == "UNO_ERR_UNSUPPORTED"


def test_tv_no_response_rows():
    t, s = _inputs(6, 3000, "bf16", seed=5)
    mask = np.zeros(6, np.uint8)
    gpu = _run(t, s, mask, 1.0)
    assert gpu["loss"] == 0.0
    assert np.all(gpu["rows"] == 0.0) and np.all(gpu["grad"] == 0.0)


def test_tv_empty_batch():
    uno = _uno()
    z = torch.empty((0, 100), dtype=torch.bfloat16, device=DEV)
    m = torch.empty((0,), dtype=torch.uint8, device=DEV)
    loss, rows, grad = uno.uno_tv_loss_fwd_bwd(z, z, m)
    torch.cuda.synchronize()
    assert loss.item() == 0.0


def test_tv_identical_and_disjoint_rows():
    """p = q gives TV 0 and an exactly zero gradient; almost disjoint one-hot rows give TV ~ 1."""
    V = 70000
    t, _ = _inputs(4, V, "bf16", seed=9)
    s = t.copy()
    big = workloads.to_bf16_bits(np.array([60.0], np.float32))[0]
    s[2] = workloads.to_bf16_bits(np.zeros(V, np.float32))
    t2 = s[2].copy()
    t2[11] = big
    s[2, 12] = big
    t[2] = t2
    mask = np.ones(4, np.uint8)
    ref_loss, ref_rows, ref_grad = oracle.tv_loss_fwd_bwd(t, s, mask, 1.0, dtype="bf16")
    gpu = _run(t, s, mask, 1.0)
    for r in (0, 1, 3):
        assert gpu["rows"][r] == 0.0
        assert np.all(gpu["grad"][r] == 0.0)
    assert abs(gpu["rows"][2] - 1.0) < 1e-6 and abs(ref_rows[2] - 1.0) < 1e-6
    _check(gpu, ref_loss, ref_rows, ref_grad, mask)


def test_tv_repeat_runs_are_identical():
    t, s = _inputs(24, 40000, "bf16", seed=11)
    mask = np.ones(24, np.uint8)
    uno = _uno()
    td, sd, md = to_device(t, DEV), to_device(s, DEV), to_device(mask, DEV)
    first = None
    for _ in range(3):
        loss, rows, grad = uno.uno_tv_loss_fwd_bwd(td, sd, md)
        cur = (loss.clone(), rows.clone(), grad.clone())
        if first is None:
            first = cur
        else:
            for a, b in zip(cur, first):
                assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                                   b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


def _host_bits(x):
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def test_tv_full_size():
    """The self-distillation workload at full size (8 x 4096 rows, V = 151936, bf16):
    every response row's TV and the loss against the oracle (computed in row chunks
    on a thread pool), the gradient on 512 response rows spread over all eight
    sequences, and every row outside the response mask exactly zero."""
    import concurrent.futures
    import os
    cfg = workloads.TV_CONFIG
    V = cfg["V"]
    R = cfg["n_seq"] * cfg["seq_len"]
    uno = _uno()
    print("full-size TV: generating inputs", flush=True)
    t, s = workloads.tv_inputs_torch(R, V, DEV, seed=0)
    mask_np = workloads.tv_response_mask(cfg["n_seq"], cfg["seq_len"], cfg["resp_len"])
    mask = to_device(mask_np, DEV)
    loss, rows, grad = uno.uno_tv_loss_fwd_bwd(t, s, mask, temperature=1.0)
    torch.cuda.synchronize()
    print("full-size TV: kernel done, oracle over every response row", flush=True)
    rows_np = rows.cpu().numpy().astype(np.float64)
    resp = np.flatnonzero(mask_np)
    n = len(resp)
    assert np.all(rows_np[mask_np == 0] == 0.0)
    unmasked = torch.from_numpy(mask_np == 0).to(DEV)
    assert int(torch.count_nonzero(grad[unmasked])) == 0

    # gradient rows: 64 response rows of each sequence, seeded
    rng = np.random.default_rng(0)
    per_seq = [np.sort(rng.choice(resp[(resp // cfg["seq_len"]) == k], 64, replace=False))
               for k in range(cfg["n_seq"])]
    grad_rows = set(np.concatenate(per_seq).tolist())

    def oracle_chunk(idx, tt, ss):
        want = [i for i, r in enumerate(idx) if r in grad_rows]
        _, ref_rows, _ = oracle.tv_loss_fwd_bwd(tt, ss, np.ones(len(idx), np.uint8), 1.0, dtype="bf16",
                                                want_grad=False)
        ref_g = None
        if want:
            _, _, ref_g = oracle.tv_loss_fwd_bwd(tt[want], ss[want], np.ones(len(want), np.uint8), 1.0,
                                                 dtype="bf16")
            ref_g *= len(want) / n        # the oracle normalised by its own row count
        return idx, ref_rows, [idx[i] for i in want], ref_g

    ref_rows = np.zeros(R)
    checked_grad = 0
    chunk = 128
    nthreads = min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
        pending = []
        for c0 in range(0, n, chunk):
            idx = resp[c0:c0 + chunk]
            # response rows are contiguous within a sequence: slice when they are
            sl = slice(int(idx[0]), int(idx[-1]) + 1) if idx[-1] - idx[0] == len(idx) - 1 else \
                torch.from_numpy(idx).to(DEV)
            pending.append(ex.submit(oracle_chunk, idx, _host_bits(t[sl]), _host_bits(s[sl])))
            while len(pending) > 2 * nthreads or (c0 + chunk >= n and pending):
                idx_done, rr, grows, rg = pending.pop(0).result()
                ref_rows[idx_done] = rr
                if grows:
                    g = grad[torch.tensor(grows, device=DEV)].float().cpu().numpy().astype(np.float64)
                    for a in range(len(grows)):
                        nr = np.linalg.norm(rg[a])
                        assert np.linalg.norm(g[a] - rg[a]) <= 2e-2 * nr, grows[a]
                    checked_grad += len(grows)
    assert checked_grad == 512
    np.testing.assert_allclose(rows_np[resp], ref_rows[resp], rtol=1e-5, atol=2e-6)
    ref_loss = ref_rows[resp].sum() / n
    print("full-size TV loss", loss.item(), "oracle", ref_loss)
    assert abs(loss.item() - ref_loss) <= 1e-5 * ref_loss
    del t, s, grad
    torch.cuda.empty_cache()


def test_tv_equals_one_minus_measured_acceptance():
    """Rows of the self-distillation workload: the per-row TV from the TV kernel
    equals 1 - the acceptance rate the verifier measures with the filters off at
    T = 1 (teacher as the base p, student as the draft q, drafts d ~ q from the
    draft sampler), within 4 standard deviations of the binomial spread, over
    102400 independent Philox draws per row."""
    import math
    uno = _uno()
    cfg = workloads.TV_CONFIG
    V = cfg["V"]
    nrows = 3
    row_ids = [1024, 9000, 30000]                  # response rows of sequences 0, 2 and 7
    t, s = workloads.tv_rows(row_ids, V)
    ones = np.ones(nrows, np.uint8)
    td, sd = to_device(t, DEV), to_device(s, DEV)
    _, tv_dev, _ = uno.uno_tv_loss_fwd_bwd(td, sd, to_device(ones, DEV), 1.0, want_grad=False)
    torch.cuda.synchronize()
    tv = tv_dev.cpu().numpy().astype(np.float64)
    _, tv_ref, _ = oracle.tv_loss_fwd_bwd(t, s, ones, 1.0, dtype="bf16", want_grad=False)
    np.testing.assert_allclose(tv, tv_ref, rtol=1e-5, atol=2e-6)

    S, calls, b = 4096, 25, nrows + 1
    pick = torch.tensor([0] + list(range(nrows)), device=DEV)     # slot i >= 1 holds row i - 1
    p = td[pick].unsqueeze(0).expand(S, b, V).contiguous()
    q = sd[pick].unsqueeze(0).expand(S, b, V).contiguous()
    sp = dict(temperature=1.0, top_k=0, top_p=1.0, seed=77)
    pos = torch.zeros(S, dtype=torch.int64, device=DEV)
    accepted = torch.zeros(b, dtype=torch.int64, device=DEV)
    for c in range(calls):
        seq = torch.arange(S, dtype=torch.int64, device=DEV) + c * S
        d, _ = uno.uno_draft_sample(q, seq, pos, **sp)
        r = uno.uno_verify_block(p, q, d, seq, pos, want_diag=False, **sp)
        accepted += r["slot_accept"].to(torch.int64).sum(0)
    torch.cuda.synchronize()
    n = S * calls
    acc = accepted.cpu().numpy() / n
    for i in range(1, b):
        a_exp = 1.0 - tv[i - 1]
        sd_i = math.sqrt(a_exp * (1.0 - a_exp) / n)
        print("row", row_ids[i - 1], "TV", tv[i - 1], "measured acceptance", acc[i], "1 - TV", a_exp,
              "z", (acc[i] - a_exp) / sd_i)
        assert abs(acc[i] - a_exp) < 4 * sd_i, (i, acc[i], a_exp)
    del p, q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_tv_mask_at_any_byte_offset(offset):
    """The response mask is read a 4-byte word at a time through the scalar cache;
    a mask that starts at any byte offset gives the same rows and gradient."""
    uno = _uno()
    R, V = 37, 5000
    t, s = _inputs(R, V, "bf16", seed=11 + offset)
    mask = (np.random.default_rng(offset).random(R) < 0.6).astype(np.uint8)
    mask[0], mask[-1] = 1, 0
    backing = np.zeros(R + 8, np.uint8)
    backing[offset:offset + R] = mask
    mdev = to_device(backing, DEV)[offset:offset + R]
    assert mdev.data_ptr() % 4 == offset          # device allocations are at least 4-byte aligned
    loss, rows, grad = uno.uno_tv_loss_fwd_bwd(to_device(t, DEV), to_device(s, DEV), mdev,
                                               temperature=1.0, want_grad=True, want_rows=True)
    torch.cuda.synchronize()
    gpu = {"loss": float(loss.item()), "rows": rows.cpu().numpy().astype(np.float64),
           "grad": grad.float().cpu().numpy().astype(np.float64)}
    ref_loss, ref_rows, ref_grad = oracle.tv_loss_fwd_bwd(t, s, mask, 1.0, dtype="bf16")
    _check(gpu, ref_loss, ref_rows, ref_grad, mask)
