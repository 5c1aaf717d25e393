"""The verifier's allocation-free entry point, uno_verify_block_noalloc, called
through the C ABI: its results equal those of uno_verify_block with a caller
workspace, bit for bit (the same kernels on the same inputs), on calls in a row
that change the layout of the library's scratch (a full Qwen-shaped block, then a
smaller one, then the full one again); it allocates no device memory when every
output is passed in; and sizes beyond the scratch are rejected before any launch."""
import numpy as np
import pytest
import torch

import workloads
from helpers import to_device

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


def _inputs(S, b, V, seed):
    cfg = dict(workloads.VERIFY_CONFIGS["qwen"], S=S, b=b)
    p, q = workloads.verify_logits(cfg, seed=seed, V=V)
    rng = np.random.default_rng(seed)
    seq = to_device(rng.integers(0, 2**62, S, dtype=np.int64), DEV)
    pos = to_device(rng.integers(0, 100000, S, dtype=np.int64), DEV)
    pd, qd = to_device(p, DEV), to_device(q, DEV)
    d, _ = _uno().uno_draft_sample(qd, seq, pos, **SP)
    return pd, qd, d, seq, pos


def _same(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def test_noalloc_matches_the_workspace_entry_point():
    uno = _uno()
    cases = [(64, 16, 151936, 1), (7, 5, 32000, 2), (64, 16, 151936, 1)]
    for S, b, V, seed in cases:
        print(f"noalloc verify S={S} b={b} V={V} seed={seed}", flush=True)
        args = _inputs(S, b, V, seed)
        ref = uno.uno_verify_block(*args, **SP)
        got = uno.uno_verify_block_noalloc(*args, **SP)
        again = uno.uno_verify_block_noalloc(*args, **SP)
        torch.cuda.synchronize()
        assert set(got) == set(ref)
        for k in ref:
            assert _same(got[k], ref[k]), (S, b, k)
            assert _same(again[k], ref[k]), (S, b, k)
        assert int(got["accept_len"].min()) >= 1


def test_noalloc_allocates_nothing_with_outputs_given():
    uno = _uno()
    S, b, V = 16, 8, 50000
    args = _inputs(S, b, V, 3)
    out = dict(out_tokens=torch.empty((S, b), dtype=torch.int32, device=DEV),
               accept_len=torch.empty((S,), dtype=torch.int32, device=DEV),
               resampled=torch.empty((S,), dtype=torch.int32, device=DEV),
               slot_accept=torch.empty((S, b), dtype=torch.uint8, device=DEV),
               diag=torch.empty((S, b, 4), dtype=torch.float32, device=DEV))
    uno.uno_verify_block_noalloc(*args, out=out, **SP)       # the device's scratch is set up here
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    uno.uno_verify_block_noalloc(*args, out=out, **SP)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before
    ref = uno.uno_verify_block(*args, **SP)
    torch.cuda.synchronize()
    for k in ref:
        assert _same(out[k], ref[k]), k


@pytest.mark.parametrize("S,b", [(4096, 64), (65537, 2)])
def test_noalloc_rejects_sizes_beyond_its_scratch(S, b):
    uno = _uno()
    V = 8
    z = torch.zeros((S, b, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((S, b), dtype=torch.int32, device=DEV)
    ids = torch.zeros((S,), dtype=torch.int64, device=DEV)
    with pytest.raises(uno.UnoError) as e:
        uno.uno_verify_block_noalloc(z, z, d, ids, ids, **SP)
    assert e.value.status == "UNO_ERR_UNSUPPORTED"
    assert "scratch" in str(e.value)
