"""GPU parity of the row-gated LoRA linear (bf16 MFMA) against the fp64 CPU oracle.

Tolerance (bf16 inputs, fp32 accumulation, bf16 output; T rounded to bf16 on the
GPU, unrounded in the oracle): ||Y - Y_ref||_F <= 2e-2 ||Y_ref||_F and
max |Y - Y_ref| <= 2e-2 max |Y_ref|. Because the adapter's contribution is only a
few percent of Y, the delta is checked on its own: on noise rows,
||(Y_mask - Y_nomask) - s (X A^T) B^T|| <= 2e-2 ||s (X A^T) B^T||, where Y_nomask is
the same kernel run with every mask entry 0. Seed rows (mask 0) must be bitwise
equal to that run: they add exact zeros.
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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def _run(X, W, A, B, mask, scale):
    uno = _uno()
    Y = uno.uno_gated_lora_linear(X, W, A, B, mask, scale)
    torch.cuda.synchronize()
    return Y


def _check_case(M, K, N, r, scale, mask_np, rows=None, tag=0):
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=1, tag=tag)
    Xd, Wd, Ad, Bd = (to_device(a, DEV) for a in (X, W, A, B))
    Y = _bits(_run(Xd, Wd, Ad, Bd, to_device(mask_np, DEV), scale))
    Y0 = _bits(_run(Xd, Wd, Ad, Bd, to_device(np.zeros(M, np.uint8), DEV), scale))
    rows = np.arange(M) if rows is None else np.asarray(rows)
    ref = oracle.gated_lora_linear(X[rows], W, A, B, mask_np[rows], scale)
    y = _f64(Y[rows])
    assert np.linalg.norm(y - ref) <= 2e-2 * np.linalg.norm(ref)
    assert np.max(np.abs(y - ref)) <= 2e-2 * np.max(np.abs(ref))
    seed = rows[mask_np[rows] == 0]
    np.testing.assert_array_equal(Y[seed], Y0[seed])
    ref0 = oracle.gated_lora_linear(X[rows], W, A, B, np.zeros(len(rows), np.uint8), scale)
    y0 = _f64(Y0[rows])
    assert np.linalg.norm(y0 - ref0) <= 2e-2 * np.linalg.norm(ref0)
    noise = rows[mask_np[rows] == 1]
    if r > 0 and len(noise):
        delta_ref = oracle.lora_delta(X[noise], A, B, scale)
        delta = _f64(Y[noise]) - _f64(Y0[noise])
        # Y and Y0 are each rounded to bf16: that rounding (2^-9 of |Y|) is part of
        # the measured delta, so the bound adds it.
        round_err = 2.0 ** -8 * np.linalg.norm(ref[mask_np[rows] == 1])
        assert np.linalg.norm(delta - delta_ref) <= 2e-2 * np.linalg.norm(delta_ref) + round_err
    return Y


@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_tiny_gated_lora(scale):
    c = workloads.GEMM_CONFIGS["tiny"]
    (_, K, N), = c["projections"]
    mask = workloads.noise_row_mask(c["M"] // c["b"], c["b"])
    _check_case(c["M"], K, N, c["r"], scale, mask)


@pytest.mark.parametrize("M,K,N,r", [
    (200, 264, 300, 24),      # ragged in every dimension
    (129, 64, 129, 8),        # one past a tile
    (1, 8, 1, 8),             # smallest
    (300, 1000, 72, 0),       # r = 0: plain linear
    (512, 2560, 640, 64),
])
def test_ragged_shapes(M, K, N, r):
    mask = (np.random.default_rng(M * N).random(M) < 0.8).astype(np.uint8)
    _check_case(M, K, N, r, 16.0, mask)


@pytest.mark.parametrize("name,proj", [
    ("qwen", 0), ("qwen", 1), ("looped", 0), ("looped", 4), ("looped", 6), ("stress", 1), ("stress", 6),
])
def test_workload_shapes_sampled_rows(name, proj):
    c = workloads.GEMM_CONFIGS[name]
    _, K, N = c["projections"][proj]
    M = c["M"]
    mask = workloads.noise_row_mask(M // c["b"], c["b"])
    rng = np.random.default_rng(proj)
    rows = np.unique(np.concatenate([[0, 1, c["b"] - 1, c["b"], M - 1], rng.integers(0, M, 27)]))
    _check_case(M, K, N, c["r"], 1.0, mask, rows=rows, tag=proj)


def test_repeat_runs_are_identical():
    M, K, N, r = 384, 1024, 640, 32
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=3)
    args = [to_device(a, DEV) for a in (X, W, A, B)]
    mask = to_device(workloads.noise_row_mask(M // 8, 8), DEV)
    first = _bits(_run(*args, mask, 2.0))
    for _ in range(2):
        np.testing.assert_array_equal(_bits(_run(*args, mask, 2.0)), first)


def test_argument_errors():
    uno = _uno()
    X = torch.zeros((4, 12), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((4, 12), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros((8, 12), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV)
    m = torch.zeros((4,), dtype=torch.uint8, device=DEV)
    with pytest.raises(uno.UnoError) as e:
        uno.uno_gated_lora_linear(X, W, A, B, m, 1.0)      # K = 12 is not a multiple of 8
    assert e.value.status == "UNO_ERR_UNSUPPORTED"


def test_alternating_shapes_share_the_workspace():
    """Calls of different shapes reuse one workspace, whose split-K counters carry
    over from call to call: results must not depend on what ran before."""
    shapes = [(512, 2560, 640, 64), (1024, 4096, 384, 128), (200, 1000, 72, 24)]
    runs = []
    for M, K, N, r in shapes:
        X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=5)
        args = [to_device(a, DEV) for a in (X, W, A, B)]
        mask = to_device(workloads.noise_row_mask(M // 8, 8) if M % 8 == 0 else np.ones(M, np.uint8), DEV)
        runs.append((args, mask))
    first = [_bits(_run(*args, mask, 16.0)) for args, mask in runs]
    for _ in range(2):
        for (args, mask), ref in zip(reversed(runs), reversed(first)):
            np.testing.assert_array_equal(_bits(_run(*args, mask, 16.0)), ref)
