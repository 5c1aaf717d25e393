"""GPU parity of the row-gated LoRA backward (dX, dA, dB) against the fp64 CPU oracle.

Tolerance (bf16 inputs, fp32 accumulation, bf16 outputs, with X A^T and
s diag(m) dY B rounded to bf16 on the GPU and unrounded in the oracle): for each
output, ||g - g_ref||_F <= 2e-2 ||g_ref||_F and max |g - g_ref| <= 2e-2 max |g_ref|.
With no noise row the adapter gradients are exactly zero.
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


def _f64(t):
    return oracle.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _close(g, ref, what):
    nr = np.linalg.norm(ref)
    assert np.linalg.norm(g - ref) <= 2e-2 * nr + 1e-30, (what, np.linalg.norm(g - ref) / max(nr, 1e-30))
    assert np.max(np.abs(g - ref)) <= 2e-2 * np.max(np.abs(ref)) + 1e-30, what


def _run(M, K, N, r, scale, mask, dx_rows=None, seed=1, tag=0, want_dx=True):
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=seed, tag=tag)
    G = workloads.gemm_grad(M, N, seed=seed, tag=tag)
    dX, dA, dB = _uno().uno_gated_lora_linear_bwd(*(to_device(a, DEV) for a in (G, X, W, A, B)),
                                                  to_device(mask, DEV), scale, want_dx=want_dx)
    torch.cuda.synchronize()
    rows = np.arange(M) if dx_rows is None else np.asarray(dx_rows)
    dx_ref, da_ref, db_ref = oracle.gated_lora_linear_bwd(X, W, A, B, mask, scale, G) if dx_rows is None else \
        (None,) + oracle.gated_lora_linear_bwd(X, W, A, B, mask, scale, G)[1:]
    if dx_rows is not None and want_dx:
        # dX rows from the oracle on the sampled rows only (the rest of the formula is row-wise)
        dx_ref = oracle.gated_lora_linear_bwd(X[rows], W, A, B, mask[rows], scale, G[rows])[0]
    _close(_f64(dA), da_ref, "dA")
    _close(_f64(dB), db_ref, "dB")
    if want_dx:
        _close(_f64(dX)[rows], dx_ref, "dX")
    else:
        assert dX is None
    return dX, dA, dB


@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_tiny_backward(scale):
    c = workloads.GEMM_CONFIGS["tiny"]
    (_, K, N), = c["projections"]
    _run(c["M"], K, N, c["r"], scale, workloads.noise_row_mask(c["M"] // c["b"], c["b"]))


@pytest.mark.parametrize("M,K,N,r", [
    (200, 264, 296, 24),       # ragged tiles in every dimension
    (8, 8, 8, 8),              # smallest
    (512, 1024, 640, 64),
    (136, 2560, 10240, 64),    # looped-model MLP shape, few rows
    (200, 1000, 3000, 24),     # U's reduction in 3 slices, the last one short
    (96, 3072, 1024, 40),      # T's reduction in 3 slices, a partial column tile
    (504, 10200, 264, 16),     # dX on 128 x 160 tiles, ragged
    (4096, 4080, 1000, 24),    # dX on 256 x 256 tiles (one round), ragged columns
])
def test_ragged_backward(M, K, N, r):
    mask = (np.random.default_rng(M + N).random(M) < 0.8).astype(np.uint8)
    _run(M, K, N, r, 16.0, mask)


def test_backward_no_noise_rows():
    M, K, N, r = 64, 256, 192, 16
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=4)
    G = workloads.gemm_grad(M, N, seed=4)
    mask = np.zeros(M, np.uint8)
    dX, dA, dB = _uno().uno_gated_lora_linear_bwd(*(to_device(a, DEV) for a in (G, X, W, A, B)),
                                                  to_device(mask, DEV), 16.0)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dA)) == 0 and int(torch.count_nonzero(dB)) == 0
    ref = oracle.bf16_bits_to_f64(G) @ oracle.bf16_bits_to_f64(W)
    _close(_f64(dX), ref, "dX")


def test_backward_without_dx():
    _run(128, 512, 256, 32, 2.0, workloads.noise_row_mask(16, 8), want_dx=False)


WORKLOAD_PROJECTIONS = [(name, i) for name in ("qwen", "looped", "stress")
                        for i in range(len(workloads.GEMM_CONFIGS[name]["projections"]))]


@pytest.mark.parametrize("name,proj", WORKLOAD_PROJECTIONS)
def test_backward_workload_shapes(name, proj):
    """Every projection of each workload at its full shape: dX (every row), dA and dB
    against the oracle."""
    c = workloads.GEMM_CONFIGS[name]
    pname, K, N = c["projections"][proj]
    M = c["M"]
    print(f"gated LoRA backward {name}/{pname}: M={M} K={K} N={N} r={c['r']}", flush=True)
    mask = workloads.noise_row_mask(M // c["b"], c["b"])
    _run(M, K, N, c["r"], 1.0, mask, tag=proj)


def test_backward_repeat_runs_are_identical():
    M, K, N, r = 256, 512, 384, 32
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=8)
    G = workloads.gemm_grad(M, N, seed=8)
    args = [to_device(a, DEV) for a in (G, X, W, A, B)]
    mask = to_device(workloads.noise_row_mask(M // 8, 8), DEV)
    first = None
    for _ in range(3):
        out = [t.clone() for t in _uno().uno_gated_lora_linear_bwd(*args, mask, 16.0)]
        torch.cuda.synchronize()
        if first is None:
            first = out
        for a, b in zip(out, first):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_argument_errors():
    uno = _uno()
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    m = torch.zeros((12,), dtype=torch.uint8, device=DEV)
    with pytest.raises(uno.UnoError) as e:
        uno.uno_gated_lora_linear_bwd(z(12, 16), z(12, 16), z(16, 16), z(8, 16), z(16, 8), m, 1.0)
    assert e.value.status == "UNO_ERR_UNSUPPORTED"      # M = 12 is not a multiple of 8


def test_backward_with_pretransposed_weight():
    """Passing W^T gives the same bits as transposing W inside the call."""
    M, K, N, r = 256, 768, 512, 32
    X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=12)
    G = workloads.gemm_grad(M, N, seed=12)
    args = [to_device(a, DEV) for a in (G, X, W, A, B)]
    mask = to_device(workloads.noise_row_mask(M // 8, 8), DEV)
    a = _uno().uno_gated_lora_linear_bwd(*args, mask, 4.0)
    b = _uno().uno_gated_lora_linear_bwd(*args, mask, 4.0, W_t=args[2].t().contiguous())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_alternating_shapes_share_the_workspace():
    """The reduction-slice counters live in the workspace and must be left clear:
    shapes with different slice counts (U in 3, T in 3, none) alternate on one
    workspace, and every repeat is bitwise identical (slices are summed in a fixed
    order)."""
    shapes = [(256, 1024, 3072, 32), (128, 3072, 1024, 64), (64, 512, 512, 16)]
    runs = []
    for M, K, N, r in shapes:
        X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=9)
        G = workloads.gemm_grad(M, N, seed=9)
        runs.append(([to_device(a, DEV) for a in (G, X, W, A, B)],
                     to_device(workloads.noise_row_mask(M // 8, 8), DEV)))

    def once(args, mask):
        out = [t.clone() for t in _uno().uno_gated_lora_linear_bwd(*args, mask, 4.0)]
        torch.cuda.synchronize()
        return [t.view(torch.int16).cpu() for t in out]

    first = [once(*run) for run in runs]
    for _ in range(2):
        for run, ref in zip(reversed(runs), reversed(first)):
            for a, b in zip(once(*run), ref):
                assert torch.equal(a, b)


def test_backward_on_two_streams():
    """Backward calls on two streams at once, each with its own workspace: the
    LoRA-down slice counters and dX's slice tiles live in the workspace, so results
    equal the same calls made one at a time."""
    shapes = [(512, 2560, 2560, 64), (256, 1024, 3072, 32)]
    runs = []
    for M, K, N, r in shapes:
        X, W, A, B = workloads.gemm_inputs(M, K, N, r, seed=12)
        G = workloads.gemm_grad(M, N, seed=12)
        runs.append(([to_device(a, DEV) for a in (G, X, W, A, B)], to_device(workloads.noise_row_mask(M // 8, 8), DEV)))

    def call(run):
        args, mask = run
        return _uno().uno_gated_lora_linear_bwd(*args, mask, 4.0)

    ref = []
    for run in runs:
        out = call(run)
        torch.cuda.synchronize()
        ref.append([t.view(torch.int16).cpu() for t in out])
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    for rep in range(3):
        outs = [[None] * len(runs) for _ in streams]
        for si, st in enumerate(streams):
            with torch.cuda.stream(st):
                for i in (range(len(runs)) if si == 0 else reversed(range(len(runs)))):
                    outs[si][i] = call(runs[i])
        torch.cuda.synchronize()
        for si in range(len(streams)):
            for i in range(len(runs)):
                for a, b in zip(outs[si][i], ref[i]):
                    assert torch.equal(a.view(torch.int16).cpu(), b)
