"""Plain fp64 CPU oracle of the row-gated LoRA linear layer.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
CPU-baseline leg; never by the product library. Shares no code with the HIP path.

Follows the "Uno Qwen3-8B" model card (opening paragraphs): the rank-128 gated
LoRA adapter is applied only during draft-noise forwards, while seed, prefill,
verification and autoregressive rows use the frozen base weights; loading it as
an always-on adapter does not reproduce Uno. The "LoopUno" page, section
"Setup / Recipe", gives the adapter as gated LoRA r=128, alpha=2048 on all seven
projections, noise rows only, so the LoRA scale is s = alpha / r.

    Y[m, n] = sum_k X[m,k] W[n,k] + s * mask[m] * sum_j (sum_k X[m,k] A[j,k]) B[n,j]

Reading: W, A, B use the nn.Linear / PEFT storage (W [N,K], lora_A [r,K],
lora_B [N,r]); the pages' X.W is this with W transposed.
"""

import numpy as np


def bf16_bits_to_f64(x):
    x = np.asarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 tensors are passed as uint16 bit patterns")
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gated_lora_linear(X, W, A, B, row_mask, scale):
    """fp64 Y [M,N] from bf16 bit-pattern inputs."""
    x = bf16_bits_to_f64(X)
    w = bf16_bits_to_f64(W)
    a = bf16_bits_to_f64(A)
    bb = bf16_bits_to_f64(B)
    m = np.asarray(row_mask).astype(np.float64)
    base = x @ w.T
    delta = (x @ a.T) @ bb.T
    return base + scale * m[:, None] * delta


def lora_delta(X, A, B, scale):
    """s * (X A^T) B^T for every row (the adapter's contribution, ungated)."""
    x = bf16_bits_to_f64(X)
    a = bf16_bits_to_f64(A)
    bb = bf16_bits_to_f64(B)
    return scale * ((x @ a.T) @ bb.T)


def gated_lora_linear_bwd(X, W, A, B, row_mask, scale, dY):
    """fp64 gradients (dX [M,K], dA [r,K], dB [N,r]) of the row-gated LoRA linear for
    an upstream gradient dY [M,N]; the frozen base weight W gets none.

    The adapter is trained by self-distillation on the noise rows only ("LoopUno",
    "How it works" -> "Training is self-distillation"; "Setup / Recipe": gated LoRA
    on the noise rows). By the chain rule on Y = X W^T + s diag(m) (X A^T) B^T:

        U  = s diag(m) dY B            [M, r]
        dX = dY W + U A                [M, K]
        dA = U^T X                     [r, K]
        dB = s (diag(m) dY)^T (X A^T)  [N, r]
    """
    x = bf16_bits_to_f64(X)
    w = bf16_bits_to_f64(W)
    a = bf16_bits_to_f64(A)
    bb = bf16_bits_to_f64(B)
    g = bf16_bits_to_f64(dY)
    m = np.asarray(row_mask).astype(np.float64)
    gm = m[:, None] * g
    u = scale * (gm @ bb)
    dx = g @ w + u @ a
    da = u.T @ x
    db = scale * (gm.T @ (x @ a.T))
    return dx, da, db
