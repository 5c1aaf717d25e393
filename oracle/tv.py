"""Plain fp64 CPU oracle of the total-variation self-distillation loss and its gradient.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
CPU-baseline leg; never by the product library. Shares no code with the HIP path.

Follows "LoopUno: Turning Agentic Looped LLMs into Diffusion LLMs in One Hour",
section "How it works" -> "Training is self-distillation": each sequence is seen
as a clean copy through the frozen model (teacher, distribution p) and a
block-noised copy through model + LoRA (student, distribution q); the loss is
the total-variation distance between the two next-token distributions on the
response tokens, and 1 - TV is the acceptance probability of lossless
verification. The gradient flows to the student only (the teacher is frozen).

Readings (listed in the design notes):
* p = softmax(teacher / T), q = softmax(student / T) over the full vocabulary,
  no top-k / top-p.
* TV_row = 1/2 * sum_v |p_v - q_v|.
* L = sum_rows mask * TV_row / sum_rows mask (token mean over response rows of
  the whole batch); L = 0 when no row is a response row.
* dL/dz_j = q_j * (g_j - sum_v q_v g_v) / (T * N_resp), g_v = 1/2 sign(q_v - p_v),
  sign(0) = 0; zero on rows outside the response mask.
"""

import numpy as np

from .sampling import decode_logits


def softmax_rows(z, temperature):
    z = np.asarray(z, dtype=np.float64) / temperature
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def tv_loss_fwd_bwd(teacher_logits, student_logits, response_mask, temperature,
                    dtype="bf16", want_grad=True):
    """Returns (loss, tv_rows [R], grad [R,V] or None), all fp64."""
    if not temperature > 0:
        raise ValueError("temperature must be > 0 for the TV loss")
    t = decode_logits(teacher_logits, dtype)
    s = decode_logits(student_logits, dtype)
    mask = np.asarray(response_mask).astype(bool)
    p = softmax_rows(t, temperature)
    q = softmax_rows(s, temperature)
    tv = 0.5 * np.abs(p - q).sum(axis=-1)
    tv = np.where(mask, tv, 0.0)
    n = int(mask.sum())
    loss = float(tv[mask].sum() / n) if n else 0.0
    grad = None
    if want_grad:
        grad = np.zeros_like(q)
        if n:
            g = 0.5 * np.sign(q - p)
            qg = (q * g).sum(axis=-1, keepdims=True)
            grad = q * (g - qg) / (temperature * n)
            grad[~mask] = 0.0
    return loss, tv, grad
