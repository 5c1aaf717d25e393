"""Plain fp64 CPU oracle of the Uno decode step on a synthetic decoder stack.

TEST INFRASTRUCTURE ONLY: used by the tests and the smoke check; never by the
product library. Shares no code with the HIP path.

What it follows (page titles as headed on the pages):

* "LoopUno: Turning Agentic Looped LLMs into Diffusion LLMs in One Hour", section
  "How it works": each decode step drafts a block of positions in one forward, with
  the adapter switched on for the noise positions only; the unmodified model then
  verifies the block and the longest correct prefix is kept; the first position is
  always the exact AR token. Section "Why the looped model fits" and "Setup /
  Recipe": the looped model runs its 22 layers twice per token with shared weights,
  and the gated adapter sits on all seven projections. "Limits and next steps":
  drafting with one loop instead of two.
* "Uno Qwen3-8B" model card, "Evaluation protocol": the noise mode is
  random_uniform (noise tokens uniform over the vocabulary).

Readings (listed in the design notes):

* A step is a draft forward of the block rows [seed, noise_1 .. noise_{b-1}] with
  the adapter on the noise rows, the draft sampler on its logits, a frozen verify
  forward of the rows [seed, d_1 .. d_{b-1}], and lossless verification with p from
  the verify forward and q from the draft forward.
* The synthetic stack: x = rmsnorm(h) (unit gain, eps 1e-6); q, k, v = gated(x);
  attention over a one-token context (each row attends to itself, so query head j
  returns the value of kv head j // (query heads / kv heads)); h += gated_o(a);
  x = rmsnorm(h); h += gated_down(silu(gated_gate(x)) * gated_up(x)); finally
  logits = rmsnorm(h) lm_head^T.
* Tensors the path stores in bf16 (activations between steps, the residual
  stream) are rounded to bf16 (nearest even) at the same points here; everything
  else is fp64. The gated products are oracle.gated_lora_linear (T unrounded).
"""

import numpy as np

from .gated_lora import bf16_bits_to_f64, gated_lora_linear
from .philox import noise_token
from .sampling import draft_sample, verify_block

NORM_EPS = 1e-6


def to_bf16_bits(x):
    """fp64 -> bf16 bit patterns, round to nearest even (through the fp32 value)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rmsnorm(h):
    """h / sqrt(mean(h^2) + eps) per row, unit gain (fp64)."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt((h * h).mean(axis=-1, keepdims=True) + NORM_EPS)


def silu(x):
    return x / (1.0 + np.exp(-x))


def one_token_attention(v, hidden, head_dim):
    """Attention of each row over a context of itself alone: the softmax over one
    key is 1, so query head j returns the value row of its kv head."""
    kv_heads = v.shape[1] // head_dim
    group = (hidden // head_dim) // kv_heads
    heads = [v[:, (j // group) * head_dim:(j // group + 1) * head_dim] for j in range(hidden // head_dim)]
    return np.concatenate(heads, axis=1)


def _gated(model, layer, proj, x_bits, mask):
    """bf16 output of one gated projection (adapter on rows with mask 1; frozen when
    mask is None)."""
    W = model["weights"][layer][proj]
    r = model["rank"]
    if mask is None or r == 0:
        y = bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(W).T
    else:
        y = gated_lora_linear(x_bits, W, model["lora_a"][layer][proj], model["lora_b"][layer][proj], mask,
                              model["lora_scale"])
    return to_bf16_bits(y)


def forward(model, tokens, row_mask=None, loops=1):
    """fp64 logits [M, V] of the token rows. model: dict of bf16 bit arrays
    (embed, lm_head [V, H]; weights[l][j] for j in q, k, v, o, gate, up, down;
    lora_a, lora_b likewise) and sizes (head_dim, rank, lora_scale)."""
    E = model["embed"]
    H = E.shape[1]
    h = E[np.asarray(tokens, dtype=np.int64)]                       # exact bf16 rows
    x = to_bf16_bits(rmsnorm(bf16_bits_to_f64(h)))
    for _ in range(loops):
        for layer in range(len(model["weights"])):
            _q = _gated(model, layer, 0, x, row_mask)                 # q and k do not reach the output
            _k = _gated(model, layer, 1, x, row_mask)
            v = _gated(model, layer, 2, x, row_mask)
            a = one_token_attention(v, H, model["head_dim"])
            o = _gated(model, layer, 3, a, row_mask)
            h = to_bf16_bits(bf16_bits_to_f64(h) + bf16_bits_to_f64(o))
            x = to_bf16_bits(rmsnorm(bf16_bits_to_f64(h)))
            g = _gated(model, layer, 4, x, row_mask)
            u = _gated(model, layer, 5, x, row_mask)
            m = to_bf16_bits(silu(bf16_bits_to_f64(g)) * bf16_bits_to_f64(u))
            d = _gated(model, layer, 6, m, row_mask)
            h = to_bf16_bits(bf16_bits_to_f64(h) + bf16_bits_to_f64(d))
            x = to_bf16_bits(rmsnorm(bf16_bits_to_f64(h)))
    return bf16_bits_to_f64(x) @ bf16_bits_to_f64(model["lm_head"]).T


def block_rows(seed_tokens, seq_ids, pos, b, vocab, seed):
    """Draft-forward rows [seed, noise_1 .. noise_{b-1}] per sequence and their noise mask."""
    S = len(seed_tokens)
    toks = np.zeros((S, b), dtype=np.int64)
    mask = np.zeros((S, b), dtype=np.uint8)
    for s in range(S):
        toks[s, 0] = seed_tokens[s]
        for i in range(1, b):
            toks[s, i] = noise_token(seed, seq_ids[s], int(pos[s]) + i, vocab)
            mask[s, i] = 1
    return toks.reshape(-1), mask.reshape(-1)


def decode_step(model, seed_tokens, seq_ids, pos, b, temperature, top_k, top_p, seed, draft_loops=1,
                verify_loops=1):
    """One Uno step of S sequences and block b. Returns the verifier's dict plus
    drafts, draft_logits and verify_logits ([S*b, V] fp64) and the noise rows."""
    S = len(seed_tokens)
    V = model["embed"].shape[0]
    rows, mask = block_rows(seed_tokens, seq_ids, pos, b, V, seed)
    zd = forward(model, rows, mask, draft_loops)
    q = zd.astype(np.float32).reshape(S, b, V)
    drafts, _ = draft_sample(q, seq_ids, pos, temperature, top_k, top_p, seed, "f32")
    vrows = drafts.astype(np.int64).copy()
    vrows[:, 0] = seed_tokens
    zv = forward(model, vrows.reshape(-1), None, verify_loops)
    p = zv.astype(np.float32).reshape(S, b, V)
    out = verify_block(p, q, drafts, seq_ids, pos, temperature, top_k, top_p, seed, "f32")
    out.update(drafts=drafts, draft_logits=zd, verify_logits=zv, noise_rows=rows.reshape(S, b))
    return out


def ar_step(model, tokens, seq_ids, pos, temperature, top_k, top_p, seed, loops=1):
    """One autoregressive step: the frozen forward of the rows, then slot 0 of the
    verifier (the AR draw). Returns (tokens [S], logits [S, V] fp64)."""
    S = len(tokens)
    V = model["embed"].shape[0]
    z = forward(model, np.asarray(tokens, dtype=np.int64), None, loops)
    p = z.astype(np.float32).reshape(S, 1, V)
    out = verify_block(p, p, np.zeros((S, 1), np.int32), seq_ids, pos, temperature, top_k, top_p, seed, "f32")
    return out["out_tokens"][:, 0], z
