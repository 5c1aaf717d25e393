"""Python entry points with the C ABI's names (include/uno.h), over torch tensors.

Each function validates shapes and dtypes, allocates outputs, and calls the
library on the current HIP stream of the inputs' device. Results are
asynchronous like any other work on that stream.
"""

import torch

from . import _lib
import ctypes

from ._lib import SamplingParams, UnoModel, WORKSPACES, check, load, ptr, require, stream_handle


def sampling_params(temperature=1.0, top_k=50, top_p=0.95, seed=0):
    return SamplingParams(float(temperature), float(top_p), int(top_k), int(seed) & (2**64 - 1))


def _verify_outputs(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets, want_slot_accept, want_diag, out):
    if p_logits.dim() != 3:
        raise ValueError("p_logits must be [S, b, V]")
    S, b, V = p_logits.shape
    dev = p_logits.device
    require(p_logits, "p_logits")
    require(q_logits, "q_logits", dtype=p_logits.dtype, shape=(S, b, V), device=dev)
    require(draft_tokens, "draft_tokens", dtype=torch.int32, shape=(S, b), device=dev)
    require(seq_ids, "seq_ids", dtype=torch.int64, shape=(S,), device=dev)
    require(pos_offsets, "pos_offsets", dtype=torch.int64, shape=(S,), device=dev)
    o = dict(out or {})
    if "out_tokens" not in o:
        o["out_tokens"] = torch.empty((S, b), dtype=torch.int32, device=dev)
    if "accept_len" not in o:
        o["accept_len"] = torch.empty((S,), dtype=torch.int32, device=dev)
    if "resampled" not in o:
        o["resampled"] = torch.empty((S,), dtype=torch.int32, device=dev)
    if want_slot_accept and "slot_accept" not in o:
        o["slot_accept"] = torch.empty((S, b), dtype=torch.uint8, device=dev)
    if want_diag and "diag" not in o:
        o["diag"] = torch.empty((S, b, 4), dtype=torch.float32, device=dev)
    return S, b, V, dev, o


def uno_verify_block(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets,
                     temperature=1.0, top_k=50, top_p=0.95, seed=0,
                     want_slot_accept=True, want_diag=True, out=None):
    """Lossless verification of a [S, b, V] block (see uno_verify_block in uno.h).

    Returns a dict of device tensors: out_tokens [S,b] int32, accept_len [S] int32,
    resampled [S] int32, and optionally slot_accept [S,b] uint8, diag [S,b,4] f32.
    `out` may pass preallocated tensors under the same keys.
    """
    lib = load()
    S, b, V, dev, o = _verify_outputs(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets,
                                      want_slot_accept, want_diag, out)
    stream = stream_handle(dev)
    nws = lib.uno_verify_block_workspace(S, b, V)
    ws = WORKSPACES.get(dev, stream, "verify", nws)
    sp = sampling_params(temperature, top_k, top_p, seed)
    st = lib.uno_verify_block(ptr(p_logits), ptr(q_logits), _lib.dtype_code(p_logits),
                              ptr(draft_tokens), ptr(seq_ids), ptr(pos_offsets), S, b, V, sp,
                              ptr(o["out_tokens"]), ptr(o["accept_len"]), ptr(o["resampled"]),
                              ptr(o.get("slot_accept")), ptr(o.get("diag")),
                              ptr(ws), ws.numel(), stream)
    check(st, "uno_verify_block")
    return o


def uno_verify_block_noalloc(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets,
                             temperature=1.0, top_k=50, top_p=0.95, seed=0,
                             want_slot_accept=True, want_diag=True, out=None):
    """uno_verify_block without a workspace: the library's own device scratch holds the
    tickets and slot records (see uno_verify_block_noalloc in uno.h). With every output
    passed in `out`, this call allocates nothing on the device."""
    lib = load()
    S, b, V, dev, o = _verify_outputs(p_logits, q_logits, draft_tokens, seq_ids, pos_offsets,
                                      want_slot_accept, want_diag, out)
    sp = sampling_params(temperature, top_k, top_p, seed)
    st = lib.uno_verify_block_noalloc(ptr(p_logits), ptr(q_logits), _lib.dtype_code(p_logits),
                                      ptr(draft_tokens), ptr(seq_ids), ptr(pos_offsets), S, b, V, sp,
                                      ptr(o["out_tokens"]), ptr(o["accept_len"]), ptr(o["resampled"]),
                                      ptr(o.get("slot_accept")), ptr(o.get("diag")), stream_handle(dev))
    check(st, "uno_verify_block_noalloc")
    return o


def uno_draft_sample(q_logits, seq_ids, pos_offsets, temperature=1.0, top_k=50, top_p=0.95,
                     seed=0, want_flags=True):
    """Draft tokens d[s,i] ~ q~[s,i] (Philox stream 1). Returns (draft [S,b] int32, flags or None)."""
    lib = load()
    if q_logits.dim() != 3:
        raise ValueError("q_logits must be [S, b, V]")
    S, b, V = q_logits.shape
    dev = q_logits.device
    require(q_logits, "q_logits")
    require(seq_ids, "seq_ids", dtype=torch.int64, shape=(S,), device=dev)
    require(pos_offsets, "pos_offsets", dtype=torch.int64, shape=(S,), device=dev)
    draft = torch.empty((S, b), dtype=torch.int32, device=dev)
    flags = torch.empty((S, b), dtype=torch.int32, device=dev) if want_flags else None
    sp = sampling_params(temperature, top_k, top_p, seed)
    st = lib.uno_draft_sample(ptr(q_logits), _lib.dtype_code(q_logits), ptr(seq_ids),
                              ptr(pos_offsets), S, b, V, sp, ptr(draft), ptr(flags),
                              stream_handle(dev))
    check(st, "uno_draft_sample")
    return draft, flags


def uno_tv_loss_fwd_bwd(teacher_logits, student_logits, response_mask, temperature=1.0,
                        want_grad=True, want_rows=True):
    """TV self-distillation loss and gradient. Returns (loss [1] f32, tv_rows or None, grad or None)."""
    lib = load()
    if teacher_logits.dim() != 2:
        raise ValueError("teacher_logits must be [R, V]")
    R, V = teacher_logits.shape
    dev = teacher_logits.device
    require(teacher_logits, "teacher_logits")
    require(student_logits, "student_logits", dtype=teacher_logits.dtype, shape=(R, V), device=dev)
    require(response_mask, "response_mask", dtype=torch.uint8, shape=(R,), device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    rows = torch.empty((R,), dtype=torch.float32, device=dev) if want_rows else None
    grad = torch.empty_like(student_logits) if want_grad else None
    stream = stream_handle(dev)
    ws = WORKSPACES.get(dev, stream, "tv", lib.uno_tv_loss_workspace(R, V))
    st = lib.uno_tv_loss_fwd_bwd(ptr(teacher_logits), ptr(student_logits),
                                 _lib.dtype_code(teacher_logits), ptr(response_mask), R, V,
                                 float(temperature), ptr(loss), ptr(rows), ptr(grad),
                                 ptr(ws), ws.numel(), stream)
    check(st, "uno_tv_loss_fwd_bwd")
    return loss, rows, grad


def uno_gated_lora_linear(X, W, A, B, row_mask, scale=1.0, out=None):
    """Y = X W^T + scale * row_mask * (X A^T) B^T in bf16 (see uno.h)."""
    lib = load()
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[0]
    dev = X.device
    require(X, "X", dtype=torch.bfloat16)
    require(W, "W", dtype=torch.bfloat16, shape=(N, K), device=dev)
    require(A, "A", dtype=torch.bfloat16, shape=(r, K), device=dev)
    require(B, "B", dtype=torch.bfloat16, shape=(N, r), device=dev)
    require(row_mask, "row_mask", dtype=torch.uint8, shape=(M,), device=dev)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    require(Y, "Y", dtype=torch.bfloat16, shape=(M, N), device=dev)
    stream = stream_handle(dev)
    ws = WORKSPACES.get(dev, stream, "gemm", lib.uno_gated_lora_linear_workspace(M, N, K, r))
    st = lib.uno_gated_lora_linear(ptr(X), ptr(W), ptr(A), ptr(B), ptr(row_mask), float(scale),
                                   ptr(Y), M, N, K, r, ptr(ws), ws.numel(), stream)
    check(st, "uno_gated_lora_linear")
    return Y


def uno_gated_lora_linear_bwd(dY, X, W, A, B, row_mask, scale=1.0, want_dx=True, W_t=None):
    """(dX or None, dA, dB) of the row-gated LoRA linear for an upstream dY (see uno.h).
    W_t, optional, is W^T [K, N] made once by the caller (the base weight is frozen)."""
    lib = load()
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[0]
    dev = X.device
    require(X, "X", dtype=torch.bfloat16)
    require(dY, "dY", dtype=torch.bfloat16, shape=(M, N), device=dev)
    require(W, "W", dtype=torch.bfloat16, shape=(N, K), device=dev)
    require(A, "A", dtype=torch.bfloat16, shape=(r, K), device=dev)
    require(B, "B", dtype=torch.bfloat16, shape=(N, r), device=dev)
    require(row_mask, "row_mask", dtype=torch.uint8, shape=(M,), device=dev)
    if W_t is not None:
        require(W_t, "W_t", dtype=torch.bfloat16, shape=(K, N), device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if want_dx else None
    dA = torch.empty((r, K), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
    stream = stream_handle(dev)
    ws = WORKSPACES.get(dev, stream, "gemm_bwd", lib.uno_gated_lora_linear_bwd_workspace(M, N, K, r))
    st = lib.uno_gated_lora_linear_bwd(ptr(dY), ptr(X), ptr(W), ptr(W_t), ptr(A), ptr(B), ptr(row_mask), float(scale),
                                       ptr(dX), ptr(dA), ptr(dB), M, N, K, r, ptr(ws), ws.numel(), stream)
    check(st, "uno_gated_lora_linear_bwd")
    return dX, dA, dB


PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


class Model:
    """A decoder stack for uno_forward / uno_decode_step / uno_ar_step: bf16 device
    tensors and the uno_model description that points at them (see uno.h).

    embed, lm_head: [V, H]; weights: list over layers of 7 tensors in the order of
    PROJECTIONS, nn.Linear layout [out, in]; lora_a / lora_b: the same nesting of
    [r, in] / [out, r] tensors, or None for no adapter."""

    def __init__(self, embed, lm_head, weights, lora_a=None, lora_b=None, kv_width=None, head_dim=128,
                 lora_scale=1.0):
        V, H = embed.shape
        L = len(weights)
        F = weights[0][4].shape[0] if L else 0
        kvw = kv_width if kv_width is not None else (weights[0][1].shape[0] if L else H)
        r = lora_a[0][0].shape[0] if (lora_a and L) else 0
        for t, n in ((embed, "embed"), (lm_head, "lm_head")):
            require(t, n, dtype=torch.bfloat16, shape=(V, H))
        flat = [t for layer in weights for t in layer]
        for t in flat:
            require(t, "weight", dtype=torch.bfloat16, device=embed.device)
        self.tensors = [embed, lm_head] + flat
        self._w = (ctypes.c_void_p * max(1, len(flat)))(*[t.data_ptr() for t in flat])
        self._a = self._b = None
        if r:
            fa = [t for layer in lora_a for t in layer]
            fb = [t for layer in lora_b for t in layer]
            for t in fa + fb:
                require(t, "adapter factor", dtype=torch.bfloat16, device=embed.device)
            self.tensors += fa + fb
            self._a = (ctypes.c_void_p * len(fa))(*[t.data_ptr() for t in fa])
            self._b = (ctypes.c_void_p * len(fb))(*[t.data_ptr() for t in fb])
        self.desc = UnoModel(H, kvw, head_dim, F, V, L, r, float(lora_scale), embed.data_ptr(),
                             lm_head.data_ptr(), ctypes.cast(self._w, ctypes.POINTER(ctypes.c_void_p)),
                             ctypes.cast(self._a, ctypes.POINTER(ctypes.c_void_p)) if r else None,
                             ctypes.cast(self._b, ctypes.POINTER(ctypes.c_void_p)) if r else None)
        self.device = embed.device
        self.vocab, self.hidden, self.rank = V, H, r


def uno_forward(model, tokens, row_mask=None, loops=1, logits=None):
    """fp32 logits [M, V] of one forward of the token rows (see uno_forward in uno.h)."""
    lib = load()
    M = tokens.shape[0]
    dev = model.device
    require(tokens, "tokens", dtype=torch.int32, shape=(M,), device=dev)
    if row_mask is not None:
        require(row_mask, "row_mask", dtype=torch.uint8, shape=(M,), device=dev)
    out = logits if logits is not None else torch.empty((M, model.vocab), dtype=torch.float32, device=dev)
    require(out, "logits", dtype=torch.float32, shape=(M, model.vocab), device=dev)
    n = lib.uno_forward_workspace(ctypes.byref(model.desc), M)   # 0: the call reports why
    ws = WORKSPACES.get(dev, stream_handle(dev), "step", max(n, 256))
    check(lib.uno_forward(ctypes.byref(model.desc), ptr(tokens), ptr(row_mask), M, int(loops), ptr(out),
                          ptr(ws), ws.numel() if n else 0, stream_handle(dev)), "uno_forward")
    return out


def uno_decode_step(model, b, seed_tokens, seq_ids, pos_offsets, temperature=1.0, top_k=50, top_p=0.95, seed=0,
                    draft_loops=1, verify_loops=1, want_logits=False, out=None):
    """One Uno decode step (see uno_decode_step in uno.h). Returns a dict of device
    tensors: out_tokens [S,b], accept_len [S], resampled [S], draft_tokens [S,b] and,
    with want_logits, draft_logits / verify_logits [S*b, V] fp32. `out` may pass
    preallocated tensors under the same keys (then nothing is allocated)."""
    lib = load()
    S = seed_tokens.shape[0]
    dev = model.device
    require(seed_tokens, "seed_tokens", dtype=torch.int32, shape=(S,), device=dev)
    require(seq_ids, "seq_ids", dtype=torch.int64, shape=(S,), device=dev)
    require(pos_offsets, "pos_offsets", dtype=torch.int64, shape=(S,), device=dev)
    o = dict(out or {})
    for k, shape, dt in (("out_tokens", (S, b), torch.int32), ("accept_len", (S,), torch.int32),
                         ("resampled", (S,), torch.int32), ("draft_tokens", (S, b), torch.int32)):
        if k not in o:
            o[k] = torch.empty(shape, dtype=dt, device=dev)
    if want_logits:
        for k in ("draft_logits", "verify_logits"):
            if k not in o:
                o[k] = torch.empty((S * b, model.vocab), dtype=torch.float32, device=dev)
    sp = sampling_params(temperature, top_k, top_p, seed)
    n = lib.uno_decode_step_workspace(ctypes.byref(model.desc), S, b)
    ws = WORKSPACES.get(dev, stream_handle(dev), "step", max(n, 256))
    st = lib.uno_decode_step(ctypes.byref(model.desc), S, b, int(draft_loops), int(verify_loops), sp,
                             ptr(seed_tokens), ptr(seq_ids), ptr(pos_offsets), ptr(o["out_tokens"]),
                             ptr(o["accept_len"]), ptr(o["resampled"]), ptr(o["draft_tokens"]),
                             ptr(o.get("draft_logits")), ptr(o.get("verify_logits")), ptr(ws),
                             ws.numel() if n else 0, stream_handle(dev))
    check(st, "uno_decode_step")
    return o


def uno_ar_step(model, tokens, seq_ids, pos_offsets, temperature=1.0, top_k=50, top_p=0.95, seed=0, loops=1,
                want_logits=False, out=None):
    """One autoregressive step (see uno_ar_step in uno.h): returns (out_tokens [S] int32,
    logits [S, V] fp32 or None)."""
    lib = load()
    S = tokens.shape[0]
    dev = model.device
    require(tokens, "tokens", dtype=torch.int32, shape=(S,), device=dev)
    require(seq_ids, "seq_ids", dtype=torch.int64, shape=(S,), device=dev)
    require(pos_offsets, "pos_offsets", dtype=torch.int64, shape=(S,), device=dev)
    o = dict(out or {})
    if "out_tokens" not in o:
        o["out_tokens"] = torch.empty((S,), dtype=torch.int32, device=dev)
    if want_logits and "logits" not in o:
        o["logits"] = torch.empty((S, model.vocab), dtype=torch.float32, device=dev)
    sp = sampling_params(temperature, top_k, top_p, seed)
    n = lib.uno_ar_step_workspace(ctypes.byref(model.desc), S)
    ws = WORKSPACES.get(dev, stream_handle(dev), "step", max(n, 256))
    st = lib.uno_ar_step(ctypes.byref(model.desc), S, int(loops), sp, ptr(tokens), ptr(seq_ids), ptr(pos_offsets),
                         ptr(o["out_tokens"]), ptr(o.get("logits")), ptr(ws), ws.numel() if n else 0,
                         stream_handle(dev))
    check(st, "uno_ar_step")
    return o["out_tokens"], o.get("logits")
