"""Seeded synthetic inputs for the Uno block draft-and-verify hot path.

This module is the only code that both the CPU oracle's tests and the HIP path
read from. It holds none of the method's arithmetic: only seeded random draws,
their rounding to the storage type, the shapes of each workload and the noise-row
layout of a block.

Workloads (shapes and distributions as stated for each configuration; readings
where a value is not given are marked "reading"):

* ``tiny``   1 sequence x block 8, vocab 1024, fp32 logits, base ~ N(0, 2^2),
             draft = base + N(0, 0.5^2); gated LoRA d_in = d_out = 256, rank 16,
             8 rows, rows 1..7 noise rows; W ~ N(0, 0.02^2), A, B ~ N(0, 0.01^2),
             X ~ N(0, 1) (reading).
* ``qwen``   64 sequences x block 16, vocab 151936, bf16 logits, base ~ N(0, 3^2),
             draft = base + N(0, 0.7^2); rank-128 gated LoRA on 4096->4096 and
             4096->12288 projections over M = 64*16 rows, noise rows = slots 1..15.
* ``looped`` 64 x block 8, vocab 166144, base ~ N(0, 3^2) (reading), draft = base +
             N(0, 0.9^2); seven gated projections of a hidden-2560 / FFN-10240 layer,
             rank 64, M = 512.
* ``selfdistill`` 8 x 4096 tokens, response mask on the last 3072 of each
             sequence, vocab 151936, teacher ~ N(0, 3^2), student = teacher + N(0, 1).
* ``stress`` 256 x block 16, vocab 151936, base = 2 * Student-t(nu = 3),
             draft = base + N(0, 0.5^2); seven gated projections of a 4096-hidden /
             12288-FFN layer (k/v 4096->1024, reading), rank 128, M = 4096.

Sampling settings for every verify workload: T = 1.0, top-k 50, top-p 0.95,
Philox seed 0, sequence ids 0..S-1, position offsets 0.

Every logit row is generated from its own PCG64 stream keyed by (seed, workload,
sequence, slot), so any subset of rows can be regenerated on its own.
"""

import concurrent.futures
import os

import numpy as np

VERIFY_CONFIGS = {
    "tiny": dict(S=1, b=8, V=1024, dtype="f32", base="normal", base_sigma=2.0, draft_sigma=0.5),
    "qwen": dict(S=64, b=16, V=151936, dtype="bf16", base="normal", base_sigma=3.0, draft_sigma=0.7),
    "looped": dict(S=64, b=8, V=166144, dtype="bf16", base="normal", base_sigma=3.0, draft_sigma=0.9),
    "stress": dict(S=256, b=16, V=151936, dtype="bf16", base="student_t3", base_sigma=2.0, draft_sigma=0.5),
}

SAMPLING = dict(temperature=1.0, top_k=50, top_p=0.95, seed=0)

# Gated-LoRA projections (K = d_in, N = d_out) per workload.
GEMM_CONFIGS = {
    "tiny": dict(M=8, r=16, b=8, projections=[("proj", 256, 256)]),
    "qwen": dict(M=1024, r=128, b=16, projections=[("attn_4096x4096", 4096, 4096),
                                                    ("mlp_4096x12288", 4096, 12288)]),
    "looped": dict(M=512, r=64, b=8, projections=[
        ("q", 2560, 2560), ("k", 2560, 2560), ("v", 2560, 2560), ("o", 2560, 2560),
        ("gate", 2560, 10240), ("up", 2560, 10240), ("down", 10240, 2560)]),
    "stress": dict(M=4096, r=128, b=16, projections=[
        ("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
        ("gate", 4096, 12288), ("up", 4096, 12288), ("down", 12288, 4096)]),
}

TV_CONFIG = dict(n_seq=8, seq_len=4096, resp_len=3072, V=151936, teacher_sigma=3.0,
                 student_sigma=1.0, temperature=1.0)

_TAGS = {"tiny": 1, "qwen": 2, "looped": 3, "stress": 4, "selfdistill": 5, "custom": 9}


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _base_draw(rng, kind, sigma, n):
    if kind == "normal":
        return (sigma * rng.standard_normal(n, dtype=np.float32)).astype(np.float32)
    if kind == "student_t3":
        return (sigma * rng.standard_t(3, size=n)).astype(np.float32)
    raise ValueError(kind)


def logit_row_pair(cfg, s, i, seed=0, V=None):
    """(base_row, draft_row) float32 for sequence s, slot i of a verify workload."""
    c = VERIFY_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    tag = _TAGS.get(cfg, 9) if isinstance(cfg, str) else 9
    V = c["V"] if V is None else V
    rng = _rng(seed, tag, s, i)
    base = _base_draw(rng, c["base"], c["base_sigma"], V)
    draft = base + np.float32(c["draft_sigma"]) * rng.standard_normal(V, dtype=np.float32)
    return base, draft.astype(np.float32)


def verify_logits(cfg, seed=0, seqs=None, V=None, threads=None):
    """Base and draft logits [S', b, V] for the listed sequences (default: all).

    bf16 workloads return uint16 bit patterns, fp32 workloads float32 values. Rows
    are drawn on a thread pool (numpy's generators release the GIL while they fill
    a row); each row has its own stream, so the result does not depend on `threads`.
    """
    c = VERIFY_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    V = c["V"] if V is None else V
    seqs = range(c["S"]) if seqs is None else list(seqs)
    n = len(seqs)
    out_t = np.uint16 if c["dtype"] == "bf16" else np.float32
    p = np.empty((n, c["b"], V), dtype=out_t)
    q = np.empty((n, c["b"], V), dtype=out_t)

    def fill(job):
        a, s = job
        for i in range(c["b"]):
            base, draft = logit_row_pair(cfg, s, i, seed, V)
            if c["dtype"] == "bf16":
                p[a, i] = to_bf16_bits(base)
                q[a, i] = to_bf16_bits(draft)
            else:
                p[a, i] = base
                q[a, i] = draft

    jobs = list(enumerate(seqs))
    nthreads = min(16, os.cpu_count() or 1) if threads is None else max(1, int(threads))
    if nthreads == 1 or n * c["b"] * V < (1 << 22):
        for job in jobs:
            fill(job)
    else:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, jobs))
    return p, q


def noise_row_mask(S, b):
    """Row mask of a batch of S blocks of b rows: slot 0 is the seed/verify row (0),
    slots 1..b-1 are noise rows (1)."""
    m = np.ones((S, b), dtype=np.uint8)
    m[:, 0] = 0
    return m.reshape(-1)


def gemm_inputs(M, K, N, r, seed=0, tag=0):
    """bf16 bit patterns X [M,K] ~ N(0,1), W [N,K] ~ N(0,.02^2), A [r,K], B [N,r] ~ N(0,.01^2)."""
    X = to_bf16_bits(_rng(seed, 100, tag, 0, M, K).standard_normal((M, K), dtype=np.float32))
    W = to_bf16_bits(np.float32(0.02) * _rng(seed, 100, tag, 1, N, K).standard_normal((N, K), dtype=np.float32))
    A = to_bf16_bits(np.float32(0.01) * _rng(seed, 100, tag, 2, r, K).standard_normal((r, K), dtype=np.float32))
    B = to_bf16_bits(np.float32(0.01) * _rng(seed, 100, tag, 3, N, r).standard_normal((N, r), dtype=np.float32))
    return X, W, A, B


def gemm_grad(M, N, seed=0, tag=0):
    """bf16 bit patterns of an upstream gradient dY [M,N] ~ N(0, 0.01^2)."""
    return to_bf16_bits(np.float32(0.01) * _rng(seed, 101, tag, 0, M, N).standard_normal((M, N), dtype=np.float32))


def tv_response_mask(n_seq, seq_len, resp_len):
    m = np.zeros((n_seq, seq_len), dtype=np.uint8)
    m[:, seq_len - resp_len:] = 1
    return m.reshape(-1)


def tv_rows(rows, V, seed=0, teacher_sigma=3.0, student_sigma=1.0):
    """Teacher / student bf16 bit patterns for the listed flat row indices (row-addressable)."""
    rows = list(rows)
    t = np.empty((len(rows), V), dtype=np.uint16)
    s = np.empty((len(rows), V), dtype=np.uint16)
    for a, r in enumerate(rows):
        rng = _rng(seed, _TAGS["selfdistill"], r)
        tf = np.float32(teacher_sigma) * rng.standard_normal(V, dtype=np.float32)
        sf = tf + np.float32(student_sigma) * rng.standard_normal(V, dtype=np.float32)
        t[a] = to_bf16_bits(tf)
        s[a] = to_bf16_bits(sf)
    return t, s


def tv_inputs_torch(n_rows, V, device, seed=0, teacher_sigma=3.0, student_sigma=1.0, chunk=2048):
    """Teacher / student bf16 torch tensors [n_rows, V] drawn on `device` by torch's own
    generator (for the full-size workload, where drawing 10^10 values on the host is too
    slow). Rows are drawn in fixed chunks so the result depends only on (seed, V, chunk)."""
    import torch
    t = torch.empty((n_rows, V), dtype=torch.bfloat16, device=device)
    s = torch.empty((n_rows, V), dtype=torch.bfloat16, device=device)
    g = torch.Generator(device=device)
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        g.manual_seed(int(seed) * 1_000_003 + r0)
        tf = torch.randn((r1 - r0, V), generator=g, device=device, dtype=torch.float32) * teacher_sigma
        sf = tf + torch.randn((r1 - r0, V), generator=g, device=device, dtype=torch.float32) * student_sigma
        t[r0:r1] = tf.to(torch.bfloat16)
        s[r0:r1] = sf.to(torch.bfloat16)
        del tf, sf
    return t, s


# Decoder stacks of the decode step (uno_decode_step). "qwen": Qwen3-8B shapes
# (36 layers, hidden 4096, 8 kv heads of 128, FFN 12288, vocabulary 151936), rank-128
# adapter, block 16. "looped": the 3B-class looped stack of 22 layers run twice per
# token (hidden 2560, every attention projection 2560 x 2560 (reading), FFN 10240,
# vocabulary 166144), rank-64 adapter, block 8. "small" and "small_looped": reduced
# stacks of the same structure for oracle comparisons. Four sequences per step.
STEP_CONFIGS = {
    "qwen": dict(hidden=4096, kv_width=1024, head_dim=128, ffn=12288, vocab=151936, layers=36, rank=128,
                 b=16, S=4, loops=1),
    "looped": dict(hidden=2560, kv_width=2560, head_dim=128, ffn=10240, vocab=166144, layers=22, rank=64,
                   b=8, S=4, loops=2),
    "small": dict(hidden=1024, kv_width=256, head_dim=128, ffn=3072, vocab=32000, layers=2, rank=64,
                  b=8, S=4, loops=1),
    "small_looped": dict(hidden=768, kv_width=768, head_dim=128, ffn=2048, vocab=20000, layers=2, rank=32,
                         b=8, S=4, loops=2),
}
STEP_PROJ_SHAPES = ("q", "k", "v", "o", "gate", "up", "down")


def step_proj_dims(cfg):
    """(out, in) of the seven projections of one layer."""
    H, KV, F = cfg["hidden"], cfg["kv_width"], cfg["ffn"]
    return [(H, H), (KV, H), (KV, H), (H, H), (F, H), (F, H), (H, F)]


def step_model_host(cfg, seed=0, embed_sigma=1.0, weight_sigma=0.02, lora_sigma=0.01):
    """A decoder stack as bf16 bit patterns (uint16): embed / lm_head [V, H] ~
    N(0, embed_sigma^2) / N(0, weight_sigma^2); projection weights [out, in] ~
    N(0, weight_sigma^2); adapter factors A [r, in], B [out, r] ~ N(0, lora_sigma^2)."""
    c = STEP_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    V, H, r = c["vocab"], c["hidden"], c["rank"]

    def draw(sigma, shape, *key):
        return to_bf16_bits(np.float32(sigma) * _rng(seed, 200, *key).standard_normal(shape, dtype=np.float32))

    m = dict(embed=draw(embed_sigma, (V, H), 0), lm_head=draw(weight_sigma, (V, H), 1),
             weights=[], lora_a=[], lora_b=[], head_dim=c["head_dim"], rank=r, lora_scale=1.0)
    for layer in range(c["layers"]):
        dims = step_proj_dims(c)
        m["weights"].append([draw(weight_sigma, d, 2, layer, j) for j, d in enumerate(dims)])
        if r:
            m["lora_a"].append([draw(lora_sigma, (r, d[1]), 3, layer, j) for j, d in enumerate(dims)])
            m["lora_b"].append([draw(lora_sigma, (d[0], r), 4, layer, j) for j, d in enumerate(dims)])
    return m


def step_model_torch(cfg, device, seed=0, embed_sigma=1.0, weight_sigma=0.02, lora_sigma=0.01):
    """The same structure drawn on `device` by torch's generator (for the full-size
    stacks, whose 10^10 weights are too many to draw on the host)."""
    import torch
    c = STEP_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    V, H, r = c["vocab"], c["hidden"], c["rank"]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 7919 + 17)

    def draw(sigma, shape):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma).to(torch.bfloat16)

    m = dict(embed=draw(embed_sigma, (V, H)), lm_head=draw(weight_sigma, (V, H)), weights=[], lora_a=[],
             lora_b=[], head_dim=c["head_dim"], rank=r, lora_scale=1.0)

    def stacked(sigma, shapes):
        # q, k, v (and gate, up) drawn as one allocation and split into row views, so
        # that the forward can run them as one grouped product
        rows = [s[0] for s in shapes]
        return list(torch.split(draw(sigma, (sum(rows), shapes[0][1])), rows, dim=0))

    def layer(sigma, shapes):
        return stacked(sigma, shapes[0:3]) + [draw(sigma, shapes[3])] + stacked(sigma, shapes[4:6]) + \
            [draw(sigma, shapes[6])]
    for _ in range(c["layers"]):
        dims = step_proj_dims(c)
        m["weights"].append(layer(weight_sigma, dims))
        if r:
            m["lora_a"].append(layer(lora_sigma, [(r, d[1]) for d in dims]))
            m["lora_b"].append(layer(lora_sigma, [(d[0], r) for d in dims]))
    return m
