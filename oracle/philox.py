"""Philox-4x64-10 counter-based generator (oracle side; test infrastructure only).

Written from the published definition in J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (the Philox-4x64
round function, its two multipliers and its two Weyl key increments, 10 rounds).

The pages only fix that sampling runs at temperature 1.0 with one sample per
problem (Uno Qwen3-8B model card, "Evaluation protocol" table); they name no
generator. The verifier's uniforms are therefore drawn from this counter-based
generator keyed by (seed, sequence id) with the counter (absolute position,
stream, 0, 0), so every decision is reproducible from its inputs alone:

  * stream 0, word 0 -> u_acc (accept test), word 1 -> u_res (AR / residual draw)
  * stream 1, word 0 -> u_draft (the draft sampler's draw)
  * stream 2, word 0 -> the noise token of a block's noise row (random_uniform)

A 64-bit word w becomes u = (w >> 40) * 2**-24, a 24-bit uniform in [0, 1) that
is exact in both fp32 and fp64.

Pinned by tests against ``numpy.random.Philox`` (the same 4x64-10 generator).
"""

MASK64 = (1 << 64) - 1

# Round multipliers and key (Weyl) increments of Philox-4x64 (Salmon et al., SC'11).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B

STREAM_VERIFY = 0
STREAM_DRAFT = 1
STREAM_NOISE = 2


def _round(c, k):
    # One Philox-4x64 S-box/P-box round: two 64x64->128 multiplies, xor with key.
    prod0 = PHILOX_M0 * c[0]
    prod1 = PHILOX_M1 * c[2]
    hi0, lo0 = prod0 >> 64, prod0 & MASK64
    hi1, lo1 = prod1 >> 64, prod1 & MASK64
    return (hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0)


def philox4x64_10(counter, key):
    """Encrypt a 4-word counter under a 2-word key; returns 4 uint64 words."""
    c = tuple(int(x) & MASK64 for x in counter)
    k = tuple(int(x) & MASK64 for x in key)
    if len(c) != 4 or len(k) != 2:
        raise ValueError("philox4x64_10 needs a 4-word counter and a 2-word key")
    for r in range(10):
        c = _round(c, k)
        if r != 9:
            k = ((k[0] + PHILOX_W0) & MASK64, (k[1] + PHILOX_W1) & MASK64)
    return c


def word_to_uniform(w):
    """Top 24 bits of a 64-bit word as a float in [0, 1) (exact in fp32)."""
    return float((int(w) & MASK64) >> 40) * (2.0 ** -24)


def slot_uniforms(seed, seq_id, position, stream=STREAM_VERIFY):
    """(u_word0, u_word1) for one (seed, sequence, absolute position, stream)."""
    w = philox4x64_10((int(position) & MASK64, stream, 0, 0),
                      (int(seed) & MASK64, int(seq_id) & MASK64))
    return word_to_uniform(w[0]), word_to_uniform(w[1])


def noise_token(seed, seq_id, position, vocab):
    """A random_uniform noise token in [0, vocab): the top 24 bits of Philox word 0 at
    (seed, seq_id; position, stream 2, 0, 0) scaled by the vocabulary size with
    integer arithmetic, floor(w24 * vocab / 2^24)."""
    w = philox4x64_10((int(position) & MASK64, STREAM_NOISE, 0, 0),
                      (int(seed) & MASK64, int(seq_id) & MASK64))
    return ((int(w[0]) >> 40) * int(vocab)) >> 24
