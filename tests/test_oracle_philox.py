"""Pins of the oracle's Philox-4x64-10 against numpy's implementation of the same generator."""
import numpy as np
import pytest

from oracle.philox import MASK64, philox4x64_10, slot_uniforms, word_to_uniform


def _numpy_block(counter, key):
    # numpy's Philox adds one to the 256-bit counter before each encryption, so the
    # block for counter C is the first output of a generator started at C - 1.
    c = [int(x) & MASK64 for x in counter]
    v = (c[0] | (c[1] << 64) | (c[2] << 128) | (c[3] << 192)) - 1
    v &= (1 << 256) - 1
    cm1 = np.array([(v >> (64 * i)) & MASK64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(counter=cm1, key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in g.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((5, 1, 0, 0), (123, 7)),
    ((MASK64, MASK64, MASK64, MASK64), (MASK64, MASK64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_matches_numpy(counter, key):
    assert philox4x64_10(counter, key) == _numpy_block(counter, key)


def test_philox_random_keys_match_numpy():
    rng = np.random.default_rng(1)
    for _ in range(200):
        key = tuple(int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.uint64))
        ctr = (int(rng.integers(0, 2**40)), int(rng.integers(0, 2)), 0, 0)
        assert philox4x64_10(ctr, key) == _numpy_block(ctr, key)


def test_uniform_is_24_bit_and_in_range():
    assert word_to_uniform(0) == 0.0
    top = word_to_uniform(MASK64)
    assert top == 1.0 - 2.0 ** -24 and top < 1.0
    for w in (1 << 40, (1 << 41) + 12345, 0xDEADBEEF << 30):
        u = word_to_uniform(w)
        assert u * 2**24 == float(w >> 40)
        assert np.float32(u) == u  # exact in fp32


def test_streams_are_distinct():
    a = slot_uniforms(0, 3, 10, stream=0)
    b = slot_uniforms(0, 3, 10, stream=1)
    assert a != b
    assert slot_uniforms(0, 3, 10, 0) == a  # deterministic
