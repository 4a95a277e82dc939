"""Pins for the oracle's checksum (CPU only).

The pages only say that the receiver checks the rebuilt weights against a
checksum of the trainer's weights ("Every byte counts: ARCv3 and the case for
cross-region RL", section "Deep dive into ARCv3").  The format defines it as
    checksum = mix64(S XOR n),
    S = sum over k of mix64(W_k XOR (k+1)G) mod 2^64,
where mix64 is the SplitMix64 finaliser and W_k packs elements 4k..4k+3.

What pins it:
- published SplitMix64 outputs, which fix mix64;
- the closed form for an all-zero tensor, which fixes the sum, the (k+1)G
  index term and the length term;
- recovering a planted element by inverting the checksum, which fixes how
  elements are packed into words;
- exhaustive single-bit flips, which must always change the value.
"""
import json
import os

import numpy as np
import pytest

import oracle

M64 = (1 << 64) - 1
G = 0x9E3779B97F4A7C15


def _published():
    with open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.json")) as f:
        return [int(v, 16) for v in json.load(f)["outputs"]]


def _inv_xorshift_right(y, s):
    x = y
    for _ in range(64 // s + 1):
        x = y ^ (x >> s)
    return x & M64


def _inv_mix64(z):
    """Inverse of the SplitMix64 finaliser, from its definition as a chain of
    bijections: undo each xor-shift by fixed-point iteration and each odd
    multiplier by its inverse modulo 2^64."""
    z = _inv_xorshift_right(z, 31)
    z = (z * pow(0x94D049BB133111EB, -1, 1 << 64)) & M64
    z = _inv_xorshift_right(z, 27)
    z = (z * pow(0xBF58476D1CE4E5B9, -1, 1 << 64)) & M64
    z = _inv_xorshift_right(z, 30)
    return z


def test_mix64_matches_published_splitmix64_outputs():
    for k, expected in enumerate(_published()):
        assert oracle.mix64(((k + 1) * G) & M64) == expected


def test_mix64_is_a_bijection():
    rng = np.random.default_rng(1)
    xs = [int(v) for v in rng.integers(0, 1 << 63, 2000, dtype=np.uint64)] + list(range(64))
    xs += [M64, 1 << 63, G]
    for x in xs:
        assert _inv_mix64(oracle.mix64(x)) == x


def test_checksum_of_zero_tensors_closed_form():
    outs = _published()
    assert oracle.checksum(np.zeros(0, np.uint16)) == 0        # mix64(0 ^ 0) = 0
    for n in range(1, 21):
        words = -(-n // 4)
        s = sum(outs[:words]) & M64
        assert oracle.checksum(np.zeros(n, np.uint16)) == oracle.mix64(s ^ n), n


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 13, 64])
def test_checksum_recovers_a_planted_element(n):
    """Plant v at index i of a zero tensor, then invert the checksum.  The
    result must be exactly the word that holds v in lane i mod 4."""
    outs_zero = [oracle.mix64(((k + 1) * G) & M64) for k in range(-(-n // 4))]
    rng = np.random.default_rng(n)
    for i in range(n):
        v = int(rng.integers(1, 1 << 16))
        w = np.zeros(n, np.uint16)
        w[i] = v
        s = _inv_mix64(oracle.checksum(w)) ^ n
        K = i // 4
        term = (s - (sum(outs_zero) - outs_zero[K])) & M64
        word = _inv_mix64(term) ^ (((K + 1) * G) & M64)
        assert word == v << (16 * (i % 4)), (n, i)


def test_every_single_bit_flip_changes_the_checksum():
    rng = np.random.default_rng(7)
    for n in (1, 5, 17, 64):
        w = rng.integers(0, 1 << 16, n, dtype=np.uint16)
        base = oracle.checksum(w)
        for i in range(n):
            for b in range(16):
                w2 = w.copy()
                w2[i] ^= np.uint16(1 << b)
                assert oracle.checksum(w2) != base


def test_checksum_covers_the_length():
    # trailing zero elements still change the value (n is mixed in)
    assert oracle.checksum(np.zeros(4, np.uint16)) != oracle.checksum(np.zeros(3, np.uint16))
    assert oracle.checksum(np.zeros(8, np.uint16)) != oracle.checksum(np.zeros(7, np.uint16))


def test_checksum_is_position_sensitive():
    w = np.zeros(16, np.uint16)
    w[0] = 1
    w2 = np.zeros(16, np.uint16)
    w2[4] = 1
    assert oracle.checksum(w) != oracle.checksum(w2)
