"""Pins for oracle.philox: published known answers and distribution checks."""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x32, seed_key


def test_known_answer_vectors(golden_dir):
    with open(os.path.join(golden_dir, "philox4x32_10_kat.json")) as fh:
        kat = json.load(fh)
    for vec in kat["vectors"]:
        ctr = [int(w, 16) for w in vec["ctr"]]
        key = [int(w, 16) for w in vec["key"]]
        out = [int(w) for w in philox4x32(ctr, key)]
        assert out == [int(w, 16) for w in vec["out"]]


def test_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(7)
    ctr = [rng.integers(0, 2 ** 32, 50, dtype=np.uint64) for _ in range(4)]
    key = (0x12345678, 0x9ABCDEF0)
    vec = philox4x32(ctr, key)
    for i in range(50):
        one = philox4x32([c[i] for c in ctr], key)
        assert [int(w[i]) for w in vec] == [int(w) for w in one]


def test_output_words_are_uniform():
    n = 1 << 15
    words = philox4x32((np.arange(n), 3, 11, 0), seed_key(0))
    for w in words:
        counts = np.bincount((w >> np.uint32(26)).astype(np.int64), minlength=64)
        assert stats.chisquare(counts).pvalue > 1e-4
        bits = ((w[:, None] >> np.arange(32, dtype=np.uint32)) & 1).mean(axis=0)
        assert np.all(np.abs(bits - 0.5) < 0.02)


def test_counter_and_key_sensitivity():
    base = philox4x32((1, 2, 3, 4), (5, 6))
    for i in range(4):
        ctr = [1, 2, 3, 4]
        ctr[i] ^= 1
        assert philox4x32(ctr, (5, 6)) != base
    assert philox4x32((1, 2, 3, 4), (5, 7)) != base


@pytest.mark.parametrize("seed,lo,hi", [(0, 0, 0), (1, 1, 0), (2 ** 32, 0, 1),
                                        (0x0123456789ABCDEF, 0x89ABCDEF, 0x01234567)])
def test_seed_key_split(seed, lo, hi):
    assert seed_key(seed) == (lo, hi)
