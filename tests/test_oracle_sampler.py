"""Pins for oracle.sampler: closed forms, library routines, distribution tests and
exact-arithmetic checks of the acceptance rule."""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import special, stats

from oracle import sampler
from oracle.philox import philox4x32


# ---------------------------------------------------------------- entropy

def test_entropy_uniform_row():
    for V in (1, 2, 7, 4096):
        assert abs(sampler.entropy(np.full(V, 0.3, dtype=np.float32)) - math.log(V)) < 1e-12


@pytest.mark.parametrize("n,V,a,b", [(1, 4096, 12.0, 0.0), (3, 100, 2.0, -1.0), (50, 60, 0.0, 5.0),
                                     (1, 262144, 26.0, 0.0)])
def test_entropy_two_level_closed_form(n, V, a, b):
    x = np.full(V, b, dtype=np.float32)
    x[:n] = a
    za, zb = math.exp(a - max(a, b)), math.exp(b - max(a, b))
    Z = n * za + (V - n) * zb
    pa, pb = za / Z, zb / Z
    H = -(n * pa * math.log(pa) + (V - n) * pb * math.log(pb))
    assert abs(sampler.entropy(x) - H) <= 1e-10 * max(H, 1e-300) + 1e-15


def test_entropy_matches_scipy_and_is_shift_invariant():
    rng = np.random.default_rng(1)
    for scale in (0.1, 1.0, 4.0):
        x = (rng.standard_normal(3000) * scale).astype(np.float32)
        ref = stats.entropy(special.softmax(x.astype(np.float64)))
        h = sampler.entropy(x)
        assert abs(h - ref) < 1e-10
        assert 0.0 <= h <= math.log(x.size)
        assert abs(sampler.entropy(x + np.float32(37.0)) - h) < 1e-5


def test_entropy_ignores_minus_inf_and_flags_invalid_rows():
    assert abs(sampler.entropy(np.array([0, -np.inf, 0], dtype=np.float32)) - math.log(2)) < 1e-15
    assert sampler.entropy(np.array([-np.inf, 5.0], dtype=np.float32)) == 0.0
    for bad in ([0.0, np.nan], [np.inf, 0.0], [-np.inf, -np.inf]):
        assert math.isnan(sampler.entropy(np.array(bad, dtype=np.float32)))


# ---------------------------------------------------------------- noise

def test_uniform24_endpoints_and_exactness():
    u = sampler.uniform24(np.array([0, 255, 256, 0xFFFFFFFF], dtype=np.uint32))
    assert u.tolist() == [2.0 ** -25, 2.0 ** -25, 3 * 2.0 ** -25, 1 - 2.0 ** -25]
    # every value is an odd multiple of 2^-25: exact in float64, distinct per r >> 8
    assert np.all(np.mod(u * 2.0 ** 25, 2.0) == 1.0)


def test_gumbel_noise_distribution():
    g = sampler.entry_noise(3, np.arange(40000), seed=9, step=2)
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-3
    assert abs(g.mean() - np.euler_gamma) < 0.03


def test_noise_counter_layout():
    # entry v uses counter (v >> 2, row, step, 0), word v & 3; chunk c uses (c, row, step, 1) word 0
    words = philox4x32((5, 7, 3, 0), (42, 0))
    for j in range(4):
        assert sampler.entry_noise(7, np.array([20 + j]), 42, 3)[0] == sampler.gumbel(
            sampler.uniform24(np.array([words[j]])))[0]
    cw = philox4x32((5, 7, 3, 1), (42, 0))
    assert sampler.chunk_noise(7, np.array([5]), 42, 3)[0] == sampler.gumbel(
        sampler.uniform24(np.array([cw[0]])))[0]


# ---------------------------------------------------------------- token draw

def test_temperature_zero_is_first_argmax():
    x = np.array([1.0, 4.0, -2.0, 4.0], dtype=np.float32)
    assert sampler.draw_token(x, 0.0, 0, 0, 0)[0] == 1


def test_single_chunk_is_flat_gumbel_max():
    rng = np.random.default_rng(4)
    for step in range(20):
        x = rng.standard_normal(1000).astype(np.float32)
        g = sampler.entry_noise(2, np.arange(1000), 77, step)
        assert sampler.draw_token(x, 1.0, 77, step, 2)[0] == int(np.argmax(x / 1.0 + g))
        assert sampler.draw_token(x, 0.5, 77, step, 2)[0] == int(np.argmax(x.astype(np.float64) / 0.5 + g))


@pytest.mark.parametrize("temperature", [1.0, 0.6, 2.0])
def test_two_level_draw_follows_softmax(temperature):
    # 6 live entries spread over 3 chunks, the rest masked with -inf.
    V = 2600
    x = np.full(V, -np.inf, dtype=np.float32)
    live = np.array([3, 1000, 1030, 1500, 2100, 2599])
    x[live] = np.array([0.0, 1.0, -0.5, 0.3, 1.2, -1.0], dtype=np.float32)
    p = special.softmax(x[live].astype(np.float64) / temperature)
    n = 3000
    counts = np.zeros(6)
    for s in range(n):
        tok = sampler.draw_token(x, temperature, 1234, s, 0)[0]
        counts[np.searchsorted(live, tok)] += 1
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_two_level_chunk_frequencies_follow_chunk_mass():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(3000).astype(np.float32)
    x[2500] += 3.0
    mass = np.array([np.exp(x[c * 1024:(c + 1) * 1024].astype(np.float64)).sum() for c in range(3)])
    n = 2000
    counts = np.zeros(3)
    for s in range(n):
        counts[sampler.draw_token(x, 1.0, 5, s, 1)[0] // 1024] += 1
    assert stats.chisquare(counts, mass / mass.sum() * n).pvalue > 1e-4


def test_sample_rows_frozen_and_invalid():
    x = np.zeros((3, 8), dtype=np.float32)
    x[1, 2] = np.nan
    H, tok = sampler.sample_rows(x, 1.0, 0, 0, frozen=np.array([1, 0, 0], dtype=np.uint8))
    assert H[0] == np.inf and tok[0] == -1
    assert math.isnan(H[1]) and tok[1] == -1
    assert abs(H[2] - math.log(8)) < 1e-12 and 0 <= tok[2] < 8


# ---------------------------------------------------------------- acceptance

def _exact_accept_count(h_sorted, bound):
    """Exact arithmetic: position i passes iff sum_{j<i} H_j <= bound; stop at the first failure."""
    n, acc = 0, Fraction(0)
    for h in h_sorted:
        if acc > Fraction(bound):
            break
        n += 1
        acc += Fraction(h)
    return max(n, 1) if h_sorted else 0


def test_accept_exact_on_dyadic_entropies():
    # Multiples of 1/64 below 64: every float32 sum and difference here is exact,
    # so the float32 rule must agree with exact rational arithmetic.
    rng = np.random.default_rng(0)
    for _ in range(300):
        P = int(rng.integers(1, 40))
        H = (rng.integers(0, 256, P) / 64.0).astype(np.float32)
        frozen = rng.random(P) < 0.2
        bound = float(rng.integers(-8, 400)) / 64.0
        mask, n = sampler.accept(H, bound, frozen)
        cand = sorted((float(H[p]), p) for p in range(P) if not frozen[p])
        k = _exact_accept_count([h for h, _ in cand], bound)
        assert n == k == int(mask.sum())
        assert sorted(np.nonzero(mask)[0].tolist()) == sorted(p for _, p in cand[:k])


def test_accept_brute_force_all_orderings():
    H = np.array([0.5, 0.25, 0.25, 1.0, 0.125, 2.0], dtype=np.float32)
    for perm in itertools.permutations(range(6)):
        Hp = H[list(perm)]
        mask, n = sampler.accept(Hp, 0.75)
        # sorted: .125 .25 .25 .5 1 2 -> exclusive sums 0 .125 .375 .625 1.125 -> 4 pass
        assert n == 4
        assert sorted(Hp[mask == 1].tolist()) == [0.125, 0.25, 0.25, 0.5]
        # ties at 0.25: both accepted here, so the position tie-break is not visible


def test_accept_tie_break_by_position():
    H = np.array([1.0, 0.5, 0.5, 0.5], dtype=np.float32)
    mask, n = sampler.accept(H, 0.5)       # exclusive sums 0, .5, 1.0 -> two pass
    assert n == 2 and mask.tolist() == [0, 1, 1, 0]


def test_accept_special_bounds_and_nan():
    H = np.array([3.0, 1.0, np.nan, 2.0], dtype=np.float32)
    assert sampler.accept(H, np.inf)[1] == 3
    mask, n = sampler.accept(H, -1.0)
    assert n == 1 and mask.tolist() == [0, 1, 0, 0]
    assert sampler.accept(H, 0.0, frozen=np.array([1, 1, 0, 1]))[1] == 0
    assert sampler.accept(np.zeros(0, dtype=np.float32), 1.0)[1] == 0


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(0, 20, width=32), min_size=1, max_size=24),
       st.floats(-1, 30), st.lists(st.booleans(), min_size=24, max_size=24))
def test_accept_invariants(hs, bound, fro):
    H = np.array(hs, dtype=np.float32)
    P = H.size
    frozen = np.array(fro[:P])
    mask, n = sampler.accept(H, bound, frozen)
    cand = sorted((float(H[p]), p) for p in range(P) if not frozen[p])
    assert (n >= 1) == bool(cand)
    assert not np.any(mask[frozen])
    assert sorted(np.nonzero(mask)[0].tolist()) == sorted(p for _, p in cand[:n])
    assert n <= sampler.accept(H, bound + 1.0, frozen)[1]


# ---------------------------------------------------------------- confidence-threshold

def test_confidence_uniform_row():
    for V in (1, 2, 7, 4096):
        assert abs(sampler.confidence(np.full(V, -1.5, dtype=np.float32)) - 1.0 / V) < 1e-15


@pytest.mark.parametrize("n,V,a,b", [(1, 4096, 12.0, 0.0), (3, 100, 2.0, -1.0), (2, 2, 0.5, 0.5),
                                     (1, 262144, 26.0, 0.0)])
def test_confidence_two_level_closed_form(n, V, a, b):
    x = np.full(V, b, dtype=np.float32)
    x[:n] = a
    top = max(a, b)
    Z = n * math.exp(a - top) + (V - n) * math.exp(b - top)
    assert abs(sampler.confidence(x) - 1.0 / Z) <= 1e-12 / Z


def test_confidence_is_softmax_max_and_bounds_entropy():
    """The library softmax's largest entry; and since the min-entropy -ln p_max never exceeds
    the entropy, exp(-H) <= p_max <= 1, with p_max >= 1/V."""
    rng = np.random.default_rng(7)
    for scale in (0.1, 1.0, 6.0):
        x = (rng.standard_normal(5000) * scale).astype(np.float32)
        c = sampler.confidence(x)
        assert abs(c - special.softmax(x.astype(np.float64)).max()) < 1e-14
        assert math.exp(-sampler.entropy(x)) <= c * (1 + 1e-12) and c <= 1.0
        assert c >= 1.0 / x.size


def test_confidence_minus_inf_invalid_and_frozen():
    assert sampler.confidence(np.array([-np.inf, 3.0], dtype=np.float32)) == 1.0
    assert abs(sampler.confidence(np.array([0, -np.inf, 0], dtype=np.float32)) - 0.5) < 1e-15
    for bad in ([0.0, np.nan], [np.inf, 0.0], [-np.inf, -np.inf]):
        assert math.isnan(sampler.confidence(np.array(bad, dtype=np.float32)))
    logits = np.zeros((3, 8), dtype=np.float32)
    logits[2, 0] = np.nan
    c = sampler.confidence_rows(logits, frozen=np.array([0, 1, 0], dtype=np.uint8))
    assert c[0] == 0.125 and c[1] == -1.0 and math.isnan(c[2])


def _accept_by_sorting(c, thr, frozen):
    """The page's rule, written another way: candidates above the threshold, else the head
    of the candidates ordered by descending confidence then ascending position."""
    cand = [p for p in range(len(c)) if not frozen[p] and c[p] == c[p] and c[p] >= 0]
    above = [p for p in cand if c[p] > np.float32(thr)]
    if above:
        return set(above)
    if not cand:
        return set()
    return {sorted(cand, key=lambda p: (-float(c[p]), p))[0]}


def test_accept_confidence_brute_force():
    values = np.array([0.0, 0.25, 0.5, 0.9, np.float32(0.9) + np.float32(1e-7), 1.0, np.nan, -1.0],
                      dtype=np.float32)
    rng = np.random.default_rng(3)
    for P in range(1, 6):
        for _ in range(300):
            c = values[rng.integers(0, values.size, P)]
            frozen = rng.integers(0, 2, P).astype(np.uint8) if rng.random() < 0.5 else np.zeros(P, np.uint8)
            thr = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
            mask, n = sampler.accept_confidence(c, thr, frozen)
            want = _accept_by_sorting(c, thr, frozen)
            assert set(np.nonzero(mask)[0].tolist()) == want and n == len(want)


def test_accept_confidence_edges():
    c = np.array([0.9, 0.3, 0.95, 0.95], dtype=np.float32)
    mask, n = sampler.accept_confidence(c, 0.9)
    assert mask.tolist() == [0, 0, 1, 1] and n == 2            # equal to the threshold: not above
    mask, n = sampler.accept_confidence(c, 1.0)
    assert mask.tolist() == [0, 0, 1, 0] and n == 1            # fallback: first of the tied maxima
    mask, n = sampler.accept_confidence(c, 0.5, frozen=np.array([0, 0, 1, 1]))
    assert mask.tolist() == [1, 0, 0, 0] and n == 1            # frozen never accepted
    mask, n = sampler.accept_confidence(c, 0.5, frozen=np.ones(4))
    assert n == 0 and mask.sum() == 0                          # nothing to accept
    mask, n = sampler.accept_confidence(np.array([np.nan, -1.0, 0.1], dtype=np.float32), 0.9)
    assert mask.tolist() == [0, 0, 1] and n == 1               # NaN and frozen markers skipped
