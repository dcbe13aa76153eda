"""Pins of the RMS-norm and router oracle (oracle/layer.py) against closed forms, scalar
brute force and invariants; no GPU."""

import math

import numpy as np
import pytest

from oracle import layer


def brute_rmsnorm(h, w, eps):
    out = []
    for row in h:
        vals = [float(v) for v in row]
        ms = sum(v * v for v in vals) / len(vals)
        r = 1.0 / math.sqrt(ms + eps)
        out.append([v * r * float(wi) for v, wi in zip(vals, w)])
    return np.array(out)


def test_rmsnorm_matches_scalar_loops():
    rng = np.random.default_rng(0)
    h = (rng.standard_normal((5, 24)) * 2).astype(np.float16)
    w = (1 + 0.2 * rng.standard_normal(24)).astype(np.float16)
    got = layer.rmsnorm(h, w, 1e-6)
    ref = brute_rmsnorm(h.astype(np.float64), w.astype(np.float64), 1e-6)
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


def test_rmsnorm_constant_row_closed_form():
    d, c, eps = 64, 2.5, 1e-6
    h = np.full((1, d), c, dtype=np.float16)
    w = np.full(d, 0.75, dtype=np.float16)
    got = layer.rmsnorm(h, w, eps)
    assert np.allclose(got, c / math.sqrt(c * c + eps) * 0.75, rtol=1e-15)


def test_rmsnorm_unit_rms_and_eps_effect():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((7, 256)).astype(np.float16)
    w = np.ones(256, dtype=np.float16)
    for eps in (0.0, 1e-6, 0.5):
        y = layer.rmsnorm(h, w, eps)
        ms = np.mean(h.astype(np.float64) ** 2, axis=1)
        # mean(y^2) = ms / (ms + eps) exactly
        assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13)


def test_rmsnorm_scale_invariance_and_weight_linearity():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((3, 128)).astype(np.float16)
    w = (1 + 0.1 * rng.standard_normal(128)).astype(np.float16)
    y = layer.rmsnorm(h, w, 0.0)
    y4 = layer.rmsnorm((h.astype(np.float32) * 4).astype(np.float16), w, 0.0)  # exact x4
    assert np.allclose(y, y4, rtol=1e-14)
    y1 = layer.rmsnorm(h, np.ones(128, dtype=np.float16), 0.0)
    assert np.allclose(y, y1 * w.astype(np.float64)[None, :], rtol=1e-15)


def test_rmsnorm_zero_row():
    h = np.zeros((2, 64), dtype=np.float16)
    assert np.all(layer.rmsnorm(h, np.ones(64, dtype=np.float16)) == 0.0)


def test_router_matches_scalar_loops():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 32))
    W = rng.standard_normal((6, 32)).astype(np.float16)
    got = layer.router_logits(x, W)
    for t in range(4):
        for e in range(6):
            ref = sum(float(x[t, i]) * float(W[e, i]) for i in range(32))
            assert abs(got[t, e] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_router_one_hot_picks_a_column():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((5, 16)).astype(np.float16)
    x = np.zeros((1, 16))
    x[0, 9] = 1.0
    assert np.array_equal(layer.router_logits(x, W)[0], W[:, 9].astype(np.float64))


def test_router_not_transposed():
    # a non-square case where a transposed operand cannot even broadcast
    W = np.arange(12, dtype=np.float16).reshape(3, 4)
    x = np.array([[1.0, 0.0, 0.0, 2.0]])
    assert np.array_equal(layer.router_logits(x, W), [[6.0, 18.0, 30.0]])


@pytest.mark.parametrize("d", [256, 2816])
def test_workload_logits_are_about_unit_normal(d):
    from block_diffusion_lm_router_amd import workloads
    shape = workloads.LAYER if d == 2816 else workloads.TINY_LAYER
    h, wn, wr = workloads.make_norm_router(shape)
    logits = layer.router_logits(layer.rmsnorm(h, wn), wr)
    assert logits.shape == (shape.tokens, shape.experts)
    assert 0.8 < logits.std() < 1.2 and abs(logits.mean()) < 0.1
