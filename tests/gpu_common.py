"""Helpers shared by the GPU parity tests (no test functions here)."""

import sys

import numpy as np
import pytest

from conftest import gpu_available

requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")

# Tolerances.  FFN outputs: |y - y_ref| <= ABS + REL |y_ref| (allclose form, fp16 outputs).
FFN_ABS, FFN_REL = 2e-2, 1e-2
# Entropy: relative 1e-4.
H_REL = 1e-4
# Top-1 probability 1 / Z: Z is an fp32 sum of positive terms over at most ~50 sequential
# additions (per lane, per wave, per block, per split), each term an fp32 exp2 of an argument
# with at most ~3.6e-6 absolute rounding; the bound on |dZ| / Z is below 5e-6.
C_REL = 1e-5
# Token decisions at T > 0 are taken in fp64 on both sides (the GPU rescores in fp64 every
# chunk and every entry its fp32 pre-selection cannot rule out), so a mismatch is excused
# only when the oracle's own fp64 decision margin is at the level where two fp64 evaluations
# of the same definition (different exp/log implementations and summation orders) may differ.
L1_MARGIN = 1e-12
L2_MARGIN = 1e-12


def say(*args):
    """Name the case before each GPU step, flushed, so a crash log identifies it."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def top2_margin(v):
    v = np.asarray(v, dtype=np.float64)
    v = v[np.isfinite(v)]
    if v.size < 2:
        return np.inf
    part = np.partition(v, -2)
    return float(part[-1] - part[-2])


def check_ffn_close(y, ref, what, extra=0.0):
    """|y - ref| <= 2e-2 + 1e-2 |ref| (+ extra: a derived rounding bound a weight form adds)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(y - ref)
    bound = FFN_ABS + FFN_REL * np.abs(ref) + extra
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside 2e-2 + 1e-2|ref|; "
                           f"max err {err.max():.4g}, worst ratio {(err / bound).max():.3g}")
    return float(np.sqrt(np.mean((y - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
