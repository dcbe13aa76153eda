"""Pins of the denoising-loop driver oracle (oracle/loop.py); no GPU."""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import loop
from oracle.philox import philox4x32, seed_key


OPTIONS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "diffusion_options.json")))


@pytest.mark.parametrize("remaining,expect", [(0, 64), (12, 64), (64, 64), (65, 65), (200, 200),
                                              (256, 256), (257, 256), (10000, 256)])
def test_canvas_length_with_the_documented_defaults(remaining, expect):
    # the page's defaults: minimum canvas 64, maximum (the model's canvas) typically 256
    lo, hi = OPTIONS["min_canvas_default"], OPTIONS["max_canvas_typical"]
    assert (lo, hi) == (64, 256)
    assert loop.canvas_length(hi, lo, remaining) == expect
    assert loop.canvas_length(hi, lo, remaining, full_canvas=True) == hi


def test_init_canvas_mapping_edges_and_range():
    # the mapping floor(w * vocab / 2^32) on its extreme words
    for vocab in (1, 2, 262144, 1 << 24):
        assert (0 * vocab) >> 32 == 0
        assert ((2 ** 32 - 1) * vocab) >> 32 == vocab - 1
    c = loop.init_canvas(4096, 262144, seed=5, block=3)
    assert c.min() >= 0 and c.max() < 262144
    w = philox4x32((np.arange(4096), 3, 0, 2), seed_key(5))[0]
    assert np.array_equal(c, (w.astype(np.uint64) * np.uint64(262144)) >> np.uint64(32))


def test_init_canvas_is_uniform_and_seeded():
    V = 16
    c = loop.init_canvas(64000, V, seed=11, block=0)
    counts = np.bincount(c, minlength=V)
    assert stats.chisquare(counts).pvalue > 1e-4
    assert np.array_equal(c, loop.init_canvas(64000, V, seed=11, block=0))
    assert not np.array_equal(c[:100], loop.init_canvas(100, V, seed=11, block=1))
    assert not np.array_equal(c[:100], loop.init_canvas(100, V, seed=12, block=0))


def fresh(P, init):
    canvas = np.array(init, dtype=np.int64)
    return canvas, canvas.copy(), np.zeros(P, dtype=np.uint8), np.zeros(4, dtype=np.int64)


def test_stable_drafts_end_the_block_after_threshold_steps():
    P, thr = 6, 3
    canvas, prev, frozen, st = fresh(P, [9, 9, 9, 9, 9, 9])
    drafts = np.array([1, 2, 3, 4, 5, 6])
    for step in range(1, 10):
        frozen[step - 1] = 1 if step - 1 < P else 0     # one accept per step
        canvas[step - 1] = drafts[step - 1]            # the sampler's own write
        tok = np.where(frozen == 1, drafts, drafts)    # drafts identical every step
        loop.loop_update(tok, canvas, prev, frozen, st, thr, 48)
        if st[loop.DONE]:
            break
    # step 1 changes the canvas (random -> drafts); steps 2, 3, 4 are unchanged -> done at 4
    assert st[loop.STEP] == 4 and st[loop.STABLE] == 3 and st[loop.NFROZEN] == 4
    before = canvas.copy()
    loop.loop_update(np.zeros(P, dtype=np.int64), canvas, prev, frozen, st, thr, 48)
    assert st[loop.STEP] == 4 and np.array_equal(canvas, before)   # finished: no-op


def test_changing_drafts_reset_the_count_and_all_frozen_ends_the_block():
    P = 3
    canvas, prev, frozen, st = fresh(P, [0, 0, 0])
    seq = [[1, 1, 1], [1, 1, 1], [1, 2, 1], [1, 2, 1]]
    expect_stable = [1 - 1, 1, 0, 1]   # first step: canvas 0 -> 1 changes
    for tok, es in zip(seq, expect_stable):
        loop.loop_update(np.array(tok), canvas, prev, frozen, st, 5, 48)
        assert st[loop.STABLE] == es and not st[loop.DONE]
    frozen[:] = 1
    loop.loop_update(np.array([-1, -1, -1]), canvas, prev, frozen, st, 5, 48)
    assert st[loop.DONE] and st[loop.NFROZEN] == 3 and list(canvas) == [1, 2, 1]


def test_step_budget_ends_the_block_and_frozen_rows_keep_their_token():
    P = 4
    canvas, prev, frozen, st = fresh(P, [5, 6, 7, 8])
    frozen[1] = 1
    for s in range(3):
        loop.loop_update(np.array([s, -1, s + 10, s + 20]), canvas, prev, frozen, st, 10, 3)
    assert st[loop.DONE] and st[loop.STEP] == 3 and canvas[1] == 6
    canvas, prev, frozen, st = fresh(P, [5, 6, 7, 8])
    loop.loop_update(np.array([1, 2, 3, 4]), canvas, prev, frozen, st, 10, 48, write_drafts=False)
    assert list(canvas) == [5, 6, 7, 8] and st[loop.STABLE] == 1
