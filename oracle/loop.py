"""Oracle for the denoising-loop driver around the per-step sampler: the canvas length of a
block, the random initial canvas, and the per-step stability update that ends a block early.

Passages followed (pages named in the package docstring):

* Block-diffusion generation (DiffusionGemma), "How it works": the canvas of a block is
  drawn at random from the vocabulary with a seed, its length is min(max_canvas,
  max(remaining, min_canvas)), at most the step budget of steps run, and the block ends early
  once the canvas has stayed the same for stability_threshold steps in a row.
* same, "CLI flags": the minimum canvas (64) and the maximum canvas (the model's canvas
  length, 256 for the model described), the option to always use the full canvas, the step budget
  (typically 48).
* same, "Reproducibility": the seed fixes the canvas initialisation.

Readings taken where the pages are silent:

* initial id of position p of block b: Philox4x32-10 keyed by the 64-bit seed, counter
  (p, b, 0, 2), word 0, mapped to [0, vocab) as floor(word * vocab / 2^32);
* after each step the canvas holds every sampled position's draft token (the sampler
  itself writes only accepted positions; the driver then writes the drafts of the others),
  so the whole canvas is updated at every step, as the page describes; frozen positions
  keep their token;
* "unchanged" compares the whole canvas with the canvas before the step; the stable count
  is the number of consecutive unchanged steps;
* the block ends when the stable count reaches the threshold, when every position is
  frozen (nothing is left to decide), or when the step budget is spent.

Test infrastructure only.
"""

import numpy as np

from .philox import philox4x32, seed_key

# state words of the driver: steps run, consecutive unchanged steps, done flag, frozen count
STEP, STABLE, DONE, NFROZEN = range(4)


def canvas_length(max_canvas, min_canvas, remaining, full_canvas=False):
    """Tokens of the next block's canvas."""
    if full_canvas:
        return int(max_canvas)
    return int(min(max_canvas, max(remaining, min_canvas)))


def init_canvas(P, vocab, seed, block):
    """Random initial canvas int64 [P] of block ``block``."""
    p = np.arange(P, dtype=np.int64)
    w = philox4x32((p, block, 0, 2), seed_key(seed))[0].astype(np.uint64)
    return ((w * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def loop_update(tokens, canvas, prev_canvas, frozen, state, threshold, max_steps,
                write_drafts=True):
    """One step of the driver after the sampler.  Updates canvas, prev_canvas and state in place.

    tokens: the step's draft tokens (-1 where the row was not sampled: frozen before the step);
    canvas: after the sampler's own writes of accepted positions; frozen: after the step.
    A call on a finished block changes nothing.
    """
    if state[DONE]:
        return
    if write_drafts:
        sampled = tokens >= 0
        canvas[sampled] = tokens[sampled]
    changed = bool(np.any(canvas != prev_canvas))
    prev_canvas[:] = canvas
    state[STEP] += 1
    state[STABLE] = 0 if changed else state[STABLE] + 1
    state[NFROZEN] = int(np.count_nonzero(frozen))
    state[DONE] = int(state[STABLE] >= threshold or state[NFROZEN] == len(canvas)
                      or state[STEP] >= max_steps)
