"""Oracle for the per-step sampler: entropy, token draw and entropy-bound acceptance.

Passages followed (pages named in the package docstring):

* axe-diffusion-ksl-xe model card, "what the model is": a 256-token canvas is
  denoised over up to 48 steps and tokens are committed once their entropy is
  under a bound.
* same, "the kernels we built": entropy once per step in one streaming pass, and
  one gumbel-max kernel in place of softmax + multinomial, over fp32 logits.
* DiffusionGemma block-diffusion page, "Samplers", entropy-bound: per-position
  entropy, positions sorted by ascending entropy, accepted while
  (cumsum - cummax) <= bound, at least one position always accepted.
* same page, "Samplers", confidence-threshold: every unrevealed position whose
  top-1 token probability is above the threshold (flag default 0.9, validated to
  [0, 1]) is accepted; when none is, the single most confident unrevealed position
  is accepted so that every step makes progress.

Readings taken where the pages are silent or loose:

* The entropy is that of softmax(x) at temperature 1 whatever the sampling
  temperature (else temperature 0 would give zero entropy everywhere).
* Temperature 0 takes the argmax, the lowest index on ties.
* Temperature T > 0 draws token ~ softmax(x / T) by gumbel-max applied on two
  levels.  The row is cut into chunks of CHUNK = 1024 consecutive entries.
  Level 1 picks the chunk c* maximising L_c + G_c, where L_c is the log-mass
  log sum_{v in c} exp(x_v / T) and G_c a Gumbel(0, 1) draw per chunk.  Level 2
  picks, inside chunk c*, the entry maximising x_v / T + g_v, with g_v a
  Gumbel(0, 1) draw per entry.  By the Gumbel-max property applied twice,
  P(token = v) = (Z_c / Z) * (exp(x_v / T) / Z_c) = softmax(x / T)_v: the same
  distribution as one flat gumbel-max, and the same draw when the row fits in
  one chunk.  Ties go to the lower chunk, then the lower index.
* Noise: Philox4x32-10 keyed by the 64-bit seed (low word, high word).  Entry v
  of row p at step s uses counter (v >> 2, p, s, 0), word v & 3; chunk c uses
  counter (c, p, s, 1), word 0.  A word r becomes u = ((r >> 8) + 0.5) * 2^-24,
  strictly inside (0, 1) and exact in float64 (not in float32: near 1 it needs
  25 significant bits); g = -ln(-ln u), evaluated in float64.
* A row whose logits contain NaN or +inf, or are all -inf, has no defined
  distribution: entropy NaN, token -1, never accepted.
* Frozen (already committed) positions are not sampled (token -1, entropy +inf)
  and not candidates.
* Acceptance runs in float32 on the entropies it is given, sequentially in
  sorted order (ascending entropy, then ascending position): S <- S + H_i,
  c <- S - H_i, accept while c <= bound.  cummax in ascending order is H_i
  itself.  If no candidate passes and candidates exist, the first is accepted.
  Candidates are the unfrozen positions whose entropy is not NaN.
* The confidence of a position is the largest probability of softmax(x) at
  temperature 1 (the same distribution as the entropy), 1 / sum_v exp(x_v - max x)
  in float64; NaN for an invalid row, -1 for a frozen position.  "Above the
  threshold" is strict (c > threshold), compared in float32 on the confidences
  given.  Candidates are the unfrozen positions with a confidence that is not NaN
  and not negative; the fallback takes the largest confidence, the lowest position
  on ties, and accepts nothing when there is no candidate.

Everything except the acceptance scan and the 24-bit uniforms is float64.
Test infrastructure only.
"""

import numpy as np

from .philox import philox4x32, seed_key

CHUNK = 1024


def uniform24(words):
    """Map uint32 words to u = ((r >> 8) + 0.5) * 2^-24 (float64, exact, in (0, 1))."""
    r = np.asarray(words, dtype=np.uint32) >> np.uint32(8)
    return (r.astype(np.float64) + 0.5) * 2.0 ** -24


def gumbel(u):
    """Standard Gumbel draw from a uniform in (0, 1): g = -ln(-ln u)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))


def entry_noise(row, v, seed, step):
    """Gumbel noise g_v of entries ``v`` (int array) of ``row`` at ``step``."""
    v = np.asarray(v, dtype=np.int64)
    words = philox4x32((v >> 2, row, step, 0), seed_key(seed))
    stacked = np.stack(words, axis=0)
    pick = np.take_along_axis(stacked, (v & 3)[None, ...], axis=0)[0]
    return gumbel(uniform24(pick))


def chunk_noise(row, c, seed, step):
    """Gumbel noise G_c of chunks ``c`` (int array) of ``row`` at ``step``."""
    words = philox4x32((np.asarray(c, dtype=np.int64), row, step, 1), seed_key(seed))
    return gumbel(uniform24(words[0]))


def row_is_valid(x):
    """A row defines a distribution: no NaN, no +inf, at least one finite entry."""
    x = np.asarray(x, dtype=np.float64)
    return not (np.isnan(x).any() or np.isposinf(x).any() or np.isneginf(x).all())


def entropy(x):
    """H = -sum_v p_v ln p_v with p = softmax(x), in float64 (NaN if invalid).

    Entries at -inf have p = 0 and contribute nothing (the limit p ln p -> 0).
    """
    x = np.asarray(x, dtype=np.float64)
    if not row_is_valid(x):
        return np.nan
    fin = x[np.isfinite(x)]
    m = fin.max()
    z = np.exp(fin - m).sum()
    logp = (fin - m) - np.log(z)
    p = np.exp(logp)
    return float(-(p * logp).sum())


def confidence(x):
    """Top-1 probability max_v softmax(x)_v = 1 / sum_v exp(x_v - max x), in float64
    (NaN if the row is invalid).  Entries at -inf contribute exp(-inf) = 0."""
    x = np.asarray(x, dtype=np.float64)
    if not row_is_valid(x):
        return np.nan
    fin = x[np.isfinite(x)]
    return float(1.0 / np.exp(fin - fin.max()).sum())


def confidence_rows(logits, frozen=None):
    """Confidence of every row of ``logits`` [P, V]: -1 for frozen rows, NaN for invalid."""
    logits = np.asarray(logits, dtype=np.float32)
    out = np.empty(logits.shape[0])
    for p in range(logits.shape[0]):
        out[p] = -1.0 if (frozen is not None and frozen[p]) else confidence(logits[p])
    return out


def chunk_logmass(x, temperature):
    """L_c = ln sum_{v in chunk c} exp(x_v / T) for every chunk (-inf if empty)."""
    x = np.asarray(x, dtype=np.float64) / float(np.float32(temperature))
    n_chunks = -(-x.size // CHUNK)
    out = np.full(n_chunks, -np.inf)
    for c in range(n_chunks):
        seg = x[c * CHUNK:(c + 1) * CHUNK]
        fin = seg[np.isfinite(seg)]
        if fin.size:
            m = fin.max()
            out[c] = m + np.log(np.exp(fin - m).sum())
    return out


def draw_token(x, temperature, seed, step, row):
    """Token of one valid row.  Returns (token, level1_keys, level2_scores).

    ``level1_keys`` (float64 per chunk, or None at T = 0) and ``level2_scores``
    (float64 per entry of the winning chunk, or None) let tests measure how close
    a decision was.
    """
    x = np.asarray(x, dtype=np.float32)
    if float(temperature) == 0.0:
        return int(np.argmax(x)), None, None      # np.argmax: first maximal index
    t32 = float(np.float32(temperature))
    keys = chunk_logmass(x, t32) + chunk_noise(row, np.arange(-(-x.size // CHUNK)), seed, step)
    c_star = int(np.argmax(keys))                  # first maximal chunk
    v = np.arange(c_star * CHUNK, min((c_star + 1) * CHUNK, x.size))
    scores = x[v].astype(np.float64) / t32 + entry_noise(row, v, seed, step)
    return int(v[np.argmax(scores)]), keys, scores


def sample_rows(logits, temperature, seed, step, frozen=None, rows=None):
    """Entropy and token for every (or the listed) row of ``logits`` [P, V].

    Returns (entropy float64 [P], tokens int64 [P]); rows not listed are NaN / -2.
    """
    logits = np.asarray(logits, dtype=np.float32)
    P = logits.shape[0]
    H = np.full(P, np.nan)
    tok = np.full(P, -2, dtype=np.int64)
    for p in (range(P) if rows is None else rows):
        if frozen is not None and frozen[p]:
            H[p], tok[p] = np.inf, -1
            continue
        H[p] = entropy(logits[p])
        tok[p] = draw_token(logits[p], temperature, seed, step, p)[0] if np.isfinite(H[p]) else -1
    return H, tok


def accept(entropy32, bound, frozen=None):
    """Entropy-bound acceptance on float32 entropies.  Returns (mask uint8 [P], count)."""
    H = np.asarray(entropy32, dtype=np.float32)
    P = H.shape[0]
    frozen = np.zeros(P, dtype=bool) if frozen is None else np.asarray(frozen, dtype=bool)
    cand = [p for p in range(P) if not frozen[p] and not np.isnan(H[p])]
    order = sorted(cand, key=lambda p: (float(H[p]), p))
    b = np.float32(bound)
    mask = np.zeros(P, dtype=np.uint8)
    s = np.float32(0.0)
    n = 0
    for p in order:
        s = np.float32(s + H[p])
        c = np.float32(s - H[p])
        if not c <= b:
            break
        mask[p] = 1
        n += 1
    if n == 0 and order:
        mask[order[0]] = 1
        n = 1
    return mask, n


def accept_confidence(conf32, threshold, frozen=None):
    """Confidence-threshold acceptance on float32 confidences.  Returns (mask uint8 [P], count).

    Accepted: every candidate with c > threshold; if there is none, the candidate with the
    largest c (lowest position on ties).  Candidates: unfrozen, c not NaN, c >= 0.
    """
    c = np.asarray(conf32, dtype=np.float32)
    P = c.shape[0]
    frozen = np.zeros(P, dtype=bool) if frozen is None else np.asarray(frozen, dtype=bool)
    thr = np.float32(threshold)
    cand = [p for p in range(P) if not frozen[p] and not np.isnan(c[p]) and c[p] >= 0]
    mask = np.zeros(P, dtype=np.uint8)
    for p in cand:
        if c[p] > thr:
            mask[p] = 1
    n = int(mask.sum())
    if n == 0 and cand:
        best = cand[0]
        for p in cand[1:]:
            if c[p] > c[best]:
                best = p
        mask[best] = 1
        n = 1
    return mask, n
