"""Seeded synthetic inputs for the denoising-step hot path.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may consume what it
makes.  All draws use numpy's PCG64 with fixed seeds, so every array is
reproducible on any host.

Workloads (shapes from the 26B-A4B model on the axe-diffusion-ksl-xe model card,
"what the model is" / "requirements", and the DiffusionGemma page, "CLI flags"):

=========  ==========================================================================
tiny       1 MoE layer: 64 tokens, d_model 256, expert ffn 128, 8 experts top-2;
           sampler on [64, 4096] logits N(0,1) * 2, bound 1.0, temperature 1
layer      1 MoE layer at full shape: 256 tokens, d_model 2816, expert ffn 704,
           128 experts top-8, router logits N(0, 1)
short      the same layer over 64 tokens with Zipf(1.2)-skewed router logits
sampler    fp32 logits [256, 262144]: N(0, 1) plus one boosted entry per row
           (+U[0, 12]); bound 2.0; temperature 1 and 0
sampler_wide  the same with the boost drawn from U[0, 26] (entropies down to ~1e-5,
           so several positions pass the bound in one step)
stack      30 MoE layers at the layer shape with Zipf(1.2) routing, then the
           sampler; a 48-step denoising loop over a 256-token canvas
=========  ==========================================================================

Weights: packed bytes uniform over 0..255 (two independent uniform nibbles), fp16
scales uniform in [0.005, 0.02], fp16 zero-points uniform integers 0..15.
Activations N(0, 1) in fp16.  Zipf routing: logit[t, e] = ln p_rank(e) +
Gumbel(0, 1), p_r proportional to r^-1.2 over ranks 1..E, ranks a seeded
permutation of the experts; top-k of such logits is a draw without replacement
from the Zipf popularity.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    tokens: int
    d_model: int
    d_ff: int
    experts: int
    top_k: int
    group: int = 64
    zipf: float = 0.0          # 0 = N(0, 1) router logits, else the Zipf exponent


@dataclass(frozen=True)
class SamplerShape:
    positions: int
    vocab: int
    base_scale: float          # logits = base_scale * N(0, 1) (+ boost)
    boost_hi: float            # one entry per row boosted by U[0, boost_hi]; 0 = none
    bound: float
    temperature: float
    seed: int = 0              # Philox seed of the token draw


TINY_LAYER = LayerShape(64, 256, 128, 8, 2)
LAYER = LayerShape(256, 2816, 704, 128, 8)
SHORT_LAYER = LayerShape(64, 2816, 704, 128, 8, zipf=1.2)
STACK_LAYER = LayerShape(256, 2816, 704, 128, 8, zipf=1.2)
STACK_LAYERS = 30
STACK_STEPS = 48

TINY_SAMPLER = SamplerShape(64, 4096, 2.0, 0.0, 1.0, 1.0)
SAMPLER = SamplerShape(256, 262144, 1.0, 12.0, 2.0, 1.0)
SAMPLER_WIDE = SamplerShape(256, 262144, 1.0, 26.0, 2.0, 1.0)

SEED_X = 1
SEED_ROUTER = 2
SEED_PERM = 3
SEED_TINY_LOGITS = 4
SEED_LOGITS = 5
SEED_WEIGHTS = 100
SEED_HIDDEN = 6
SEED_NORM_ROUTER = 200
SEED_AFFINE = 300


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _random_bytes(rng, shape):
    n = int(np.prod(shape))
    words = rng.integers(0, 2 ** 64, size=(n + 7) // 8, dtype=np.uint64)
    return words.view(np.uint8)[:n].reshape(shape)


def _scales(rng, shape):
    u = rng.random(int(np.prod(shape)), dtype=np.float32)
    return (np.float32(0.005) + np.float32(0.015) * u).astype(np.float16).reshape(shape)


def _zeros(rng, shape):
    return (_random_bytes(rng, shape) & 0x0F).astype(np.float16)


def _biases(rng, scales):
    """Affine biases b = -z' s with a continuous z' ~ U[0, 15] (so b / s is not an integer),
    rounded to fp16: the same range as the asymmetric form's -z s."""
    zc = rng.random(scales.shape, dtype=np.float32) * np.float32(15.0)
    return (-(zc * scales.astype(np.float32))).astype(np.float16)


def make_weights(shape: LayerShape, layer: int = 0, gate_up_group: int = None,
                 down_group: int = None, affine: bool = False):
    """Packed uint4 expert weights of one layer (seed 100 + layer).

    Layout (see include/bdstep.h): gate_up_q [E][2f][d/2] (gate rows first),
    gate_up_scale / gate_up_zero fp16 [E][2f][d/g]; down_q [E][d][f/2],
    down_scale / down_zero fp16 [E][d][f/g_down].  The group sizes default to shape.group;
    gate_up_group=128 with down_group=64 is the format of the model card's checkpoint.
    affine=True puts affine biases (seed 300 + layer) in the *_zero arrays instead of
    zero-points.
    """
    E, d, f = shape.experts, shape.d_model, shape.d_ff
    g = gate_up_group or shape.group
    gd = down_group or shape.group
    rng = _rng(SEED_WEIGHTS + layer)
    w = {
        "gate_up_q": _random_bytes(rng, (E, 2 * f, d // 2)),
        "gate_up_scale": _scales(rng, (E, 2 * f, d // g)),
        "gate_up_zero": _zeros(rng, (E, 2 * f, d // g)),
        "down_q": _random_bytes(rng, (E, d, f // 2)),
        "down_scale": _scales(rng, (E, d, f // gd)),
        "down_zero": _zeros(rng, (E, d, f // gd)),
    }
    if affine:
        brng = _rng(SEED_AFFINE + layer)
        w["gate_up_zero"] = _biases(brng, w["gate_up_scale"])
        w["down_zero"] = _biases(brng, w["down_scale"])
    return w


def make_activations(shape: LayerShape, seed: int = SEED_X):
    """x ~ N(0, 1) as fp16 [T, d]."""
    rng = _rng(seed)
    return rng.standard_normal((shape.tokens, shape.d_model), dtype=np.float32).astype(np.float16)


def make_router_logits(shape: LayerShape, layer: int = 0):
    """fp32 [T, E] router logits: N(0, 1), or Zipf-skewed when shape.zipf > 0."""
    T, E = shape.tokens, shape.experts
    if shape.zipf <= 0:
        return _rng(SEED_ROUTER).standard_normal((T, E), dtype=np.float32)
    ranks = _rng(SEED_PERM).permutation(E) + 1
    log_pop = -shape.zipf * np.log(ranks.astype(np.float64))
    log_pop -= np.log(np.exp(log_pop).sum())
    u = _rng(SEED_ROUTER + layer).random((T, E))
    u = np.clip(u, 1e-300, None)
    return (log_pop[None, :] - np.log(-np.log(u))).astype(np.float32)


def make_layer(shape: LayerShape, layer: int = 0):
    """(x, router_logits, weights) of one layer."""
    return make_activations(shape), make_router_logits(shape, layer), make_weights(shape, layer)


def make_norm_router(shape: LayerShape, layer: int = 0):
    """Inputs of the RMS norm and router projection of one layer.

    hidden h ~ 3 N(0, 1) fp16 [T, d] (seed 6); norm weight 1 + 0.1 N(0, 1) fp16 [d] and router
    matrix N(0, 1) / sqrt(d) fp16 [E, d] (seed 200 + layer), so that the logits of a normed
    row are about N(0, 1), as the router logits of the other workloads.
    """
    T, d, E = shape.tokens, shape.d_model, shape.experts
    h = (3.0 * _rng(SEED_HIDDEN).standard_normal((T, d), dtype=np.float32)).astype(np.float16)
    rng = _rng(SEED_NORM_ROUTER + layer)
    w_norm = (1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32)).astype(np.float16)
    w_router = (rng.standard_normal((E, d), dtype=np.float32) / np.float32(np.sqrt(d))).astype(np.float16)
    return h, w_norm, w_router


def make_logits(shape: SamplerShape, seed: int = None):
    """fp32 [P, V] sampler logits: base_scale * N(0, 1), one entry per row boosted."""
    if seed is None:
        seed = SEED_TINY_LOGITS if shape.vocab <= 4096 else SEED_LOGITS
    rng = _rng(seed)
    P, V = shape.positions, shape.vocab
    x = rng.standard_normal((P, V), dtype=np.float32)
    if shape.base_scale != 1.0:
        x *= np.float32(shape.base_scale)
    if shape.boost_hi > 0:
        idx = rng.integers(0, V, size=P)
        boost = rng.random(P, dtype=np.float32) * np.float32(shape.boost_hi)
        x[np.arange(P), idx] += boost
    return x


def expert_bytes(shape: LayerShape, gate_up_group: int = None, down_group: int = None):
    """Packed bytes of one expert: nibbles plus fp16 scale and zero of both matrices (at the
    shape's group size, or the given per-matrix group sizes)."""
    d, f = shape.d_model, shape.d_ff
    gg, gd = gate_up_group or shape.group, down_group or shape.group
    gate_up = 2 * f * (d // 2) + 2 * (2 * f * (d // gg) * 2)
    down = d * (f // 2) + 2 * (d * (f // gd) * 2)
    return gate_up, down
