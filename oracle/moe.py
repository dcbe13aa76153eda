"""Oracle for the W4A16 mixture-of-experts FFN and its fixed-order combine.

Passages followed (pages named in the package docstring):

* axe-diffusion-ksl-xe model card, "what the model is": 128 experts, top-8
  routing per token.
* same, "the kernels we built": expert weights are asymmetric uint4 with an fp16
  scale and zero-point per group, read as packed nibbles and dequantised; the
  activation is folded into the first (gate/up) GEMM's epilogue; the weighted
  combine is a fixed-order reduction rather than an atomic index_add.
* same, "requirements": two nibbles per byte, groups run along the contraction
  dimension (down_proj's contraction dimension is 704).

Readings taken where the pages are silent:

* byte i of a packed row holds element 2i in its low nibble and 2i+1 in its
  high nibble; rows are output features, packed along the contraction dim K;
* the fused gate_up matrix holds the gate rows first (rows 0..f-1), then the up
  rows (f..2f-1);
* the gated activation is GeGLU with the tanh form of GELU,
  gelu(a) = a/2 * (1 + tanh(sqrt(2/pi) * (a + 0.044715 a^3)));
* top-k orders experts by descending router logit, the lower expert id first on
  equal logits; the k weights are the softmax over the k selected logits;
* the combine sums slot j = 0..k-1 in ascending order.

Everything is computed in float64 from the exact widened fp16/uint4 inputs, with
no intermediate rounding.  Test infrastructure only.
"""

import numpy as np

GROUP = 64


def unpack_nibbles(packed):
    """uint8 [..., K/2] -> int64 [..., K]; element 2i is the low nibble of byte i."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & 0x0F).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(packed, scale, zero, group=GROUP):
    """Dequantise one matrix: w[n, k] = (q[n, k] - z[n, k // g]) * s[n, k // g].

    ``packed`` uint8 [N, K/2]; ``scale`` and ``zero`` fp16 [N, K/g].  The fp16
    values are widened exactly to float64, so the result is exact.
    """
    q = unpack_nibbles(packed).astype(np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float16).astype(np.float64), group, axis=-1)
    z = np.repeat(np.asarray(zero, dtype=np.float16).astype(np.float64), group, axis=-1)
    return (q - z) * s


def dequant_affine(packed, scale, bias, group=GROUP):
    """Affine form: w[n, k] = q[n, k] * s[n, k // g] + b[n, k // g] (exact in float64).

    The MLX-style 4-bit checkpoints (a 4/64 affine format named on the TensorFold XPU page)
    store a free fp16 bias per group instead of an integer zero-point; b = -z * s gives back
    the asymmetric form.
    """
    q = unpack_nibbles(packed).astype(np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float16).astype(np.float64), group, axis=-1)
    b = np.repeat(np.asarray(bias, dtype=np.float16).astype(np.float64), group, axis=-1)
    return q * s + b


def route_topk(router_logits, k):
    """Top-k experts per token and their softmax weights.

    Returns ids int32 [T, k] (descending logit, lower id first on ties) and
    weights float64 [T, k] = softmax over the k selected logits.
    """
    logits = np.asarray(router_logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # np.lexsort sorts by the last key first: logit descending, then id ascending.
        order = np.lexsort((np.arange(E), -logits[t]))
        ids[t] = order[:k]
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    weights = ex / ex.sum(axis=1, keepdims=True)
    return ids, weights


def gelu_tanh(a):
    """GELU in the tanh form (Hendrycks & Gimpel, 2016)."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (a + 0.044715 * a ** 3)))


def expert_matrices(weights, e, group=GROUP, down_group=None, affine=False):
    """Dense float64 gate, up and down matrices of expert ``e``.

    ``weights`` maps the names gate_up_q, gate_up_scale, gate_up_zero, down_q,
    down_scale, down_zero to arrays laid out [E][rows][...] as in the C header.
    ``group`` is the gate/up group size, ``down_group`` the down one (None: the same);
    the checkpoint format on the model card's "requirements" groups gate_up at 128 and
    down at 64.  With ``affine`` the *_zero arrays hold the affine bias b instead of a
    zero-point (w = q s + b).  Returns (W_gate [f, d], W_up [f, d], W_down [d, f]).
    """
    deq = dequant_affine if affine else dequant
    gu = deq(weights["gate_up_q"][e], weights["gate_up_scale"][e],
             weights["gate_up_zero"][e], group)
    f = gu.shape[0] // 2
    wd = deq(weights["down_q"][e], weights["down_scale"][e],
             weights["down_zero"][e], group if down_group is None else down_group)
    return gu[:f], gu[f:], wd


def expert_ffn(x_rows, w_gate, w_up, w_down):
    """o = W_down (gelu(W_gate x) * (W_up x)) for each row of ``x_rows`` [M, d]."""
    x = np.asarray(x_rows, dtype=np.float64)
    a = x @ w_gate.T
    u = x @ w_up.T
    return (gelu_tanh(a) * u) @ w_down.T


def moe_expert_outputs(x, ids, weights, group=GROUP, tokens=None, down_group=None,
                       affine=False):
    """Per-assignment expert outputs o[t, j] = FFN_{ids[t, j]}(x[t]).

    ``x`` fp16 [T, d]; returns float64 [T, k, d].  With ``tokens`` given, only
    those token rows are computed (the others stay NaN).
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    T, k = ids.shape
    d = x64.shape[1]
    out = np.full((T, k, d), np.nan)
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    mask = np.zeros(T, dtype=bool)
    mask[rows] = True
    for e in np.unique(ids[rows]):
        tt, jj = np.nonzero((ids == e) & mask[:, None])
        w_gate, w_up, w_down = expert_matrices(weights, int(e), group, down_group, affine)
        out[tt, jj] = expert_ffn(x64[tt], w_gate, w_up, w_down)
    return out


def combine(expert_out, topk_weights):
    """y[t] = sum_{j=0}^{k-1} w[t, j] * o[t, j], slots in ascending order."""
    o = np.asarray(expert_out, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    y = np.zeros((o.shape[0], o.shape[2]))
    for j in range(o.shape[1]):
        y = y + w[:, j:j + 1] * o[:, j]
    return y


def moe_ffn(x, router_logits, weights, k, group=GROUP, tokens=None, down_group=None,
            affine=False):
    """The whole layer: route, run the selected experts, combine.

    Returns (ids, topk_weights, expert_out [T, k, d], y [T, d]) in float64.
    """
    ids, tw = route_topk(router_logits, k)
    o = moe_expert_outputs(x, ids, weights, group, tokens, down_group, affine)
    return ids, tw, o, combine(o, tw)
