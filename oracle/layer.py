"""Oracle for the two steps either side of the expert FFN in a layer: the RMS norm that
produces the FFN's input, and the router projection whose logits feed the top-k.

Passages followed (pages named in the package docstring):

* axe-diffusion-ksl-xe model card, "the kernels we built": the RMS norm runs as one fused
  launch (it was about six elementwise launches), 180 times per forward pass.
* same, "what the model is": 128 experts, top-8 routing per token; the router scores
  every expert for every token.

Readings taken where the pages are silent:

* RMS norm: y = h / sqrt(mean_d(h^2) + eps) * w, per row, with a learned per-feature
  weight w and eps = 1e-6 (no mean subtraction, no bias, w used as stored);
* router: logits[t, e] = sum_d x[t, d] * W_r[e, d] with W_r stored expert-major [E][d]
  (out x in, like the expert matrices), no bias; the logits are the input of the top-k.

Everything is float64 from the exactly widened fp16 inputs, with no intermediate rounding.
Test infrastructure only.
"""

import numpy as np

RMS_EPS = 1e-6


def rmsnorm(h, weight, eps=RMS_EPS):
    """Row-wise RMS norm of h [T, d] with weight [d]: float64 [T, d]."""
    h = np.asarray(h, dtype=np.float16).astype(np.float64)
    w = np.asarray(weight, dtype=np.float16).astype(np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return h / np.sqrt(ms + eps) * w[None, :]


def router_logits(x, w_router):
    """logits [T, E] = x [T, d] @ W_r[E, d]^T in float64 (x taken as given)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float16).astype(np.float64)
    return x @ w.T
