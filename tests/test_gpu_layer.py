"""GPU parity of the layer neighbours of the FFN (moe_rmsnorm, moe_router_logits) against the
CPU oracle, through the C ABI.

Bars (derived from the arithmetic):
* RMS norm, fp16 out: |y - y_ref| <= (2^-11 + 2e-6) |y_ref| + 2^-24 -- one round-to-nearest
  to fp16 of an fp32 value within a few fp32 ulps of the exact one.
* Router logits from the GPU's own normed rows: |l - l_ref| <= 2e-5 sum_i |x_i W_ei| -- fp32
  accumulation over at most d/128 + 4 sequential additions of MFMA partial sums.
* From the hidden state end to end: the norm's fp16 rounding adds 2^-11 sum_i |x_i W_ei|.
* Top-k ids of the GPU's logits: bit-exact against the oracle's top-k of the same logits.
"""

import numpy as np
import pytest

from block_diffusion_lm_router_amd import workloads
from oracle import layer as olayer, moe as omoe
from gpu_common import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

NORM_REL = 2.0 ** -11 + 2e-6
NORM_ABS = 2.0 ** -24
ROUTER_REL = 2e-5


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


def run(bd, h_np, wn_np, wr_np, eps=olayer.RMS_EPS):
    import torch
    T, d = h_np.shape
    E = wr_np.shape[0]
    h = torch.from_numpy(np.ascontiguousarray(h_np)).cuda()
    wn = torch.from_numpy(np.ascontiguousarray(wn_np)).cuda()
    wr = torch.from_numpy(np.ascontiguousarray(wr_np)).cuda()
    y = torch.empty((T, d), dtype=torch.float16, device="cuda")
    logits = torch.full((T, E), np.nan, dtype=torch.float32, device="cuda")
    bd.moe_rmsnorm(h, wn, y, eps)
    bd.moe_router_logits(y, wr, logits)
    torch.cuda.synchronize()
    return y.cpu().numpy(), logits.cpu().numpy()


def check_norm(y, h, wn, eps=olayer.RMS_EPS):
    ref = olayer.rmsnorm(h, wn, eps)
    err = np.abs(y.astype(np.float64) - ref)
    bound = NORM_REL * np.abs(ref) + NORM_ABS
    assert np.all(err <= bound), f"norm: worst ratio {(err / bound).max():.3g}"


def check_router(logits, x16, wr, extra_rel=0.0):
    x = x16.astype(np.float64)
    ref = olayer.router_logits(x, wr)
    mag = np.abs(x) @ np.abs(wr.astype(np.float64)).T
    err = np.abs(logits.astype(np.float64) - ref)
    bound = (ROUTER_REL + extra_rel) * mag + 1e-30
    assert np.all(err <= bound), f"router: worst ratio {(err / bound).max():.3g}"


@pytest.mark.parametrize("which", ["tiny", "layer", "short"])
def test_workload_shapes(bd, which):
    shape = {"tiny": workloads.TINY_LAYER, "layer": workloads.LAYER,
             "short": workloads.SHORT_LAYER}[which]
    h, wn, wr = workloads.make_norm_router(shape)
    say("norm+router", which, h.shape, wr.shape)
    y, logits = run(bd, h, wn, wr)
    check_norm(y, h, wn)
    check_router(logits, y, wr)
    # end to end from the hidden state: the fp16 rounding of the normed rows on top
    x_ref = olayer.rmsnorm(h, wn)
    ref = olayer.router_logits(x_ref, wr)
    mag = np.abs(x_ref) @ np.abs(wr.astype(np.float64)).T
    assert np.all(np.abs(logits - ref) <= (ROUTER_REL + NORM_REL) * mag)
    # the top-k of the GPU's logits, on the GPU, is the oracle's top-k of the same logits
    import torch
    k = shape.top_k
    wq = workloads.make_weights(shape) if which == "tiny" else None
    if wq is not None:
        w = bd.MoeWeights.from_numpy(wq, k)
        ids = torch.empty((shape.tokens, k), dtype=torch.int32, device="cuda")
        tw = torch.empty((shape.tokens, k), dtype=torch.float32, device="cuda")
        ws = bd.moe_workspace(shape.tokens, w)
        bd.moe_route_topk(w, torch.from_numpy(logits).cuda(), ids, tw, ws)
        torch.cuda.synchronize()
        ref_ids, _ = omoe.route_topk(logits, k)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)


@pytest.mark.parametrize("T,d,E", [(1, 128, 1), (3, 256, 5), (17, 384, 33), (37, 1024, 16),
                                   (64, 4096, 256), (100, 2816, 128)])
def test_ragged_shapes(bd, T, d, E):
    rng = np.random.default_rng(T * 31 + d + E)
    h = (rng.standard_normal((T, d)) * rng.uniform(0.01, 20)).astype(np.float16)
    wn = (1 + 0.3 * rng.standard_normal(d)).astype(np.float16)
    wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float16)
    say("norm+router ragged", T, d, E)
    y, logits = run(bd, h, wn, wr)
    check_norm(y, h, wn)
    check_router(logits, y, wr)


def test_norm_special_rows(bd):
    d = 512
    rng = np.random.default_rng(9)
    h = rng.standard_normal((6, d)).astype(np.float16)
    h[0] = 0                                         # zero row -> zeros (eps keeps it finite)
    h[1] = 60000                                     # large values: squares exact, sum in fp32
    h[2] = np.float16(1e-4)                          # tiny values: eps dominates
    h[3, ::2] = 0
    wn = (1 + 0.1 * rng.standard_normal(d)).astype(np.float16)
    wr = (rng.standard_normal((8, d)) / np.sqrt(d)).astype(np.float16)
    say("norm special rows")
    for eps in (1e-6, 0.0, 0.25):
        if eps == 0.0:
            hh = h[1:].copy()                        # a zero row has no norm without eps
        else:
            hh = h
        y, logits = run(bd, hh, wn, wr, eps)
        check_norm(y, hh, wn, eps)
        check_router(logits, y, wr)
    y, _ = run(bd, h, wn, wr)
    assert np.all(y[0] == 0)


def test_repeat_runs_bit_identical(bd):
    h, wn, wr = workloads.make_norm_router(workloads.LAYER)
    say("norm+router repeat")
    a = run(bd, h, wn, wr)
    for _ in range(2):
        b = run(bd, h, wn, wr)
        assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
