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


def test_gated_norm_and_router(bd):
    """The gated forms: with the driver's done flag clear they write exactly what the plain
    forms write; with it set they write nothing."""
    import torch
    shape = workloads.LAYER
    h_np, wn_np, wr_np = workloads.make_norm_router(shape)
    T, d, E = shape.tokens, shape.d_model, shape.experts
    h = torch.from_numpy(h_np).cuda()
    wn = torch.from_numpy(wn_np).cuda()
    wr = torch.from_numpy(wr_np).cuda()
    y0 = torch.empty((T, d), dtype=torch.float16, device="cuda")
    l0 = torch.empty((T, E), dtype=torch.float32, device="cuda")
    bd.moe_rmsnorm(h, wn, y0)
    bd.moe_router_logits(y0, wr, l0)
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    y1 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    l1 = torch.full((T, E), 7.0, dtype=torch.float32, device="cuda")
    say("gated norm+router: running")
    bd.moe_rmsnorm(h, wn, y1, loop_state=state)
    bd.moe_router_logits(y1, wr, l1, loop_state=state)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
    state[2] = 1
    y2 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    l2 = torch.full((T, E), 7.0, dtype=torch.float32, device="cuda")
    say("gated norm+router: done")
    bd.moe_rmsnorm(h, wn, y2, loop_state=state)
    bd.moe_router_logits(y0, wr, l2, loop_state=state)
    torch.cuda.synchronize()
    assert bool((y2 == 7.0).all()) and bool((l2 == 7.0).all())


@pytest.mark.parametrize("which,n_layers", [("tiny", 3), ("layer", 2)])
def test_chained_layers(bd, which, n_layers):
    """Layers chained on the device as the chain workload runs them: RMS norm, router
    projection, the one-call FFN (routing, gate/up, down) and the combine, whose output is the
    next layer's input (the combine and the next layer's norm in one launch).  Every stage is checked against the oracle fed that stage's GPU inputs
    (a routing decision taken from slightly different upstream values would otherwise be
    compared with a different one): the norm and router bars above, top-k ids bit-exact,
    expert outputs and combined outputs to the FFN bars."""
    import torch
    from test_gpu_moe import Layer, check_layer
    shape = {"tiny": workloads.TINY_LAYER, "layer": workloads.LAYER}[which]
    T, d, f, E, k = shape.tokens, shape.d_model, shape.d_ff, shape.experts, shape.top_k
    h0, _, _ = workloads.make_norm_router(shape)
    weights, norms, routers = [], [], []
    for l in range(n_layers):
        w_np = workloads.make_weights(shape, l)
        _, wn, wr = workloads.make_norm_router(shape, l)
        weights.append((w_np, bd.MoeWeights.from_numpy(w_np, k, prepare=True)))
        norms.append(torch.from_numpy(wn).cuda())
        routers.append(torch.from_numpy(wr).cuda())
    ws = bd.moe_workspace(T, weights[0][1])
    h = [torch.from_numpy(h0).cuda()] + [torch.empty((T, d), dtype=torch.float16, device="cuda")
                                          for _ in range(n_layers)]
    xs, lgs, got = [], [], []
    say("chained layers", which, n_layers)
    x = torch.empty((T, d), dtype=torch.float16, device="cuda")
    bd.moe_rmsnorm(h[0], norms[0], x)
    for l in range(n_layers):
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        o = torch.full((T, k, d), float("nan"), dtype=torch.float32, device="cuda")
        bd.moe_router_logits(x, routers[l], lg)
        bd.moe_w4a16_ffn(weights[l][1], x, lg, ids, tw, o, ws)
        xs.append(x)
        if l + 1 < n_layers:       # the combine and the next layer's norm in one launch
            x = torch.empty((T, d), dtype=torch.float16, device="cuda")
            bd.moe_combine_rmsnorm(o, tw, norms[l + 1], h[l + 1], x)
        else:
            bd.moe_combine_fixed_order(o, tw, h[l + 1])
        lgs.append(lg)
        got.append((ids, tw, o))
    torch.cuda.synchronize()
    for l in range(n_layers):
        h_l = h[l].cpu().numpy()
        x_l = xs[l].cpu().numpy()
        lg_l = lgs[l].cpu().numpy()
        check_norm(x_l, h_l, norms[l].cpu().numpy())
        check_router(lg_l, x_l, routers[l].cpu().numpy())
        layer = Layer(bd, shape, x=x_l, logits=lg_l, weights=weights[l][0], layer=l)
        ids, tw, o = got[l]
        check_layer(layer, (ids.cpu().numpy(), tw.cpu().numpy(), o.cpu().numpy(),
                            h[l + 1].cpu().numpy()))
        assert np.isfinite(h[l + 1].cpu().numpy().astype(np.float32)).all()


def _combine_norm_inputs(T, k, d, seed):
    rng = np.random.default_rng(seed)
    o = (rng.standard_normal((T, k, d)) * rng.uniform(0.1, 30)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    wn = (1 + 0.2 * rng.standard_normal(d)).astype(np.float16)
    return o, w, wn


@pytest.mark.parametrize("T,k,d", [(256, 8, 2816), (1, 8, 8), (5, 1, 8), (7, 3, 4096),
                                   (64, 16, 1024), (33, 8, 4088), (300, 2, 2816),
                                   (64, 8, 4096), (3, 8, 1032)])
def test_combine_rmsnorm_matches_combine_then_norm(bd, T, k, d):
    """moe_combine_rmsnorm against the two launches it replaces (bit for bit, both outputs)
    and against the oracle: y to the combine's bar (one fp16 rounding plus k fp32 roundings),
    xn to the norm's bar from the GPU's y."""
    import torch
    o_np, w_np, wn_np = _combine_norm_inputs(T, k, d, T * 7 + k * 3 + d)
    o, w, wn = (torch.from_numpy(a).cuda() for a in (o_np, w_np, wn_np))
    y2 = torch.empty((T, d), dtype=torch.float16, device="cuda")
    x2 = torch.empty((T, d), dtype=torch.float16, device="cuda")
    bd.moe_combine_fixed_order(o, w, y2)
    bd.moe_rmsnorm(y2, wn, x2)
    y1 = torch.full((T, d), float("nan"), dtype=torch.float16, device="cuda")
    x1 = torch.full((T, d), float("nan"), dtype=torch.float16, device="cuda")
    say("combine+norm one launch", T, k, d)
    bd.moe_combine_rmsnorm(o, w, wn, y1, x1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))
    y = y1.cpu().numpy()
    ref = omoe.combine(o_np.astype(np.float64), w_np.astype(np.float64))
    half_ulp = 0.5 * np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    fp32_sum = 2.0 ** -24 * k * np.einsum("tj,tjd->td", np.abs(w_np.astype(np.float64)),
                                          np.abs(o_np.astype(np.float64)))
    assert np.all(np.abs(y.astype(np.float64) - ref) <= half_ulp * 1.0001 + fp32_sum)
    check_norm(x1.cpu().numpy(), y, wn_np)


def test_combine_rmsnorm_gated(bd):
    """The gated form writes what the plain one writes while the block runs, nothing once the
    driver state says done."""
    import torch
    T, k, d = 64, 8, 2816
    o_np, w_np, wn_np = _combine_norm_inputs(T, k, d, 11)
    o, w, wn = (torch.from_numpy(a).cuda() for a in (o_np, w_np, wn_np))
    y0 = torch.empty((T, d), dtype=torch.float16, device="cuda")
    x0 = torch.empty((T, d), dtype=torch.float16, device="cuda")
    bd.moe_combine_rmsnorm(o, w, wn, y0, x0)
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    y1 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    x1 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    say("gated combine+norm: running")
    bd.moe_combine_rmsnorm(o, w, wn, y1, x1, loop_state=state)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    assert torch.equal(x1.view(torch.int16), x0.view(torch.int16))
    state[2] = 1
    y2 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    x2 = torch.full((T, d), 7.0, dtype=torch.float16, device="cuda")
    say("gated combine+norm: done")
    bd.moe_combine_rmsnorm(o, w, wn, y2, x2, loop_state=state)
    torch.cuda.synchronize()
    assert bool((y2 == 7.0).all()) and bool((x2 == 7.0).all())
