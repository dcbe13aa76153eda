"""The entry points under HIP graph capture, as the benchmark replays them.

A captured MoE layer (route, gate/up, down, combine), a captured sampler step and two
chained layers (norm, router, FFN, the combine with the next norm) are
replayed several times, with other eager work and synchronisations between the replays;
every replay must reproduce the eager result bit for bit (all kernels are deterministic),
and outputs are poisoned before each replay so that a launch missing from the graph shows.
"""

import numpy as np
import pytest

from block_diffusion_lm_router_amd import workloads
from gpu_common import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

REPLAYS = 3


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


def _moe_buffers(shape):
    import torch
    T, k, d = shape.tokens, shape.top_k, shape.d_model
    return (torch.empty((T, k), dtype=torch.int32, device="cuda"),
            torch.empty((T, k), dtype=torch.float32, device="cuda"),
            torch.empty((T, k, d), dtype=torch.float32, device="cuda"),
            torch.empty((T, d), dtype=torch.float16, device="cuda"))


def _moe_layer(bd, w, x, logits, bufs, ws):
    ids, tw, o, y = bufs
    bd.moe_route_topk(w, logits, ids, tw, ws)
    bd.moe_w4a16_gate_up(w, x, ws)
    bd.moe_w4a16_down(w, x.shape[0], o, ws)
    bd.moe_combine_fixed_order(o, tw, y)


def _poison(bufs):
    ids, tw, o, y = bufs
    ids.fill_(-7)
    tw.fill_(float("nan"))
    o.fill_(float("nan"))
    y.fill_(float("nan"))


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
@pytest.mark.parametrize("shape", [workloads.TINY_LAYER, workloads.SHORT_LAYER],
                         ids=["tiny", "short"])
def test_moe_layer_graph_replays(bd, shape, prepared):
    import torch
    say("graph moe layer", shape.tokens, shape.d_model, shape.experts, shape.top_k, prepared)
    w = bd.MoeWeights.from_numpy(workloads.make_weights(shape, 0), shape.top_k, prepare=prepared)
    x = torch.from_numpy(workloads.make_activations(shape)).cuda()
    logits = torch.from_numpy(workloads.make_router_logits(shape, 0)).cuda()
    # a second routing of the same layer, run eagerly between replays to disturb the workspace
    logits2 = torch.from_numpy(workloads.make_router_logits(shape, 1)).cuda()
    x2 = torch.flip(x, dims=[0]).contiguous()
    ws = bd.moe_workspace(shape.tokens, w)
    bufs = _moe_buffers(shape)

    _moe_layer(bd, w, x, logits, bufs, ws)
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _moe_layer(bd, w, x, logits, bufs, ws)
    other = _moe_buffers(shape)
    for r in range(REPLAYS):
        _poison(bufs)
        torch.cuda.synchronize()
        say("replay", r)
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(bufs, ref, ("ids", "weights", "expert_out", "y")):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager run"
        _moe_layer(bd, w, x2, logits2, other, ws)   # eager work on the shared workspace
        torch.cuda.synchronize()


def test_sampler_step_graph_replays(bd):
    import torch
    shape = workloads.TINY_SAMPLER
    P, V = shape.positions, shape.vocab
    say("graph sampler step", P, V)
    logits = torch.from_numpy(workloads.make_logits(shape)).cuda()
    ws = bd.sample_workspace(P, V)
    frozen0 = torch.zeros(P, dtype=torch.uint8, device="cuda")
    frozen0[::5] = 1
    canvas0 = torch.full((P,), 3, dtype=torch.int32, device="cuda")

    def make():
        return dict(frozen=frozen0.clone(), canvas=canvas0.clone(),
                    tok=torch.empty(P, dtype=torch.int32, device="cuda"),
                    H=torch.empty(P, dtype=torch.float32, device="cuda"),
                    acc=torch.empty(P, dtype=torch.uint8, device="cuda"),
                    n=torch.empty(1, dtype=torch.int32, device="cuda"))

    def run(b, step):
        bd.diffusion_sample_step(logits, shape.temperature, shape.bound, shape.seed, step,
                                 b["frozen"], b["canvas"], b["tok"], b["H"], b["acc"], b["n"], ws)

    eager = make()
    run(eager, 5)
    torch.cuda.synchronize()
    b = make()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(b, 5)
    other = make()
    for r in range(REPLAYS):
        b["frozen"].copy_(frozen0)
        b["canvas"].copy_(canvas0)
        for key in ("tok", "n"):
            b[key].fill_(-9)
        b["H"].fill_(float("nan"))
        b["acc"].fill_(7)
        torch.cuda.synchronize()
        say("replay", r)
        g.replay()
        torch.cuda.synchronize()
        for key in eager:
            assert torch.equal(b[key], eager[key]), f"replay {r}: {key} differs from eager"
        n = int(b["n"].item())
        assert 1 <= n == int(b["acc"].sum().item())
        run(other, 11)                               # eager work on the shared workspace
        torch.cuda.synchronize()
    assert np.array_equal(b["frozen"].cpu().numpy() > 0,
                          (frozen0.cpu().numpy() > 0) | (b["acc"].cpu().numpy() > 0))


def test_chained_layers_graph_replays(bd):
    """Two chained layers as the chain workload captures them (gated launches: RMS norm, router
    projection, the one-call FFN, the combine with the next layer's norm, then the last
    combine): every replay reproduces the eager chain bit for bit."""
    import torch
    shape = workloads.TINY_LAYER
    T, d, E, k = shape.tokens, shape.d_model, shape.experts, shape.top_k
    say("graph chained layers", T, d, E, k)
    h0_np, _, _ = workloads.make_norm_router(shape)
    h0 = torch.from_numpy(h0_np).cuda()
    layers = []
    for l in range(2):
        _, wn, wr = workloads.make_norm_router(shape, l)
        layers.append((bd.MoeWeights.from_numpy(workloads.make_weights(shape, l), k, prepare=True),
                       torch.from_numpy(wn).cuda(), torch.from_numpy(wr).cuda()))
    ws = bd.moe_workspace(T, layers[0][0])
    state = torch.zeros(4, dtype=torch.int32, device="cuda")

    def make():
        return dict(xn=torch.empty((T, d), dtype=torch.float16, device="cuda"),
                    rl=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                    ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                    tw=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                    o=torch.empty((T, k, d), dtype=torch.float32, device="cuda"),
                    y0=torch.empty((T, d), dtype=torch.float16, device="cuda"),
                    y1=torch.empty((T, d), dtype=torch.float16, device="cuda"))

    def chain(b):
        bd.moe_rmsnorm(h0, layers[0][1], b["xn"], loop_state=state)
        for l, (w, wn, wr) in enumerate(layers):
            bd.moe_router_logits(b["xn"], wr, b["rl"], loop_state=state)
            bd.moe_w4a16_ffn(w, b["xn"], b["rl"], b["ids"], b["tw"], b["o"], ws, loop_state=state)
            if l == 0:
                bd.moe_combine_rmsnorm(b["o"], b["tw"], layers[1][1], b["y0"], b["xn"],
                                       loop_state=state)
            else:
                bd.moe_combine_fixed_order(b["o"], b["tw"], b["y1"], loop_state=state)

    eager = make()
    chain(eager)
    torch.cuda.synchronize()
    b = make()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(b)
    other = make()
    for r in range(REPLAYS):
        for key, t in b.items():
            t.fill_(-3 if t.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        say("replay", r)
        g.replay()
        torch.cuda.synchronize()
        for key in eager:
            assert torch.equal(b[key], eager[key]), f"replay {r}: {key} differs from eager"
        chain(other)                                 # eager work on the shared workspace
        torch.cuda.synchronize()
