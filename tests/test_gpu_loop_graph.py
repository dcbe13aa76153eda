"""GPU: one block of the denoising loop captured in a single HIP graph and replayed, with the
done gate: canvas init, then max_steps x (two MoE layers through the gated FFN and combine,
the gated sampler step, the loop update).  After the block ends, every gated launch must leave
its outputs alone; the live steps must match the oracle in lockstep (tokens bit-exact, masks
fed the GPU's entropies, canvas, frozen set and driver state bit-exact; top-k ids bit-exact
and the FFN output within the FFN bar).

Source: DiffusionGemma block-diffusion page, "How it works" (random initial canvas, at most the
step budget, early stop once the canvas is unchanged for stability_threshold steps).
"""

import numpy as np
import pytest

from block_diffusion_lm_router_amd import workloads
from oracle import loop as oloop, moe as omoe, sampler as osamp
from gpu_common import check_ffn_close, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

SENT = -7


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


def capture_block(bd, layers, x, logits, temperature, bound, threshold, max_steps, seed, vocab):
    import torch
    shape = workloads.TINY_LAYER
    T, d, k = shape.tokens, shape.d_model, shape.top_k
    P, V = logits.shape
    L = len(layers)
    dev = "cuda"
    buf = {
        "ids": torch.empty((max_steps, L, T, k), dtype=torch.int32, device=dev),
        "y": torch.empty((max_steps, L, T, d), dtype=torch.float16, device=dev),
        "tok": torch.empty((max_steps, P), dtype=torch.int32, device=dev),
        "H": torch.empty((max_steps, P), dtype=torch.float32, device=dev),
        "acc": torch.empty((max_steps, P), dtype=torch.uint8, device=dev),
        "cnt": torch.empty(max_steps, dtype=torch.int32, device=dev),
        "canvas": torch.empty(P, dtype=torch.int32, device=dev),
        "prev": torch.empty(P, dtype=torch.int32, device=dev),
        "frozen": torch.empty(P, dtype=torch.uint8, device=dev),
        "state": torch.empty(4, dtype=torch.int32, device=dev),
    }
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    o = torch.empty((T, k, d), dtype=torch.float32, device=dev)
    mws = [bd.moe_workspace(T, w) for w, _ in layers]
    sws = bd.sample_workspace(P, V)
    lg = torch.from_numpy(logits).cuda()
    xd = torch.from_numpy(x).cuda()
    st = buf["state"]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bd.diffusion_canvas_init(buf["canvas"], buf["prev"], buf["frozen"], st, vocab, seed, 0)
        for s in range(max_steps):
            for li, ((w, r), ws) in enumerate(zip(layers, mws)):
                bd.moe_w4a16_ffn(w, xd, r, buf["ids"][s, li], tw, o, ws, loop_state=st)
                bd.moe_combine_fixed_order(o, tw, buf["y"][s, li], loop_state=st)
            bd.diffusion_sample_step(lg, temperature, bound, seed, s, buf["frozen"], buf["canvas"],
                                     buf["tok"][s], buf["H"][s], buf["acc"][s],
                                     buf["cnt"][s:s + 1], sws, loop_state=st)
            bd.diffusion_loop_update(buf["tok"][s], buf["canvas"], buf["prev"], buf["frozen"], st,
                                     threshold, max_steps)
    keep = (tw, o, mws, sws, lg, xd)
    return g, buf, keep


def fill_sentinels(buf):
    for key in ("ids", "tok", "H", "cnt", "acc"):
        buf[key].fill_(SENT if key != "acc" else 7)
    buf["y"].fill_(float("nan"))
    for key in ("canvas", "prev", "state"):
        buf[key].fill_(SENT)
    buf["frozen"].fill_(5)


def check_against_oracle(buf, x, w_np, r_np, logits, temperature, bound, threshold, max_steps,
                         seed, vocab, k):
    """Lockstep with the oracle; returns the number of steps the block ran."""
    P = logits.shape[0]
    got = {key: t.cpu().numpy() for key, t in buf.items()}
    c_o = oloop.init_canvas(P, vocab, seed, 0)
    p_o = c_o.copy()
    f_o = np.zeros(P, dtype=np.uint8)
    s_o = np.zeros(4, dtype=np.int64)
    ref_ffn = [omoe.moe_ffn(x, r, w, k) for w, r in zip(w_np, r_np)]
    ran = 0
    for s in range(max_steps):
        if s_o[oloop.DONE]:
            # gated: nothing written at this step
            assert np.all(got["ids"][s] == SENT) and np.all(np.isnan(got["y"][s].astype(np.float32)))
            assert np.all(got["tok"][s] == SENT) and np.all(got["cnt"][s] == SENT)
            assert np.all(got["acc"][s] == 7)
            continue
        ran += 1
        for li, (ids_r, _, _, y_r) in enumerate(ref_ffn):
            assert np.array_equal(got["ids"][s, li], ids_r), f"step {s} layer {li}: ids"
            check_ffn_close(got["y"][s, li].astype(np.float64), y_r, f"step {s} layer {li}: y")
        H_ref, tok_ref = osamp.sample_rows(logits, temperature, seed, s, frozen=f_o)
        assert np.array_equal(got["tok"][s], tok_ref), f"step {s}: tokens"
        H_gpu = got["H"][s]
        live = f_o == 0
        assert np.all(np.abs(H_gpu[live] - H_ref[live]) <= 1e-4 * H_ref[live])
        mask, n = osamp.accept(H_gpu, bound, f_o)
        assert got["cnt"][s] == n and np.array_equal(got["acc"][s], mask), f"step {s}: mask"
        c_o[mask == 1] = tok_ref[mask == 1]
        f_o = np.maximum(f_o, mask)
        oloop.loop_update(tok_ref, c_o, p_o, f_o, s_o, threshold, max_steps)
    assert np.array_equal(got["canvas"], c_o) and np.array_equal(got["prev"], p_o)
    assert np.array_equal(got["frozen"], f_o)
    assert np.array_equal(got["state"], s_o)
    return ran


@pytest.mark.parametrize("case", ["ends early", "runs to budget"])
def test_captured_gated_block_matches_oracle(bd, case):
    import torch
    shape = workloads.TINY_LAYER
    x = workloads.make_activations(shape)
    w_np = [workloads.make_weights(shape, l) for l in range(2)]
    r_np = [workloads.make_router_logits(shape, l) for l in range(2)]
    layers = [(bd.MoeWeights.from_numpy(w, shape.top_k, prepare=True),
               torch.from_numpy(r).cuda()) for w, r in zip(w_np, r_np)]
    logits = workloads.make_logits(workloads.TINY_SAMPLER)          # [64, 4096]
    temperature, threshold, max_steps = (0.0, 2, 10) if case == "ends early" else (1.0, 3, 6)
    bound, seed, vocab = 1.0, 3, 4096
    say("captured gated block", case)
    g, buf, keep = capture_block(bd, layers, x, logits, temperature, bound, threshold,
                                 max_steps, seed, vocab)
    results = []
    for rep in range(2):
        fill_sentinels(buf)                        # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ran = check_against_oracle(buf, x, w_np, r_np, logits, temperature, bound, threshold,
                                   max_steps, seed, vocab, shape.top_k)
        results.append({key: t.cpu().numpy().copy() for key, t in buf.items()})
    for key in results[0]:
        assert np.array_equal(results[0][key].view(np.uint8), results[1][key].view(np.uint8)), key
    if case == "ends early":
        assert ran == 3          # drafts written at step 0, then two unchanged steps
    else:
        assert ran == max_steps
    del keep
