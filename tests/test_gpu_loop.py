"""GPU parity of the denoising-loop driver (diffusion_canvas_init, diffusion_loop_update) with
the sampler steps, in lockstep with the CPU oracle, through the C ABI.

Bars: the initial canvas bit-exact; at every step the acceptance mask (fed the GPU's entropies
or confidences), the canvas, the previous canvas, the frozen set and the driver state bit-exact;
tokens at T = 0 bit-exact and at T > 0 bit-exact except near-ties (counted).
"""

import numpy as np
import pytest

from oracle import loop as oloop, sampler as osamp
from gpu_common import requires_gpu, say
from test_gpu_sampler import check_tokens_sampled

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


@pytest.mark.parametrize("P,vocab,seed,block", [(1, 1, 0, 0), (7, 5, 3, 1), (256, 262144, 0, 0),
                                                (1000, 1 << 24, (7 << 32) | 9, 77),
                                                (1024, 262144, 123456789, 4)])
def test_canvas_init_matches_oracle(bd, P, vocab, seed, block):
    import torch
    canvas = torch.full((P,), -9, dtype=torch.int32, device="cuda")
    prev = torch.full((P,), -9, dtype=torch.int32, device="cuda")
    frozen = torch.ones(P, dtype=torch.uint8, device="cuda")
    state = torch.full((4,), 5, dtype=torch.int32, device="cuda")
    say("canvas init", P, vocab, seed, block)
    bd.diffusion_canvas_init(canvas, prev, frozen, state, vocab, seed, block)
    torch.cuda.synchronize()
    ref = oloop.init_canvas(P, vocab, seed, block)
    assert np.array_equal(canvas.cpu().numpy(), ref)
    assert np.array_equal(prev.cpu().numpy(), ref)
    assert not frozen.cpu().numpy().any() and not state.cpu().numpy().any()


def run_block(bd, logits_for_step, temperature, rule, param, threshold, max_steps, seed=0,
              vocab=None):
    """Drive one block on the GPU, checking every step against the oracle; returns the steps."""
    import torch
    P, V = logits_for_step(0).shape
    vocab = vocab or V
    canvas = torch.empty(P, dtype=torch.int32, device="cuda")
    prev = torch.empty(P, dtype=torch.int32, device="cuda")
    frozen = torch.empty(P, dtype=torch.uint8, device="cuda")
    state = torch.empty(4, dtype=torch.int32, device="cuda")
    tok = torch.empty(P, dtype=torch.int32, device="cuda")
    stat = torch.empty(P, dtype=torch.float32, device="cuda")
    acc = torch.empty(P, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = bd.sample_workspace(P, V)
    bd.diffusion_canvas_init(canvas, prev, frozen, state, vocab, seed, 0)
    c_o = oloop.init_canvas(P, vocab, seed, 0)
    p_o = c_o.copy()
    f_o = np.zeros(P, dtype=np.uint8)
    s_o = np.zeros(4, dtype=np.int64)
    excused = 0
    for step in range(max_steps + 2):
        x = logits_for_step(step)
        lg = torch.from_numpy(x).cuda()
        if rule == "entropy":
            bd.diffusion_sample_step(lg, temperature, param, seed, step, frozen, canvas, tok, stat,
                                     acc, cnt, ws)
        else:
            bd.diffusion_sample_step_confidence(lg, temperature, param, seed, step, frozen, canvas,
                                                tok, stat, acc, cnt, ws)
        bd.diffusion_loop_update(tok, canvas, prev, frozen, state, threshold, max_steps)
        torch.cuda.synchronize()
        t_np, st_np = tok.cpu().numpy(), stat.cpu().numpy()
        was_frozen = f_o.copy()
        if s_o[oloop.DONE]:
            # the sampler still runs (it has no done gate); the driver state must not move
            assert np.array_equal(state.cpu().numpy(), s_o)
            break
        rows = [p for p in range(P) if not was_frozen[p]]
        excused += check_tokens_sampled(x, t_np, temperature, seed, step, rows=rows,
                                        frozen=was_frozen)
        if rule == "entropy":
            mask, n = osamp.accept(st_np, param, was_frozen)
        else:
            mask, n = osamp.accept_confidence(st_np, param, was_frozen)
        assert int(cnt.item()) == n and np.array_equal(acc.cpu().numpy(), mask), f"step {step}"
        c_o[mask == 1] = t_np[mask == 1]
        f_o = np.maximum(f_o, mask)
        oloop.loop_update(t_np.astype(np.int64), c_o, p_o, f_o, s_o, threshold, max_steps)
        assert np.array_equal(frozen.cpu().numpy(), f_o), f"step {step}: frozen"
        assert np.array_equal(canvas.cpu().numpy(), c_o), f"step {step}: canvas"
        assert np.array_equal(prev.cpu().numpy(), p_o), f"step {step}: prev"
        assert np.array_equal(state.cpu().numpy(), s_o), f"step {step}: state {state.cpu().numpy()} vs {s_o}"
    assert s_o[oloop.DONE]
    return int(s_o[oloop.STEP]), excused


def test_argmax_block_ends_on_stability(bd):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((64, 4096)) * 2).astype(np.float32)
    say("loop: T=0 entropy-bound, stable drafts")
    steps, _ = run_block(bd, lambda s: x, 0.0, "entropy", 1.0, threshold=3, max_steps=48)
    assert steps == 4    # random canvas -> drafts at step 1, then 3 unchanged steps


def test_sampled_block_runs_to_budget_or_all_frozen(bd):
    rng = np.random.default_rng(22)
    base = rng.standard_normal((48, 2048)).astype(np.float32)
    idx = rng.integers(0, 2048, 48)
    base[np.arange(48), idx] += rng.uniform(0, 26, 48).astype(np.float32)
    say("loop: T=1 entropy-bound, drifting logits")
    steps, excused = run_block(bd, lambda s: base + np.float32(0.05 * s), 1.0, "entropy", 2.0,
                               threshold=4, max_steps=12, seed=5)
    assert excused == 0 and 1 <= steps <= 12


def test_confidence_block(bd):
    rng = np.random.default_rng(23)
    base = rng.standard_normal((40, 3000)).astype(np.float32)
    base[np.arange(40), rng.integers(0, 3000, 40)] += rng.uniform(0, 20, 40).astype(np.float32)
    say("loop: T=0.7 confidence-threshold")
    steps, excused = run_block(bd, lambda s: base, 0.7, "confidence", 0.9, threshold=2,
                               max_steps=30, seed=8, vocab=3000)
    assert excused == 0 and steps <= 30


def test_drafts_off_and_finished_block_is_left_alone(bd):
    import torch
    P = 10
    canvas = torch.arange(P, dtype=torch.int32, device="cuda")
    prev = canvas.clone()
    frozen = torch.zeros(P, dtype=torch.uint8, device="cuda")
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    tok = torch.full((P,), 99, dtype=torch.int32, device="cuda")
    say("loop: drafts off")
    bd.diffusion_loop_update(tok, canvas, prev, frozen, state, 2, 48, write_drafts=False)
    bd.diffusion_loop_update(tok, canvas, prev, frozen, state, 2, 48, write_drafts=False)
    torch.cuda.synchronize()
    assert np.array_equal(canvas.cpu().numpy(), np.arange(P))
    assert list(state.cpu().numpy()) == [2, 2, 1, 0]
    bd.diffusion_loop_update(tok, canvas, prev, frozen, state, 2, 48)   # done: no-op
    torch.cuda.synchronize()
    assert np.array_equal(canvas.cpu().numpy(), np.arange(P))
    assert list(state.cpu().numpy()) == [2, 2, 1, 0]


def test_full_size_block_in_lockstep(bd):
    """The sampler workload's logits ([256, 262144], T = 1, bound 2.0) driven for six steps
    (the budget), every step checked against the oracle: masks, canvas, frozen set, state."""
    from block_diffusion_lm_router_amd import workloads
    shape = workloads.SAMPLER
    x = workloads.make_logits(shape)
    say("loop: full-size block", x.shape)
    steps, excused = run_block(bd, lambda s: x, shape.temperature, "entropy", shape.bound,
                               threshold=3, max_steps=6, seed=shape.seed)
    assert steps == 6 and excused == 0
