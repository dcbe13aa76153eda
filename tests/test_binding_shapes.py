"""CPU-only: every wrapper of the binding checks tensor shapes against what the kernels assume
and raises ValueError before any pointer is passed on (the C ABI receives only pointers, so
a mis-shaped tensor would otherwise become an out-of-bounds access on the device)."""

import numpy as np
import pytest
import torch

from block_diffusion_lm_router_amd import _binding as bd


class StubWeights:
    """The attributes the wrappers read from MoeWeights (no device memory)."""
    num_experts, top_k, d_model, d_ff = 8, 2, 256, 128

    def ref(self):
        raise AssertionError("the shape check must fail before the weights are marshalled")


W = StubWeights()
T = 16


def t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def expect(fn, *args):
    with pytest.raises(ValueError, match="shape|elements|must be"):
        fn(*args)


def test_moe_wrappers_check_shapes():
    ws = t(64, dtype=torch.uint8)
    ids, tw = t(T, 2, dtype=torch.int32), t(T, 2)
    expect(bd.moe_route_topk, W, t(T, 7), ids, tw, ws)                 # E mismatch
    expect(bd.moe_route_topk, W, t(T, 8), t(T, 3, dtype=torch.int32), tw, ws)
    expect(bd.moe_route_topk, W, t(T, 8), ids, t(T + 1, 2), ws)
    expect(bd.moe_w4a16_gate_up, W, t(T, 255, dtype=torch.float16), ws)
    expect(bd.moe_w4a16_down, W, T, t(T, 2, 255), ws)
    expect(bd.moe_w4a16_down, W, T, t(T - 1, 2, 256), ws)
    x = t(T, 256, dtype=torch.float16)
    o = t(T, 2, 256)
    expect(bd.moe_w4a16_ffn, W, x, t(T, 8), ids, tw, t(T, 3, 256), ws)
    expect(bd.moe_w4a16_ffn, W, x, t(T + 1, 8), ids, tw, o, ws)
    expect(bd.moe_w4a16_ffn, W, t(T, 128, dtype=torch.float16), t(T, 8), ids, tw, o, ws)
    expect(bd.moe_combine_fixed_order, o, t(T, 3), t(T, 256, dtype=torch.float16))
    expect(bd.moe_combine_fixed_order, o, tw, t(T, 255, dtype=torch.float16))
    expect(bd.moe_combine_fixed_order, t(T, 256), tw, t(T, 256, dtype=torch.float16))
    h16, wn = t(T, 256, dtype=torch.float16), t(256, dtype=torch.float16)
    expect(bd.moe_combine_rmsnorm, o, t(T, 3), wn, h16, h16)                 # weights [T, k]
    expect(bd.moe_combine_rmsnorm, o, tw, wn, t(T, 255, dtype=torch.float16), h16)
    expect(bd.moe_combine_rmsnorm, o, tw, wn, h16, t(T + 1, 256, dtype=torch.float16))
    expect(bd.moe_combine_rmsnorm, o, tw, t(255, dtype=torch.float16), h16, h16)
    expect(bd.moe_combine_rmsnorm, t(T, 256), tw, wn, h16, h16)


def test_moe_weights_check_array_shapes():
    E, f, d = 2, 64, 128
    arrays = {"gate_up_q": t(E, 2 * f, d // 2, dtype=torch.uint8),
              "gate_up_scale": t(E, 2 * f, d // 64, dtype=torch.float16),
              "gate_up_zero": t(E, 2 * f, d // 64 + 1, dtype=torch.float16),   # wrong
              "down_q": t(E, d, f // 2, dtype=torch.uint8),
              "down_scale": t(E, d, f // 64, dtype=torch.float16),
              "down_zero": t(E, d, f // 64, dtype=torch.float16)}
    expect(bd.MoeWeights, arrays, 1)
    arrays["gate_up_zero"] = t(E, 2 * f, d // 64, dtype=torch.float16)
    arrays["down_q"] = t(E, d + 1, f // 2, dtype=torch.uint8)                 # wrong
    expect(bd.MoeWeights, arrays, 1)


def test_sampler_wrappers_check_shapes():
    P, V = 8, 64
    lg = t(P, V)
    ok_i, ok_f, ok_u = t(P, dtype=torch.int32), t(P), t(P, dtype=torch.uint8)
    bad_i, bad_f, bad_u = t(P + 1, dtype=torch.int32), t(P - 1), t(2 * P, dtype=torch.uint8)
    cnt, ws = t(1, dtype=torch.int32), t(64, dtype=torch.uint8)
    expect(bd.diffusion_sample_entropy, t(P * V), 1.0, 0, 0, None, ok_i, ok_f, ws)
    expect(bd.diffusion_sample_entropy, lg, 1.0, 0, 0, bad_u, ok_i, ok_f, ws)
    expect(bd.diffusion_sample_entropy, lg, 1.0, 0, 0, None, bad_i, ok_f, ws)
    expect(bd.diffusion_sample_entropy, lg, 1.0, 0, 0, None, ok_i, bad_f, ws)
    expect(bd.diffusion_accept_entropy_bound, ok_f, bad_i, 1.0, ok_u, ok_i, ok_u, cnt)
    expect(bd.diffusion_accept_entropy_bound, ok_f, ok_i, 1.0, ok_u, bad_i, ok_u, cnt)
    expect(bd.diffusion_accept_entropy_bound, ok_f, ok_i, 1.0, ok_u, ok_i, bad_u, cnt)
    expect(bd.diffusion_accept_entropy_bound, ok_f, ok_i, 1.0, ok_u, ok_i, ok_u,
           t(0, dtype=torch.int32))
    expect(bd.diffusion_sample_step, lg, 1.0, 2.0, 0, 0, ok_u, bad_i, ok_i, ok_f, ok_u, cnt, ws)
    expect(bd.diffusion_sample_step, lg, 1.0, 2.0, 0, 0, ok_u, ok_i, ok_i, ok_f, bad_u, cnt, ws)
    expect(bd.diffusion_sample_confidence, lg, 1.0, 0, 0, None, ok_i, None, bad_f, ws)
    expect(bd.diffusion_accept_confidence, bad_f, ok_i, 0.9, ok_u, ok_i, ok_u, cnt)
    expect(bd.diffusion_sample_step_confidence, lg, 1.0, 0.9, 0, 0, bad_u, ok_i, ok_i, ok_f,
           ok_u, cnt, ws)


def test_loop_wrappers_check_shapes():
    P = 8
    c, u = t(P, dtype=torch.int32), t(P, dtype=torch.uint8)
    st = t(4, dtype=torch.int32)
    expect(bd.diffusion_canvas_init, c, t(P + 1, dtype=torch.int32), u, st, 100, 0, 0)
    expect(bd.diffusion_canvas_init, c, c, u, t(3, dtype=torch.int32), 100, 0, 0)
    expect(bd.diffusion_loop_update, t(P - 1, dtype=torch.int32), c, c, u, st, 2, 8)
    expect(bd.diffusion_loop_update, c, c, c, t(P + 2, dtype=torch.uint8), st, 2, 8)


def test_shape_checks_run_before_the_gpu_checks():
    # a CPU tensor of the right shape passes the shape check and is then refused as not on
    # the GPU: the order of the checks is shape first
    with pytest.raises(ValueError, match="GPU tensor"):
        bd.moe_combine_fixed_order(t(T, 2, 256), t(T, 2), t(T, 256, dtype=torch.float16))
    assert np.isfinite(1.0)
