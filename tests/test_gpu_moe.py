"""GPU parity of the MoE FFN (moe_route_topk / moe_w4a16_gate_up / moe_w4a16_down /
moe_w4a16_ffn / moe_combine_fixed_order) against the CPU oracle, through the C ABI.

Bars: top-k ids bit-exact; routing weights within fp32 rounding; per-assignment expert
outputs and combined outputs within 2e-2 abs + 1e-2 rel of the fp64 oracle; the combine
bit-identical across repeated runs.
"""

import numpy as np
import pytest

from block_diffusion_lm_router_amd import workloads
from oracle import moe as omoe
from gpu_common import check_ffn_close, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


class Layer:
    """One layer's inputs on the host and on the device."""

    def __init__(self, bd, shape, x=None, logits=None, weights=None, layer=0, affine=False):
        import torch
        self.shape = shape
        self.x = workloads.make_activations(shape) if x is None else x
        self.logits = workloads.make_router_logits(shape, layer) if logits is None else logits
        self.w_np = workloads.make_weights(shape, layer) if weights is None else weights
        # group sizes as the scale arrays' shapes imply (gate/up, down)
        self.groups = (shape.d_model // self.w_np["gate_up_scale"].shape[-1],
                       shape.d_ff // self.w_np["down_scale"].shape[-1])
        self.affine = affine
        self.w = bd.MoeWeights.from_numpy(self.w_np, shape.top_k, affine=affine)
        self.x_d = torch.from_numpy(self.x).cuda()
        self.logits_d = torch.from_numpy(self.logits).cuda()

    def run(self, bd, fused=True, prepared=True):
        """One FFN pass; prepared=True uses the packed streams (256-row GEMM tiles), False the
        raw nibble, scale and zero arrays (128-row tiles)."""
        import torch
        if prepared and self.w.packed is None:
            self.w.prepare()
        elif not prepared and self.w.packed is not None:
            self.w.unprepare()
        T, k, d = self.shape.tokens, self.shape.top_k, self.shape.d_model
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        o = torch.full((T, k, d), float("nan"), dtype=torch.float32, device="cuda")
        y = torch.empty((T, d), dtype=torch.float16, device="cuda")
        ws = bd.moe_workspace(T, self.w)
        if fused:
            bd.moe_w4a16_ffn(self.w, self.x_d, self.logits_d, ids, tw, o, ws)
        else:
            bd.moe_route_topk(self.w, self.logits_d, ids, tw, ws)
            bd.moe_w4a16_gate_up(self.w, self.x_d, ws)
            bd.moe_w4a16_down(self.w, T, o, ws)
        bd.moe_combine_fixed_order(o, tw, y)
        torch.cuda.synchronize()
        return ids.cpu().numpy(), tw.cpu().numpy(), o.cpu().numpy(), y.cpu().numpy()


def outputs_and_h_rounding_bound(layer, ids, rows):
    """Oracle expert outputs o[t, j] and the worst-case effect on them of storing the
    GeGLU activations h in fp16 (the MFMA operand precision): |W_down| @ |h| * 2^-11.  The
    affine form also rounds every weight to fp16 once (2^-11 relative): the down weights add
    the same bound again and the gate/up weights, through h, about as much once more."""
    T, k = ids.shape
    d = layer.shape.d_model
    o = np.full((T, k, d), np.nan)
    bound = np.full((T, k, d), np.nan)
    mask = np.zeros(T, dtype=bool)
    mask[rows] = True
    x64 = layer.x.astype(np.float64)
    for e in np.unique(ids[rows]):
        tt, jj = np.nonzero((ids == e) & mask[:, None])
        wg, wu, wd = omoe.expert_matrices(layer.w_np, int(e), *layer.groups, affine=layer.affine)
        o[tt, jj] = omoe.expert_ffn(x64[tt], wg, wu, wd)
        h = omoe.gelu_tanh(x64[tt] @ wg.T) * (x64[tt] @ wu.T)
        bound[tt, jj] = (np.abs(h) @ np.abs(wd.T)) * 2.0 ** -11 * (3.0 if layer.affine else 1.0)
    return o, bound


def check_layer(layer, got, tokens=None):
    """ids bit-exact; y (the fp16 FFN output) within 2e-2 + 1e-2|ref|; the fp32 per-assignment
    outputs within that plus the fp16 rounding bound of h, and rel-L2 <= 1e-3."""
    ids, tw, o, y = got
    ref_ids, ref_w = omoe.route_topk(layer.logits, layer.shape.top_k)
    assert np.array_equal(ids, ref_ids), "top-k ids differ"
    np.testing.assert_allclose(tw, ref_w, rtol=2e-6, atol=1e-7)
    rows = np.arange(layer.shape.tokens) if tokens is None else np.asarray(tokens)
    o_ref, o_bound = outputs_and_h_rounding_bound(layer, ref_ids, rows)
    err = np.abs(o[rows] - o_ref[rows])
    lim = 2e-2 + 1e-2 * np.abs(o_ref[rows]) + o_bound[rows]
    assert np.all(err <= lim), f"expert_out: {int((err > lim).sum())} outside; worst {(err / lim).max():.3g}"
    rel_l2 = np.sqrt(np.sum(err ** 2) / np.sum(o_ref[rows] ** 2))
    assert rel_l2 < 1e-3, f"expert_out rel-L2 {rel_l2:.3g}"
    y_ref = omoe.combine(o_ref[rows], ref_w[rows])
    # The affine form rounds every weight to fp16 once; its worst-case effect on the expert
    # outputs (o_bound) reaches y through the combine's weights.  The asymmetric form feeds
    # exact (q - z) to the MFMA and is held to the plain bar.
    extra = omoe.combine(o_bound[rows], ref_w[rows]) if layer.affine else 0.0
    return check_ffn_close(y[rows].astype(np.float64), y_ref, "y", extra=extra)


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
def test_tiny_layer(bd, prepared):
    say("tiny layer", prepared)
    layer = Layer(bd, workloads.TINY_LAYER)
    got = layer.run(bd, prepared=prepared)
    rel = check_layer(layer, got)
    assert rel < 2e-3
    got2 = layer.run(bd, fused=False, prepared=prepared)
    for a, b in zip(got, got2):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
@pytest.mark.parametrize("T,E,k,d,f", [(1, 4, 1, 128, 64), (3, 8, 3, 256, 192),
                                       (100, 4, 2, 128, 64), (77, 16, 4, 384, 128),
                                       (250, 2, 2, 128, 64)])
def test_ragged_buckets(bd, T, E, k, d, f, prepared):
    """Buckets of 1..T tokens: partial 16-row tiles, several 32-token items per expert;
    d_ff % 128 == 64 and d_model % 256 == 128 leave the last 256-row tile half empty."""
    shape = workloads.LayerShape(T, d, f, E, k)
    say("ragged buckets", T, E, k, d, f, prepared)
    layer = Layer(bd, shape, layer=T + E)
    check_layer(layer, layer.run(bd, prepared=prepared))


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
@pytest.mark.parametrize("T,E,k,d,f", [(96, 16, 4, 1024, 640), (200, 8, 2, 768, 576),
                                       (512, 8, 8, 640, 576), (2048, 4, 4, 640, 576),
                                       (33, 128, 8, 2816, 704)])
def test_larger_shapes(bd, T, E, k, d, f, prepared):
    """Odd group counts (576, 704: a half last stage), ragged 256-row tiles (640, 576),
    experts with many 32-token items, ragged items, the full expert shape."""
    shape = workloads.LayerShape(T, d, f, E, k)
    say("larger shapes", T, E, k, d, f, prepared)
    layer = Layer(bd, shape, layer=7 + T % 5)
    check_layer(layer, layer.run(bd, prepared=prepared))


def packed_stream(w_np, which, d, f, E):
    """The packed stream moe_w4a16_prepare documents, rebuilt by re-indexing the raw arrays:
    [E][tiles][stages][18432 B], per stage the nibble runs of (wave, set, lane) and then the
    (scale, zero) pairs of (wave, row)."""
    name = "gate_up" if which == 0 else "down"
    q = w_np[name + "_q"]
    sc = w_np[name + "_scale"].view(np.uint16)
    ze = w_np[name + "_zero"].view(np.uint16)
    K = d if which == 0 else f
    R = 2 * f if which == 0 else d
    G, tiles = K // 64, (-(-f // 128) if which == 0 else -(-d // 256))
    NS = (G + 1) // 2

    def mrow(t, tr):
        if which == 0:
            col = 128 * t + (tr & 127)
            return (0 if tr < 128 else f) + col if col < f else -1
        row = 256 * t + tr
        return row if row < R else -1

    def tile_row(w, S, n):
        return 128 * S + 16 * w + n if which == 0 else 32 * w + 16 * S + n

    out = np.zeros((E, tiles, NS, 18432), dtype=np.uint8)
    for t in range(tiles):
        for s in range(NS):
            g0, g1 = 2 * s, 2 * s + 1
            for w in range(8):
                for S in range(2):
                    for l in range(64):
                        n, b = l % 16, l // 16
                        row = mrow(t, tile_row(w, S, n))
                        if row < 0:
                            continue
                        o = ((2 * w + S) * 64 + l) * 16
                        out[:, t, s, o:o + 8] = q[:, row, 32 * g0 + 8 * b:32 * g0 + 8 * b + 8]
                        if g1 < G:
                            out[:, t, s, o + 8:o + 16] = q[:, row, 32 * g1 + 8 * b:32 * g1 + 8 * b + 8]
                for n in range(16):
                    for S in range(2):
                        row = mrow(t, tile_row(w, S, n))
                        if row < 0:
                            continue
                        vals = [sc[:, row, g0], sc[:, row, g1] if g1 < G else 0 * sc[:, row, g0],
                                ze[:, row, g0], ze[:, row, g1] if g1 < G else 0 * ze[:, row, g0]]
                        o = 16384 + (16 * w + n) * 16 + 8 * S
                        out[:, t, s, o:o + 8] = np.stack(vals, axis=-1).astype(np.uint16).view(np.uint8)
    return out


@pytest.mark.parametrize("d,f,E", [(256, 128, 3), (384, 192, 2), (640, 576, 2)])
def test_packed_layout(bd, d, f, E):
    """moe_w4a16_prepare writes exactly the documented packed stream (bit-exact against a
    re-indexing of the raw arrays): odd group counts, ragged last tiles, both matrices."""
    import torch
    shape = workloads.LayerShape(4, d, f, E, 1)
    w_np = workloads.make_weights(shape, 5)
    say("packed layout", d, f, E)
    w = bd.MoeWeights.from_numpy(w_np, 1).prepare()
    torch.cuda.synchronize()
    for which in (0, 1):
        want = packed_stream(w_np, which, d, f, E)
        got = w.packed[which].cpu().numpy().reshape(want.shape)
        assert np.array_equal(got, want), f"matrix {which}: packed stream differs"


def test_packed_without_raw_arrays(bd):
    """With the packed streams attached the GEMMs never read the raw arrays: releasing them
    leaves the results bit-identical."""
    say("packed, raw arrays released")
    layer = Layer(bd, workloads.SHORT_LAYER)
    got = layer.run(bd, prepared=True)
    layer.w = bd.MoeWeights.from_numpy(layer.w_np, layer.shape.top_k, prepare=True, drop_raw=True)
    got2 = layer.run(bd, prepared=True)
    for a, b in zip(got, got2):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_single_expert_and_zero_input(bd):
    shape = workloads.LayerShape(40, 256, 128, 1, 1)
    say("single expert / zero input")
    layer = Layer(bd, shape, logits=np.zeros((40, 1), dtype=np.float32), layer=3)
    check_layer(layer, layer.run(bd))
    zero = Layer(bd, shape, x=np.zeros((40, 256), dtype=np.float16),
                 logits=np.zeros((40, 1), dtype=np.float32), layer=3)
    _, _, o, y = zero.run(bd)
    assert np.all(o == 0) and np.all(y == 0)


def test_router_ties_take_lower_expert(bd):
    shape = workloads.LayerShape(16, 128, 64, 8, 3)
    logits = np.zeros((16, 8), dtype=np.float32)
    logits[:, 5] = 1.0
    logits[3, [1, 6]] = 1.0
    logits[7, :] = -0.0
    say("router ties")
    layer = Layer(bd, shape, logits=logits, layer=1)
    check_layer(layer, layer.run(bd))


def test_combine_bit_identical_and_within_fp16_rounding(bd):
    import torch
    rng = np.random.default_rng(4)
    T, k, d = 200, 8, 2816
    o = torch.from_numpy(rng.standard_normal((T, k, d)).astype(np.float32) * 30).cuda()
    w = torch.from_numpy(rng.random((T, k)).astype(np.float32)).cuda()
    say("combine repeat")
    outs = []
    for _ in range(5):
        y = torch.empty((T, d), dtype=torch.float16, device="cuda")
        bd.moe_combine_fixed_order(o, w, y)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    for y in outs[1:]:
        assert np.array_equal(y.view(np.uint16), outs[0].view(np.uint16))
    o_np, w_np = o.cpu().numpy().astype(np.float64), w.cpu().numpy().astype(np.float64)
    ref = omoe.combine(o_np, w_np)
    y = outs[0].astype(np.float64)
    # one fp16 rounding (half an ulp of the result) plus k fp32 roundings of the running sum
    half_ulp = 0.5 * np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    fp32_sum = 2.0 ** -24 * k * np.einsum("tj,tjd->td", np.abs(w_np), np.abs(o_np))
    assert np.all(np.abs(y - ref) <= half_ulp * 1.0001 + fp32_sum)


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
def test_full_layer_every_token(bd, prepared):
    """Full shape (256 tokens, 128 experts, top-8, uniform routing): ids, every expert-output
    row and every combined row against the oracle."""
    say("full layer", prepared)
    layer = Layer(bd, workloads.LAYER)
    got = layer.run(bd, prepared=prepared)
    check_layer(layer, got)


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
def test_short_zipf_layer(bd, prepared):
    """64 tokens with Zipf-skewed routing: small and large buckets in one launch; every row
    against the oracle."""
    say("short zipf layer", prepared)
    layer = Layer(bd, workloads.SHORT_LAYER)
    got = layer.run(bd, prepared=prepared)
    counts = np.bincount(got[0].ravel(), minlength=128)
    assert counts.max() > bd.BD_MOE_ITEM_TOKENS   # the hottest expert spans several work items
    check_layer(layer, got)


@pytest.mark.parametrize("layer_id", [0, 29])
def test_stack_layer_bench_config(bd, layer_id):
    """A layer of the benchmark stack in the benchmark's launch configuration (packed streams,
    raw arrays released; 256 tokens, Zipf routing, the hottest expert split over several work
    items): ids, every expert-output row and every combined row against the oracle."""
    shape = workloads.STACK_LAYER
    say("stack layer bench config", layer_id)
    layer = Layer(bd, shape, layer=layer_id)
    layer.w = bd.MoeWeights.from_numpy(layer.w_np, shape.top_k, prepare=True, drop_raw=True)
    got = layer.run(bd, prepared=True)
    ids = got[0]
    counts = np.bincount(ids.ravel(), minlength=shape.experts)
    assert counts.max() > 2 * bd.BD_MOE_ITEM_TOKENS   # several work items for one expert
    check_layer(layer, got)


def routing_state(bd, ws, T, E, k):
    """(offsets, items, perm) read back from a workspace after moe_route_topk, at the offsets
    include/bdstep.h documents for the routing state."""
    A = T * k
    up = lambda n: (n + 255) // 256 * 256
    max_items = A // bd.BD_MOE_ITEM_TOKENS + min(E, A)
    raw = ws.cpu().numpy()
    o_items = up(4 * (E + 1))
    o_perm = o_items + up(4 * (1 + 3 * max_items))
    offsets = raw[:4 * (E + 1)].view(np.int32)
    items_all = raw[o_items:o_items + 4 * (1 + 3 * max_items)].view(np.int32)
    n = int(items_all[0])
    assert 0 <= n <= max_items
    items = items_all[1:1 + 3 * n].reshape(n, 3)
    perm = raw[o_perm:o_perm + 4 * A].view(np.int32)
    return offsets, items, perm


def stable_bucketing(ids, E, item_tokens):
    """The bucketing written out plainly: a stable counting sort of the assignments (t, j),
    in token order, by expert; the offsets are the exclusive prefix of the counts, and each
    expert's bucket is cut into consecutive work items of at most item_tokens positions."""
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[ids[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm = np.zeros(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            perm[fill[e]] = t * k + j
            fill[e] += 1
    items = []
    for e in range(E):
        for q in range(0, int(counts[e]), item_tokens):
            items.append((e, int(offsets[e]) + q, min(item_tokens, int(counts[e]) - q)))
    return offsets, np.array(items, dtype=np.int64).reshape(-1, 3), perm


@pytest.mark.parametrize("which", ["layer", "stack", "short", "widest", "ragged"])
def test_bucket_contents_bit_exact(bd, which):
    """The routing state the GEMMs consume (expert offsets, work list, bucket permutation) is
    bit-exact against a stable counting sort of the oracle's top-k ids."""
    import torch
    shapes = {"layer": (workloads.LAYER, 0), "stack": (workloads.STACK_LAYER, 7),
              "short": (workloads.SHORT_LAYER, 3),
              "widest": (workloads.LayerShape(1500, 128, 64, 256, 16), 11),
              "ragged": (workloads.LayerShape(77, 384, 128, 16, 4), 2)}
    shape, lid = shapes[which]
    T, E, k = shape.tokens, shape.experts, shape.top_k
    logits = workloads.make_router_logits(shape, lid)
    say("bucket contents", which)
    w = bd.MoeWeights.from_numpy(workloads.make_weights(
        workloads.LayerShape(T, 128, 64, E, k), 0), k)  # only the routing shape matters here
    ws = torch.full((bd.moe_workspace_size(T, w),), 0xA5, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    bd.moe_route_topk(w, torch.from_numpy(logits).cuda(), ids, tw, ws)
    torch.cuda.synchronize()
    ref_ids, _ = omoe.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    offsets, items, perm = routing_state(bd, ws, T, E, k)
    r_off, r_items, r_perm = stable_bucketing(ref_ids, E, bd.BD_MOE_ITEM_TOKENS)
    assert np.array_equal(offsets, r_off), "expert offsets differ"
    assert np.array_equal(perm, r_perm), "bucket permutation differs"
    assert np.array_equal(items, r_items), "work list differs"


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
def test_widest_routing(bd, prepared):
    """256 experts, top-16, 1500 tokens: the largest expert count and k the ABI accepts, and a
    bucketing that takes two token passes; small expert matrices keep the oracle quick."""
    shape = workloads.LayerShape(1500, 128, 64, 256, 16)
    say("widest routing", prepared)
    layer = Layer(bd, shape, layer=11)
    got = layer.run(bd, prepared=prepared)
    assert not np.isnan(got[2]).any()
    check_layer(layer, got)


# ---------------------------------------------------------------- checkpoint format groups


def test_group128_packed_streams(bd):
    """Repacking 128-groups.  Down: the stream of the same weights written as 64-groups whose
    pairs share a scale and zero-point, byte for byte.  Gate/up: the compact stream, whose
    17,408-byte stages hold the same 16 KB of nibbles and then, for (w, n) = 0..127, the
    (scale, zero) of tile row R(w, 0, n) and of R(w, 1, n), i.e. the duplicated stream with
    each 128-group's scale and zero-point kept once."""
    import torch
    shape = workloads.LayerShape(8, 512, 256, 3, 2)
    w128 = workloads.make_weights(shape, 3, gate_up_group=128, down_group=128)
    w64 = dict(w128)
    for k in ("gate_up_scale", "gate_up_zero", "down_scale", "down_zero"):
        w64[k] = np.ascontiguousarray(np.repeat(w128[k], 2, axis=-1))
    say("group-128 packing")
    a = bd.MoeWeights.from_numpy(w128, 2, prepare=True)
    b = bd.MoeWeights.from_numpy(w64, 2, prepare=True)
    assert (a.group_size, a.down_group_size, b.group_size) == (128, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(a.packed[1], b.packed[1])
    dup = b.packed[0].cpu().numpy().reshape(-1, 18432)
    got = a.packed[0].cpu().numpy()
    assert got.size == dup.shape[0] * 17408
    got = got.reshape(-1, 17408)
    assert np.array_equal(got[:, :16384], dup[:, :16384])
    sz = dup[:, 16384:].view(np.uint16).reshape(-1, 128, 8)     # (w, n): A s0 s1 z0 z1, B ...
    want = sz[:, :, [0, 2, 4, 6]]                                # A s z, B s z
    assert np.array_equal(got[:, 16384:].view(np.uint16).reshape(-1, 128, 4), want)
    assert np.array_equal(sz[:, :, [1, 3, 5, 7]], want)          # the duplicates it drops


@pytest.mark.parametrize("which", ["tiny", "layer"])
def test_checkpoint_format_layer(bd, which):
    """gate/up grouped at 128, down at 64 (the checkpoint format) through the packed streams:
    ids bit-exact, outputs within the FFN bar on every token (tiny and full shape); the raw-array GEMM refuses the 128-groups."""
    shape = workloads.TINY_LAYER if which == "tiny" else workloads.LAYER
    w_np = workloads.make_weights(shape, 5, gate_up_group=128, down_group=64)
    say("checkpoint format", which)
    layer = Layer(bd, shape, weights=w_np)
    assert layer.groups == (128, 64)
    check_layer(layer, layer.run(bd, prepared=True))
    layer.w.unprepare()
    with pytest.raises(bd.BdError):
        layer.run(bd, prepared=False)


# ---------------------------------------------------------------- affine weight form


@pytest.mark.parametrize("which", ["tiny", "tiny_g128", "layer"])
def test_affine_layer(bd, which):
    """The affine form (w = q s + b, free fp16 bias) through the packed streams: ids bit-exact,
    outputs within the FFN bar on every token (tiny and full shapes);
    the raw-array GEMM refuses it.  tiny_g128 groups both matrices at 128 (the repacking
    spreads a 128-group's bias like its zero-point)."""
    shape = workloads.LAYER if which == "layer" else workloads.TINY_LAYER
    g = 128 if which == "tiny_g128" else None
    w_np = workloads.make_weights(shape, 2, gate_up_group=g, down_group=g, affine=True)
    say("affine layer", which)
    layer = Layer(bd, shape, weights=w_np, affine=True)
    check_layer(layer, layer.run(bd, prepared=True))
    layer.w.unprepare()
    with pytest.raises(bd.BdError):
        layer.run(bd, prepared=False)


def test_affine_with_exact_bias_matches_the_asymmetric_form(bd):
    """b = -z s with power-of-two scales makes every fp16 weight q s + b exact, so the affine
    path must agree with the asymmetric one up to fp32 summation order."""
    shape = workloads.LayerShape(96, 512, 256, 8, 2)
    w_np = workloads.make_weights(shape, 4)
    rng = np.random.default_rng(5)
    for kind in ("gate_up", "down"):
        sc = w_np[kind + "_scale"]
        w_np[kind + "_scale"] = (np.float16(2.0) ** -rng.integers(5, 8, sc.shape)).astype(np.float16)
    aff = dict(w_np)
    for kind in ("gate_up", "down"):
        aff[kind + "_zero"] = (-(w_np[kind + "_zero"].astype(np.float64)
                                 * w_np[kind + "_scale"].astype(np.float64))).astype(np.float16)
        assert np.array_equal(aff[kind + "_zero"].astype(np.float64),
                              -(w_np[kind + "_zero"].astype(np.float64) * w_np[kind + "_scale"].astype(np.float64)))
    say("affine exact bias")
    a = Layer(bd, shape, weights=w_np)
    b = Layer(bd, shape, weights=aff, x=a.x, logits=a.logits, affine=True)
    ga = a.run(bd, prepared=True)
    gb = b.run(bd, prepared=True)
    assert np.array_equal(ga[0], gb[0])
    o_a, o_b = ga[2].astype(np.float64), gb[2].astype(np.float64)
    scale = np.sqrt(np.mean(o_a ** 2))
    assert np.max(np.abs(o_a - o_b)) <= 1e-5 * scale + 2.0 ** -11 * np.max(np.abs(o_a))


# ---------------------------------------------------------------- full-shape determinism


@pytest.mark.parametrize("which", ["layer", "stack"])
def test_full_shape_repeats_bit_identical(bd, which):
    """The full layer (uniform routing) and a Zipf stack layer in the benchmark's launch
    configuration (packed streams, raw arrays released), ten runs each: top-k ids and
    weights, every expert output and the combined y bit-identical from run to run (a 1-ulp
    change could flip an acceptance and fork the denoising trajectory)."""
    shape = workloads.LAYER if which == "layer" else workloads.STACK_LAYER
    say("full-shape repeats", which)
    layer = Layer(bd, shape, layer=0 if which == "layer" else 5)
    layer.w = bd.MoeWeights.from_numpy(layer.w_np, shape.top_k, prepare=True, drop_raw=True)
    first = layer.run(bd, prepared=True)
    assert not np.isnan(first[2]).any()
    for rep in range(9):
        got = layer.run(bd, prepared=True, fused=(rep % 2 == 0))
        for a, b in zip(first, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"run {rep + 2} differs"


# ---------------------------------------------------------------- wide expert ffn (d_ff > 1024)


@pytest.mark.parametrize("prepared", [False, True], ids=["tile128", "packed256"])
@pytest.mark.parametrize("f", [1216, 2048])
def test_wide_expert_ffn(bd, f, prepared):
    """d_ff above 1024: the down GEMM's activation rows no longer fit LDS, so the packed path
    streams them per stage (the non-resident kernel); 1216 has an odd group count (19)."""
    shape = workloads.LayerShape(48, 256, f, 6, 2)
    say("wide expert ffn", f, prepared)
    layer = Layer(bd, shape, layer=f % 7)
    check_layer(layer, layer.run(bd, prepared=prepared))
