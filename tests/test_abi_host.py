"""Host-side checks of libbdstep (no GPU needed): the shared library loads, exports every
function include/bdstep.h declares, and its argument validation rejects bad calls before
anything is enqueued."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bdstep.h")


@pytest.fixture(scope="module")
def lib():
    from block_diffusion_lm_router_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from block_diffusion_lm_router_amd import build
        build.build()
    return _binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for required in ("moe_w4a16_ffn", "moe_combine_fixed_order", "diffusion_sample_step",
                     "moe_route_topk", "moe_w4a16_gate_up", "moe_w4a16_down",
                     "diffusion_sample_entropy", "diffusion_accept_entropy_bound"):
        assert required in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    from block_diffusion_lm_router_amd import _binding
    names = declared_functions()
    assert len(names) >= 13
    for name in names:
        assert hasattr(lib, name), f"{name} declared but not exported"
        assert name in _binding.SIGNATURES, f"{name} has no binding signature"
    assert set(_binding.SIGNATURES) == set(names)


def test_workspace_size_under_both_names(lib):
    w = _weights()
    for T in (1, 64, 256, 4096):
        n = lib.bd_moe_workspace_size(T, ctypes.byref(w))
        assert n > 0 and lib.bd_moe_w4a16_ffn_workspace_size(T, ctypes.byref(w)) == n
    assert lib.bd_moe_w4a16_ffn_workspace_size(0, ctypes.byref(w)) == 0


def test_header_constants_match_the_binding():
    from block_diffusion_lm_router_amd import _binding
    text = open(HEADER).read()
    for name in ("BD_MOE_ITEM_TOKENS", "BD_SAMPLE_CHUNK"):
        value = int(re.search(rf"#define {name} (\d+)", text).group(1))
        assert getattr(_binding, name) == value, name


def test_version_and_status_strings(lib):
    version = int(re.search(r"#define BD_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.bd_abi_version() == version
    for s in range(7):
        assert len(lib.bd_status_string(s)) > 0
    assert lib.bd_status_string(99) == b"unknown status"


def _weights(E=128, k=8, d=2816, f=704, g=64, ptr=0x1000, gd=0, fmt=0):
    from block_diffusion_lm_router_amd._binding import MoeWeightsC
    p = ctypes.c_void_p(ptr)
    return MoeWeightsC(E, k, d, f, g, p, p, p, p, p, p, None, None, gd, fmt)


def test_moe_workspace_size(lib):
    w = _weights()
    n = lib.bd_moe_workspace_size(256, ctypes.byref(w))
    A = 256 * 8
    assert n >= A * 704 * 2 + A * 4 + 129 * 4
    assert lib.bd_moe_workspace_size(0, ctypes.byref(w)) == 0
    bad = _weights(g=128)
    assert lib.bd_moe_workspace_size(256, ctypes.byref(bad)) == 0
    assert lib.bd_moe_workspace_size(256, None) == 0


@pytest.mark.parametrize("kw,T,code", [
    (dict(), 0, 2), (dict(), 65537, 2), (dict(E=0), 4, 2), (dict(E=257), 4, 2),
    (dict(k=0), 4, 2), (dict(k=17), 4, 2), (dict(E=4, k=5), 4, 2),
    (dict(g=32), 4, 5), (dict(g=128, gd=256), 4, 5), (dict(d=2880), 4, 5), (dict(f=700), 4, 5),
    (dict(g=128, d=2880 - 64), 4, 2), (dict(gd=128), 4, 2), (dict(fmt=2), 4, 5),
])
def test_moe_shape_validation(lib, kw, T, code):
    w = _weights(**kw)
    P = ctypes.c_void_p(0x1000)
    assert lib.moe_route_topk(ctypes.byref(w), T, P, P, P, P, 1 << 40, None) == code


def test_moe_pointer_and_workspace_validation(lib):
    w = _weights()
    P = ctypes.c_void_p(0x1000)
    need = lib.bd_moe_workspace_size(256, ctypes.byref(w))
    assert lib.moe_route_topk(ctypes.byref(w), 256, None, P, P, P, need, None) == 1
    assert lib.moe_route_topk(ctypes.byref(w), 256, P, P, P, None, need, None) == 1
    assert lib.moe_route_topk(ctypes.byref(w), 256, P, P, P, P, need - 1, None) == 4
    assert lib.moe_route_topk(ctypes.byref(w), 256, ctypes.c_void_p(0x1002), P, P, P, need, None) == 3
    assert lib.moe_w4a16_gate_up(ctypes.byref(w), 256, ctypes.c_void_p(0x1008), P, need, None) == 3
    assert lib.moe_w4a16_down(ctypes.byref(w), 256, P, ctypes.c_void_p(0x1004), need, None) == 3
    nulls = _weights(ptr=0)
    assert lib.moe_w4a16_gate_up(ctypes.byref(nulls), 256, P, P, need, None) == 1
    assert lib.moe_w4a16_ffn(ctypes.byref(w), 256, P, P, P, P, P, P, 16, None) == 4


def test_combine_validation(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.moe_combine_fixed_order(P, P, 4, 8, 2818, P, None) == 2
    assert lib.moe_combine_fixed_order(P, P, 4, 17, 2816, P, None) == 2
    assert lib.moe_combine_fixed_order(None, P, 4, 8, 2816, P, None) == 1
    assert lib.moe_combine_fixed_order(P, P, 4, 8, 2816, ctypes.c_void_p(0x1008), None) == 3


def test_sampler_validation(lib):
    P = ctypes.c_void_p(0x1000)
    n = lib.bd_sample_workspace_size(256, 262144)
    assert n >= 256 * 40          # one 40-byte partial state per split and row
    assert lib.bd_sample_workspace_size(0, 10) == 0
    assert lib.bd_sample_workspace_size(1025, 10) == 0
    assert lib.bd_sample_workspace_size(10, (1 << 24) + 1) == 0
    call = lib.diffusion_sample_entropy
    assert call(P, 256, 262144, -1.0, 0, 0, None, P, P, P, n, None) == 2
    assert call(P, 256, 262144, float("nan"), 0, 0, None, P, P, P, n, None) == 2
    assert call(P, 256, 262144, float("inf"), 0, 0, None, P, P, P, n, None) == 2
    assert call(P, 256, 262144, 1e-45, 0, 0, None, P, P, P, n, None) == 2   # 1/T overflows
    assert call(P, 256, 262144, 1.0, 0, 0, None, P, P, P, n - 1, None) == 4
    assert call(None, 256, 262144, 1.0, 0, 0, None, P, P, P, n, None) == 1
    assert call(ctypes.c_void_p(0x1004), 256, 262144, 1.0, 0, 0, None, P, P, P, n, None) == 3
    acc = lib.diffusion_accept_entropy_bound
    assert acc(P, P, 0, 1.0, None, None, P, P, None) == 2
    assert acc(P, P, 1025, 1.0, None, None, P, P, None) == 2
    assert acc(P, P, 8, float("nan"), None, None, P, P, None) == 2
    assert acc(P, P, 8, 1.0, None, None, None, P, None) == 1
    step = lib.diffusion_sample_step
    assert step(P, 8, 100, 1.0, float("inf"), 0, 0, None, None, P, P, P, P, P, 1 << 20, None) == 2
    assert lib.bd_hbm_copy(P, P, 17, None) == 2
    assert lib.bd_hbm_copy(None, P, 16, None) == 1
    assert lib.bd_hbm_read(P, 17, P, None) == 2
    assert lib.bd_hbm_read(None, 16, P, None) == 1
    assert lib.bd_hbm_read(P, 16, None, None) == 1
    assert lib.bd_hbm_read(ctypes.c_void_p(0x1004), 16, P, None) == 3


def test_confidence_sampler_validation(lib):
    import json
    opts = json.load(open(os.path.join(ROOT, "tests", "golden", "diffusion_options.json")))
    lo, hi = opts["confidence_threshold_range"]
    P = ctypes.c_void_p(0x1000)
    acc = lib.diffusion_accept_confidence
    # the documented range is accepted at both ends (the call then fails only on P = 0)
    assert acc(P, P, 0, lo, None, None, P, P, None) == 2
    assert acc(None, P, 8, lo, None, None, P, P, None) == 1
    assert acc(None, P, 8, hi, None, None, P, P, None) == 1
    assert acc(None, P, 8, opts["confidence_threshold_default"], None, None, P, P, None) == 1
    n = lib.bd_sample_workspace_size(256, 262144)
    call = lib.diffusion_sample_confidence
    assert call(P, 256, 262144, -1.0, 0, 0, None, P, None, P, P, n, None) == 2
    assert call(P, 256, 262144, 1.0, 0, 0, None, P, None, None, P, n, None) == 1
    assert call(P, 256, 262144, 1.0, 0, 0, None, P, None, P, P, n - 1, None) == 4
    assert call(P, 256, 262144, 1.0, 0, 0, None, P, ctypes.c_void_p(0x1002), P, P, n, None) == 3
    acc = lib.diffusion_accept_confidence
    for bad in (-0.01, 1.01, float("nan"), float("inf")):
        assert acc(P, P, 8, bad, None, None, P, P, None) == 2
    assert acc(P, P, 0, 0.9, None, None, P, P, None) == 2
    assert acc(P, P, 1025, 0.9, None, None, P, P, None) == 2
    assert acc(None, P, 8, 0.9, None, None, P, P, None) == 1
    assert acc(P, P, 8, 0.9, None, ctypes.c_void_p(0x1001), P, P, None) == 3
    step = lib.diffusion_sample_step_confidence
    assert step(P, 8, 100, 1.0, 1.5, 0, 0, None, None, P, P, P, P, P, 1 << 20, None) == 2
    assert step(P, 8, 100, 1.0, 0.9, 0, 0, None, None, P, None, P, P, P, 1 << 20, None) == 1


def test_norm_router_validation(lib):
    P = ctypes.c_void_p(0x1000)
    norm = lib.moe_rmsnorm
    assert norm(P, P, 0, 2816, 1e-6, P, None) == 2
    assert norm(P, P, 4, 2820, 1e-6, P, None) == 2
    assert norm(P, P, 4, 4104, 1e-6, P, None) == 2
    assert norm(P, P, 4, 2816, -1.0, P, None) == 2
    assert norm(P, P, 4, 2816, float("nan"), P, None) == 2
    assert norm(None, P, 4, 2816, 1e-6, P, None) == 1
    assert norm(P, ctypes.c_void_p(0x1008), 4, 2816, 1e-6, P, None) == 3
    rt = lib.moe_router_logits
    assert rt(P, P, 4, 2880, 128, P, None) == 2
    assert rt(P, P, 4, 2816, 0, P, None) == 2
    assert rt(P, P, 4, 2816, 257, P, None) == 2
    assert rt(P, P, 65537, 2816, 128, P, None) == 2
    assert rt(P, None, 4, 2816, 128, P, None) == 1
    assert rt(ctypes.c_void_p(0x1002), P, 4, 2816, 128, P, None) == 3


def test_combine_rmsnorm_validation(lib):
    """Every case fails a host check, so no kernel is launched on the placeholder pointers."""
    P = ctypes.c_void_p(0x1000)
    cn = lib.moe_combine_rmsnorm
    assert cn(P, P, 0, 8, 2816, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 0, 2816, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 17, 2816, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 8, 2820, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 8, 4104, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 8, 0, P, 1e-6, P, P, None) == 2
    assert cn(P, P, 4, 8, 2816, P, -1.0, P, P, None) == 2
    assert cn(P, P, 4, 8, 2816, P, float("nan"), P, P, None) == 2
    assert cn(None, P, 4, 8, 2816, P, 1e-6, P, P, None) == 1
    assert cn(P, P, 4, 8, 2816, None, 1e-6, P, P, None) == 1
    assert cn(P, P, 4, 8, 2816, P, 1e-6, P, None, None) == 1
    assert cn(ctypes.c_void_p(0x1004), P, 4, 8, 2816, P, 1e-6, P, P, None) == 3
    assert cn(P, P, 4, 8, 2816, ctypes.c_void_p(0x1008), 1e-6, P, P, None) == 3
    assert cn(P, P, 4, 8, 2816, P, 1e-6, P, ctypes.c_void_p(0x1008), None) == 3
    cg = lib.moe_combine_rmsnorm_gated
    assert cg(P, P, 4, 8, 2816, P, 1e-6, P, P, None, None) == 1
    assert cg(P, P, 4, 8, 2816, P, 1e-6, P, P, ctypes.c_void_p(0x1002), None) == 3
    assert cg(P, P, 0, 8, 2816, P, 1e-6, P, P, P, None) == 2


def test_loop_driver_validation(lib):
    from oracle import loop
    for args in [(256, 64, 0, 0), (256, 64, 12, 0), (256, 64, 100, 0), (256, 64, 999, 0),
                 (256, 64, 12, 1), (32, 64, 5, 0), (1, 1, 0, 0)]:
        assert lib.bd_canvas_length(*args) == loop.canvas_length(*args[:3], bool(args[3]))
    assert lib.bd_canvas_length(0, 64, 5, 0) == 0
    assert lib.bd_canvas_length(256, 0, 5, 0) == 0
    assert lib.bd_canvas_length(256, 64, -1, 0) == 0
    P = ctypes.c_void_p(0x1000)
    init = lib.diffusion_canvas_init
    assert init(P, P, P, P, 0, 100, 0, 0, None) == 2
    assert init(P, P, P, P, 1025, 100, 0, 0, None) == 2
    assert init(P, P, P, P, 8, 0, 0, 0, None) == 2
    assert init(P, P, P, P, 8, (1 << 24) + 1, 0, 0, None) == 2
    assert init(P, None, P, P, 8, 100, 0, 0, None) == 1
    assert init(P, P, P, ctypes.c_void_p(0x1002), 8, 100, 0, 0, None) == 3
    upd = lib.diffusion_loop_update
    assert upd(P, P, P, P, P, 8, 0, 48, 1, None) == 2
    assert upd(P, P, P, P, P, 8, 3, 0, 1, None) == 2
    assert upd(None, P, P, P, P, 8, 3, 48, 1, None) == 1
    assert upd(P, P, P, P, None, 8, 3, 48, 1, None) == 1
    assert upd(ctypes.c_void_p(0x1001), P, P, P, P, 8, 3, 48, 1, None) == 3


def test_prepare_sizes_and_validation(lib):
    w = _weights()
    ref = ctypes.byref(w)
    # [E][tiles][stages][18432 bytes]: gate/up 6 tiles of 128 columns x 22 stages, down 11
    # tiles of 256 rows x 6 stages (11 groups: the last stage holds one).
    assert lib.bd_moe_packed_size(ref, 0) == 128 * 6 * 22 * 18432
    assert lib.bd_moe_packed_size(ref, 1) == 128 * 11 * 6 * 18432
    assert lib.bd_moe_packed_size(ref, 2) == 0
    p = ctypes.c_void_p(0x1000)
    assert lib.moe_w4a16_prepare(ref, None, p, None) == 1              # BD_ERR_NULL
    assert lib.moe_w4a16_prepare(ref, ctypes.c_void_p(0x1008), p, None) == 3   # BD_ERR_ALIGN
    bad = _weights(g=32)
    assert lib.moe_w4a16_prepare(ctypes.byref(bad), p, p, None) == 5   # BD_ERR_UNSUPPORTED
    bad = _weights(g=128)                                              # down at 128: 704 % 128
    assert lib.moe_w4a16_prepare(ctypes.byref(bad), p, p, None) == 2   # BD_ERR_SHAPE
    # the checkpoint format (gate/up 128, down 64): the gate/up stream keeps one scale and
    # zero-point per 128-group (17,408-byte stages), the down stream is the 64-group one
    ck = _weights(g=128, gd=64)
    assert lib.bd_moe_packed_size(ctypes.byref(ck), 0) == 128 * 6 * 22 * 17408
    assert lib.bd_moe_packed_size(ctypes.byref(ck), 1) == 128 * 11 * 6 * 18432
    # a 128-group over raw arrays is refused by the GEMMs; with the packed stream it is not
    ws = ctypes.c_void_p(0x10000)
    assert lib.moe_w4a16_gate_up(ctypes.byref(ck), 256, p, ws, 1 << 30, None) == 5
    assert lib.moe_w4a16_down(ctypes.byref(_weights(g=64, gd=128, f=768)), 256, p, ws, 1 << 30,
                              None) == 5
    # the affine form over raw arrays is refused by the GEMMs (it needs the packed stream)
    aff = _weights(fmt=1)
    assert lib.bd_moe_packed_size(ctypes.byref(aff), 0) == 128 * 6 * 22 * 18432
    assert lib.moe_w4a16_gate_up(ctypes.byref(aff), 256, p, ws, 1 << 30, None) == 5
    assert lib.moe_w4a16_down(ctypes.byref(aff), 256, p, ws, 1 << 30, None) == 5
    # a misaligned packed stream is rejected by the GEMM entry points before any launch
    w.gate_up_packed = 0x1008
    ws = ctypes.c_void_p(0x10000)
    assert lib.moe_w4a16_gate_up(ref, 256, p, ws, 1 << 30, None) == 3


def test_noalloc_sampler_step_validation(lib):
    """The allocation-free sampler step validates like diffusion_sample_step and returns before
    any device work (no GPU needed for these)."""
    P = ctypes.c_void_p(0x1000)
    call = lib.diffusion_sample_step_noalloc
    assert call(P, 0, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, None) == 2
    assert call(P, 1025, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, None) == 2
    assert call(P, 8, 4096, float("nan"), 2.0, 0, 0, None, None, P, P, P, P, None) == 2
    assert call(P, 8, 4096, 1.0, float("inf"), 0, 0, None, None, P, P, P, P, None) == 2
    assert call(None, 8, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, None) == 1
    assert call(P, 8, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, None, None) == 1
    assert call(ctypes.c_void_p(0x1004), 8, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P,
                None) == 3


def test_gated_entry_points_validate_the_gate(lib):
    """The gated variants need a device loop state (NULL or misaligned is refused before any
    device work) and otherwise validate like their ungated forms."""
    P = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    w = _weights()
    need = lib.bd_moe_workspace_size(256, ctypes.byref(w))
    ffn = lib.moe_w4a16_ffn_gated
    assert ffn(ctypes.byref(w), 256, P, P, P, P, P, P, need, None, None) == 1
    assert ffn(ctypes.byref(w), 256, P, P, P, P, P, P, need, odd, None) == 3
    assert ffn(ctypes.byref(w), 0, P, P, P, P, P, P, need, P, None) == 2
    comb = lib.moe_combine_fixed_order_gated
    assert comb(P, P, 4, 8, 2816, P, None, None) == 1
    assert comb(P, P, 4, 8, 2818, P, P, None) == 2
    n = lib.bd_sample_workspace_size(64, 4096)
    step = lib.diffusion_sample_step_gated
    assert step(P, 64, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, P, n, None, None) == 1
    assert step(P, 64, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, P, n, odd, None) == 3
    assert step(P, 0, 4096, 1.0, 2.0, 0, 0, None, None, P, P, P, P, P, n, P, None) == 2
    conf = lib.diffusion_sample_step_confidence_gated
    assert conf(P, 64, 4096, 1.0, 0.9, 0, 0, None, None, P, P, P, P, P, n, None, None) == 1
    assert conf(P, 64, 4096, 1.0, 1.5, 0, 0, None, None, P, P, P, P, P, n, P, None) == 2
    norm = lib.moe_rmsnorm_gated
    assert norm(P, P, 256, 2816, ctypes.c_float(1e-6), P, None, None) == 1
    assert norm(P, P, 256, 2816, ctypes.c_float(1e-6), P, odd, None) == 3
    assert norm(P, P, 256, 2817, ctypes.c_float(1e-6), P, P, None) == 2
    assert norm(P, P, 256, 2816, ctypes.c_float(-1.0), P, P, None) == 2
    router = lib.moe_router_logits_gated
    assert router(P, P, 256, 2816, 128, P, None, None) == 1
    assert router(P, P, 256, 2816, 128, P, odd, None) == 3
    assert router(P, P, 256, 2880, 128, P, P, None) == 2
    assert router(None, P, 256, 2816, 128, P, P, None) == 1
