"""ctypes binding of libbdstep (see include/bdstep.h).  Argument marshalling only.

Every function takes torch tensors that live on the GPU, checks dtype, shape and
contiguity, and passes raw device pointers plus the current torch stream to the C
ABI.  No step of the hot path runs here: if the shared library is missing the
import of any entry point raises, there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdstep.so")

BD_SAMPLE_CHUNK = 1024
BD_MOE_ITEM_TOKENS = 32

_STATUS = {0: "ok", 1: "BD_ERR_NULL", 2: "BD_ERR_SHAPE", 3: "BD_ERR_ALIGN",
           4: "BD_ERR_WORKSPACE", 5: "BD_ERR_UNSUPPORTED", 6: "BD_ERR_HIP"}

# Every symbol the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32


class MoeWeightsC(ctypes.Structure):
    """Mirror of bd_moe_weights."""
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("gate_up_q", _P),
        ("gate_up_scale", _P),
        ("gate_up_zero", _P),
        ("down_q", _P),
        ("down_scale", _P),
        ("down_zero", _P),
        ("gate_up_packed", _P),
        ("down_packed", _P),
        ("down_group_size", ctypes.c_int32),
        ("format", ctypes.c_int32),
    ]


_W = ctypes.POINTER(MoeWeightsC)

SIGNATURES = {
    "bd_abi_version": (_I, []),
    "bd_status_string": (ctypes.c_char_p, [_I]),
    "bd_moe_workspace_size": (_SZ, [_I, _W]),
    "bd_moe_w4a16_ffn_workspace_size": (_SZ, [_I, _W]),
    "bd_moe_packed_size": (_SZ, [_W, _I]),
    "moe_w4a16_prepare": (_I, [_W, _P, _P, _P]),
    "moe_route_topk": (_I, [_W, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_w4a16_gate_up": (_I, [_W, _I, _P, _P, _SZ, _P]),
    "moe_w4a16_down": (_I, [_W, _I, _P, _P, _SZ, _P]),
    "moe_w4a16_ffn": (_I, [_W, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_w4a16_ffn_gated": (_I, [_W, _I, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "moe_combine_fixed_order": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moe_combine_fixed_order_gated": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "moe_combine_rmsnorm": (_I, [_P, _P, _I, _I, _I, _P, _F, _P, _P, _P]),
    "moe_combine_rmsnorm_gated": (_I, [_P, _P, _I, _I, _I, _P, _F, _P, _P, _P, _P]),
    "moe_rmsnorm": (_I, [_P, _P, _I, _I, _F, _P, _P]),
    "moe_rmsnorm_gated": (_I, [_P, _P, _I, _I, _F, _P, _P, _P]),
    "moe_router_logits": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moe_router_logits_gated": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "bd_sample_workspace_size": (_SZ, [_I, _I]),
    "diffusion_sample_entropy": (_I, [_P, _I, _I, _F, _U64, _U32, _P, _P, _P, _P, _SZ, _P]),
    "diffusion_accept_entropy_bound": (_I, [_P, _P, _I, _F, _P, _P, _P, _P, _P]),
    "diffusion_sample_step": (_I, [_P, _I, _I, _F, _F, _U64, _U32, _P, _P, _P, _P, _P, _P, _P,
                                   _SZ, _P]),
    "diffusion_sample_step_gated": (_I, [_P, _I, _I, _F, _F, _U64, _U32, _P, _P, _P, _P, _P, _P,
                                         _P, _SZ, _P, _P]),
    "diffusion_sample_step_noalloc": (_I, [_P, _I, _I, _F, _F, _U64, _U32, _P, _P, _P, _P, _P,
                                           _P, _P]),
    "diffusion_sample_confidence": (_I, [_P, _I, _I, _F, _U64, _U32, _P, _P, _P, _P, _P, _SZ,
                                         _P]),
    "diffusion_accept_confidence": (_I, [_P, _P, _I, _F, _P, _P, _P, _P, _P]),
    "diffusion_sample_step_confidence": (_I, [_P, _I, _I, _F, _F, _U64, _U32, _P, _P, _P, _P, _P,
                                              _P, _P, _SZ, _P]),
    "diffusion_sample_step_confidence_gated": (_I, [_P, _I, _I, _F, _F, _U64, _U32, _P, _P, _P,
                                                    _P, _P, _P, _P, _SZ, _P, _P]),
    "bd_canvas_length": (_I, [_I, _I, _I, _I]),
    "diffusion_canvas_init": (_I, [_P, _P, _P, _P, _I, _I, _U64, _U32, _P]),
    "diffusion_loop_update": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "bd_hbm_copy": (_I, [_P, _P, _SZ, _P]),
    "bd_hbm_read": (_I, [_P, _SZ, _P, _P]),
}

_lib = None


class BdError(RuntimeError):
    pass


def load():
    """Load libbdstep.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_diffusion_lm_router_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status, what):
    if status != 0:
        msg = load().bd_status_string(status).decode()
        raise BdError(f"{what}: {_STATUS.get(status, status)} ({msg})")


_binding_calls = False


def _invoke(name, *cargs):
    """Call entry point `name` with marshalled arguments and raise on a non-zero status.
    Under bind() the call is not made: the arguments are handed back instead."""
    if _binding_calls:
        return name, cargs
    _check(getattr(load(), name)(*cargs), name)


def bind(fn, *args, **kwargs):
    """Marshal the arguments of wrapper `fn` once (pointers, sizes, the current stream) and
    return a zero-argument callable that launches the entry point with them.  Repeated
    launches of the same call skip the per-call checks and conversions, which keeps the
    host ahead of the GPU when a loop issues many short launches."""
    global _binding_calls
    _binding_calls = True
    try:
        name, cargs = fn(*args, **kwargs)
    finally:
        _binding_calls = False
    raw = getattr(load(), name)

    def call():
        status = raw(*cargs)
        if status != 0:
            _check(status, name)
    return call


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name, what):
    """Raise ValueError unless tensor t has exactly `shape` (checked before any pointer is
    taken, so a mis-shaped tensor never reaches the kernels)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _gate(loop_state, what):
    """The marshalled loop-driver state of a gated call (int32, at least 4 elements)."""
    _at_least(loop_state, 4, "loop_state", what)
    return _ptr(loop_state, torch.int32, "loop_state")


def _at_least(t, n, name, what):
    if t is not None and t.numel() < n:
        raise ValueError(f"{what}: {name} needs at least {n} elements, got {t.numel()}")


class MoeWeights:
    """Device tensors of one layer's packed expert weights plus the C struct over them."""

    KEYS = ("gate_up_q", "gate_up_scale", "gate_up_zero", "down_q", "down_scale", "down_zero")

    def __init__(self, tensors, top_k, group_size=None, down_group_size=None, affine=False):
        """Group sizes default to what the scale arrays' shapes imply (d_model / groups of
        gate/up, d_ff / groups of down).  affine=True: the *_zero arrays hold the biases of the
        affine form w = q s + b (BD_FORMAT_AFFINE; the GEMMs then need prepare())."""
        self.tensors = tensors
        gq = tensors["gate_up_q"]
        E, two_f, half_d = gq.shape
        self.num_experts, self.d_ff, self.d_model = E, two_f // 2, half_d * 2
        if group_size is None:
            group_size = self.d_model // tensors["gate_up_scale"].shape[-1]
        if down_group_size is None:
            down_group_size = self.d_ff // tensors["down_scale"].shape[-1]
        self.top_k, self.group_size, self.down_group_size = top_k, group_size, down_group_size
        self.affine = affine
        E, f, d = self.num_experts, self.d_ff, self.d_model
        want = {"gate_up_q": (E, 2 * f, d // 2),
                "gate_up_scale": (E, 2 * f, d // group_size),
                "gate_up_zero": (E, 2 * f, d // group_size),
                "down_q": (E, d, f // 2),
                "down_scale": (E, d, f // down_group_size),
                "down_zero": (E, d, f // down_group_size)}
        for key, shape in want.items():
            _shape(tensors[key], shape, key, "MoeWeights")
        dtypes = {"gate_up_q": torch.uint8, "down_q": torch.uint8}
        ptrs = {k: _ptr(tensors[k], dtypes.get(k, torch.float16), k) for k in self.KEYS}
        self.c = MoeWeightsC(E, top_k, self.d_model, self.d_ff, group_size,
                             *[ptrs[k] for k in self.KEYS], None, None, down_group_size,
                             1 if affine else 0)
        self.packed = None

    def prepare(self, drop_raw=False):
        """Repack both matrices (moe_w4a16_prepare) and attach the packed streams, so the
        GEMMs use their 256-row tiles.  drop_raw=True then releases the raw arrays (the GEMMs
        no longer read them; the 128-row path is gone for this object).  Returns self."""
        lib = load()
        sizes = [lib.bd_moe_packed_size(self.ref(), m) for m in (0, 1)]
        if 0 in sizes:
            raise BdError("bd_moe_packed_size: invalid shape")
        dev = self.tensors["gate_up_q"].device
        self.packed = [torch.empty(n, dtype=torch.uint8, device=dev) for n in sizes]
        _check(lib.moe_w4a16_prepare(self.ref(), ctypes.c_void_p(self.packed[0].data_ptr()),
                                     ctypes.c_void_p(self.packed[1].data_ptr()), _stream()),
               "moe_w4a16_prepare")
        self.c.gate_up_packed = self.packed[0].data_ptr()
        self.c.down_packed = self.packed[1].data_ptr()
        if drop_raw:
            for k in self.KEYS:
                setattr(self.c, k, None)
            self.tensors = {}
        return self

    def unprepare(self):
        """Detach the packed streams (the GEMMs go back to their 128-row tiles)."""
        if not self.tensors:
            raise BdError("the raw weight arrays were released")
        self.c.gate_up_packed = None
        self.c.down_packed = None
        self.packed = None
        return self

    @classmethod
    def from_numpy(cls, arrays, top_k, device="cuda", group_size=None, prepare=False,
                   drop_raw=False, down_group_size=None, affine=False):
        t = {k: torch.from_numpy(arrays[k]).to(device) for k in cls.KEYS}
        w = cls(t, top_k, group_size, down_group_size, affine)
        return w.prepare(drop_raw=drop_raw) if prepare else w

    def ref(self):
        return ctypes.byref(self.c)


def abi_version():
    return load().bd_abi_version()


def moe_workspace_size(T, w: MoeWeights):
    n = load().bd_moe_workspace_size(T, w.ref())
    if n == 0:
        raise BdError("bd_moe_workspace_size: invalid shape")
    return n


def moe_workspace(T, w: MoeWeights, device="cuda"):
    return torch.zeros(moe_workspace_size(T, w), dtype=torch.uint8, device=device)


def moe_route_topk(w, router_logits, topk_ids, topk_weights, workspace):
    T = router_logits.shape[0]
    what = "moe_route_topk"
    _shape(router_logits, (T, w.num_experts), "router_logits", what)
    _shape(topk_ids, (T, w.top_k), "topk_ids", what)
    _shape(topk_weights, (T, w.top_k), "topk_weights", what)
    return _invoke("moe_route_topk", w.ref(), T,
                   _ptr(router_logits, torch.float32, "router_logits"),
                   _ptr(topk_ids, torch.int32, "topk_ids"),
                   _ptr(topk_weights, torch.float32, "topk_weights"),
                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())


def moe_w4a16_gate_up(w, x, workspace):
    _shape(x, (x.shape[0], w.d_model), "x", "moe_w4a16_gate_up")
    return _invoke("moe_w4a16_gate_up", w.ref(), x.shape[0], _ptr(x, torch.float16, "x"),
                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())


def moe_w4a16_down(w, T, expert_out, workspace):
    _shape(expert_out, (T, w.top_k, w.d_model), "expert_out", "moe_w4a16_down")
    return _invoke("moe_w4a16_down", w.ref(), T, _ptr(expert_out, torch.float32, "expert_out"),
                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())


def moe_w4a16_ffn(w, x, router_logits, topk_ids, topk_weights, expert_out, workspace,
                  loop_state=None):
    """loop_state (int32 [4]) selects moe_w4a16_ffn_gated: nothing runs once the loop is done."""
    T, what = x.shape[0], "moe_w4a16_ffn"
    _shape(x, (T, w.d_model), "x", what)
    _shape(router_logits, (T, w.num_experts), "router_logits", what)
    _shape(topk_ids, (T, w.top_k), "topk_ids", what)
    _shape(topk_weights, (T, w.top_k), "topk_weights", what)
    _shape(expert_out, (T, w.top_k, w.d_model), "expert_out", what)
    args = (w.ref(), x.shape[0], _ptr(x, torch.float16, "x"),
            _ptr(router_logits, torch.float32, "router_logits"),
            _ptr(topk_ids, torch.int32, "topk_ids"),
            _ptr(topk_weights, torch.float32, "topk_weights"),
            _ptr(expert_out, torch.float32, "expert_out"),
            _ptr(workspace, torch.uint8, "workspace"), workspace.numel())
    if loop_state is not None:
        return _invoke("moe_w4a16_ffn_gated", *args, _gate(loop_state, what), _stream())
    return _invoke("moe_w4a16_ffn", *args, _stream())


def moe_combine_fixed_order(expert_out, topk_weights, y, loop_state=None):
    if expert_out.dim() != 3:
        raise ValueError("moe_combine_fixed_order: expert_out must be [T, k, d]")
    T, k, d = expert_out.shape
    _shape(topk_weights, (T, k), "topk_weights", "moe_combine_fixed_order")
    _shape(y, (T, d), "y", "moe_combine_fixed_order")
    args = (_ptr(expert_out, torch.float32, "expert_out"),
            _ptr(topk_weights, torch.float32, "topk_weights"), T, k, d, _ptr(y, torch.float16, "y"))
    if loop_state is not None:
        return _invoke("moe_combine_fixed_order_gated", *args,
                       _gate(loop_state, "moe_combine_fixed_order"), _stream())
    return _invoke("moe_combine_fixed_order", *args, _stream())


def moe_combine_rmsnorm(expert_out, topk_weights, weight, y, xn, eps=1e-6, loop_state=None):
    """y = moe_combine_fixed_order(expert_out, topk_weights); xn = moe_rmsnorm(y, weight)."""
    if expert_out.dim() != 3:
        raise ValueError("moe_combine_rmsnorm: expert_out must be [T, k, d]")
    T, k, d = expert_out.shape
    _shape(topk_weights, (T, k), "topk_weights", "moe_combine_rmsnorm")
    _shape(y, (T, d), "y", "moe_combine_rmsnorm")
    _shape(xn, (T, d), "xn", "moe_combine_rmsnorm")
    if weight.numel() != d:
        raise ValueError("moe_combine_rmsnorm: weight must be [d]")
    args = (_ptr(expert_out, torch.float32, "expert_out"),
            _ptr(topk_weights, torch.float32, "topk_weights"), T, k, d,
            _ptr(weight, torch.float16, "weight"), float(eps), _ptr(y, torch.float16, "y"),
            _ptr(xn, torch.float16, "xn"))
    if loop_state is not None:
        return _invoke("moe_combine_rmsnorm_gated", *args,
                       _gate(loop_state, "moe_combine_rmsnorm"), _stream())
    return _invoke("moe_combine_rmsnorm", *args, _stream())


def moe_rmsnorm(h, weight, y, eps=1e-6, loop_state=None):
    T, d = h.shape
    if weight.numel() != d or tuple(y.shape) != (T, d):
        raise ValueError("moe_rmsnorm: weight must be [d] and y [T, d]")
    args = (_ptr(h, torch.float16, "h"), _ptr(weight, torch.float16, "weight"), T, d, float(eps),
            _ptr(y, torch.float16, "y"))
    if loop_state is not None:
        return _invoke("moe_rmsnorm_gated", *args, _gate(loop_state, "moe_rmsnorm"), _stream())
    return _invoke("moe_rmsnorm", *args, _stream())


def moe_router_logits(x, w_router, logits, loop_state=None):
    T, d = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != d or tuple(logits.shape) != (T, E):
        raise ValueError("moe_router_logits: w_router must be [E, d] and logits [T, E]")
    args = (_ptr(x, torch.float16, "x"), _ptr(w_router, torch.float16, "w_router"), T, d, E,
            _ptr(logits, torch.float32, "logits"))
    if loop_state is not None:
        return _invoke("moe_router_logits_gated", *args, _gate(loop_state, "moe_router_logits"),
                       _stream())
    return _invoke("moe_router_logits", *args, _stream())


def sample_workspace_size(P, V):
    n = load().bd_sample_workspace_size(P, V)
    if n == 0:
        raise BdError("bd_sample_workspace_size: invalid shape")
    return n


def sample_workspace(P, V, device="cuda"):
    return torch.zeros(sample_workspace_size(P, V), dtype=torch.uint8, device=device)


def _rows(what, P, **named):
    """Every named per-position tensor must be [P]."""
    for name, t in named.items():
        _shape(t, (P,), name, what)


def _logits_shape(logits, what):
    if logits.dim() != 2:
        raise ValueError(f"{what}: logits must be [P, V]")
    return logits.shape


def diffusion_sample_entropy(logits, temperature, seed, step, frozen, tokens_out, entropy_out,
                             workspace):
    P, V = _logits_shape(logits, "diffusion_sample_entropy")
    _rows("diffusion_sample_entropy", P, frozen=frozen, tokens_out=tokens_out,
          entropy_out=entropy_out)
    return _invoke("diffusion_sample_entropy", _ptr(logits, torch.float32, "logits"), P, V,
                   float(temperature), int(seed), int(step), _ptr(frozen, torch.uint8, "frozen"),
                   _ptr(tokens_out, torch.int32, "tokens_out"),
                   _ptr(entropy_out, torch.float32, "entropy_out"),
                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())


def diffusion_accept_entropy_bound(entropy, tokens, bound, frozen, canvas, accept_out,
                                   num_accepted):
    P = entropy.shape[0]
    _rows("diffusion_accept_entropy_bound", P, entropy=entropy, tokens=tokens, frozen=frozen,
          canvas=canvas, accept_out=accept_out)
    _at_least(num_accepted, 1, "num_accepted", "diffusion_accept_entropy_bound")
    return _invoke("diffusion_accept_entropy_bound", _ptr(entropy, torch.float32, "entropy"),
                   _ptr(tokens, torch.int32, "tokens"), P, float(bound),
                   _ptr(frozen, torch.uint8, "frozen"), _ptr(canvas, torch.int32, "canvas"),
                   _ptr(accept_out, torch.uint8, "accept_out"),
                   _ptr(num_accepted, torch.int32, "num_accepted"), _stream())


def diffusion_sample_step(logits, temperature, entropy_bound, seed, step, frozen, canvas,
                          tokens_out, entropy_out, accept_out, num_accepted, workspace,
                          loop_state=None):
    P, V = _logits_shape(logits, "diffusion_sample_step")
    _rows("diffusion_sample_step", P, frozen=frozen, canvas=canvas, tokens_out=tokens_out,
          entropy_out=entropy_out, accept_out=accept_out)
    _at_least(num_accepted, 1, "num_accepted", "diffusion_sample_step")
    args = (_ptr(logits, torch.float32, "logits"), P, V, float(temperature),
            float(entropy_bound), int(seed), int(step), _ptr(frozen, torch.uint8, "frozen"),
            _ptr(canvas, torch.int32, "canvas"), _ptr(tokens_out, torch.int32, "tokens_out"),
            _ptr(entropy_out, torch.float32, "entropy_out"),
            _ptr(accept_out, torch.uint8, "accept_out"),
            _ptr(num_accepted, torch.int32, "num_accepted"),
            _ptr(workspace, torch.uint8, "workspace"), workspace.numel())
    if loop_state is not None:
        return _invoke("diffusion_sample_step_gated", *args,
                       _gate(loop_state, "diffusion_sample_step"), _stream())
    return _invoke("diffusion_sample_step", *args, _stream())


def diffusion_sample_step_noalloc(logits, temperature, entropy_bound, seed, step, frozen, canvas,
                                  tokens_out, entropy_out, accept_out, num_accepted):
    P, V = _logits_shape(logits, "diffusion_sample_step_noalloc")
    _rows("diffusion_sample_step_noalloc", P, frozen=frozen, canvas=canvas, tokens_out=tokens_out,
          entropy_out=entropy_out, accept_out=accept_out)
    _at_least(num_accepted, 1, "num_accepted", "diffusion_sample_step_noalloc")
    return _invoke("diffusion_sample_step_noalloc", _ptr(logits, torch.float32, "logits"), P, V,
                   float(temperature), float(entropy_bound), int(seed), int(step),
                   _ptr(frozen, torch.uint8, "frozen"), _ptr(canvas, torch.int32, "canvas"),
                   _ptr(tokens_out, torch.int32, "tokens_out"),
                   _ptr(entropy_out, torch.float32, "entropy_out"),
                   _ptr(accept_out, torch.uint8, "accept_out"),
                   _ptr(num_accepted, torch.int32, "num_accepted"), _stream())


def diffusion_sample_confidence(logits, temperature, seed, step, frozen, tokens_out, entropy_out,
                                confidence_out, workspace):
    P, V = _logits_shape(logits, "diffusion_sample_confidence")
    _rows("diffusion_sample_confidence", P, frozen=frozen, tokens_out=tokens_out,
          entropy_out=entropy_out, confidence_out=confidence_out)
    return _invoke("diffusion_sample_confidence", _ptr(logits, torch.float32, "logits"), P, V,
                   float(temperature), int(seed), int(step), _ptr(frozen, torch.uint8, "frozen"),
                   _ptr(tokens_out, torch.int32, "tokens_out"),
                   _ptr(entropy_out, torch.float32, "entropy_out"),
                   _ptr(confidence_out, torch.float32, "confidence_out"),
                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())


def diffusion_accept_confidence(confidence, tokens, threshold, frozen, canvas, accept_out,
                                num_accepted):
    P = confidence.shape[0]
    _rows("diffusion_accept_confidence", P, confidence=confidence, tokens=tokens, frozen=frozen,
          canvas=canvas, accept_out=accept_out)
    _at_least(num_accepted, 1, "num_accepted", "diffusion_accept_confidence")
    return _invoke("diffusion_accept_confidence", _ptr(confidence, torch.float32, "confidence"),
                   _ptr(tokens, torch.int32, "tokens"), P, float(threshold),
                   _ptr(frozen, torch.uint8, "frozen"), _ptr(canvas, torch.int32, "canvas"),
                   _ptr(accept_out, torch.uint8, "accept_out"),
                   _ptr(num_accepted, torch.int32, "num_accepted"), _stream())


def diffusion_sample_step_confidence(logits, temperature, threshold, seed, step, frozen, canvas,
                                     tokens_out, confidence_out, accept_out, num_accepted,
                                     workspace, loop_state=None):
    P, V = _logits_shape(logits, "diffusion_sample_step_confidence")
    _rows("diffusion_sample_step_confidence", P, frozen=frozen, canvas=canvas,
          tokens_out=tokens_out, confidence_out=confidence_out, accept_out=accept_out)
    _at_least(num_accepted, 1, "num_accepted", "diffusion_sample_step_confidence")
    args = (_ptr(logits, torch.float32, "logits"), P, V, float(temperature), float(threshold),
            int(seed), int(step), _ptr(frozen, torch.uint8, "frozen"),
            _ptr(canvas, torch.int32, "canvas"), _ptr(tokens_out, torch.int32, "tokens_out"),
            _ptr(confidence_out, torch.float32, "confidence_out"),
            _ptr(accept_out, torch.uint8, "accept_out"),
            _ptr(num_accepted, torch.int32, "num_accepted"),
            _ptr(workspace, torch.uint8, "workspace"), workspace.numel())
    if loop_state is not None:
        return _invoke("diffusion_sample_step_confidence_gated", *args,
                       _gate(loop_state, "diffusion_sample_step_confidence"), _stream())
    return _invoke("diffusion_sample_step_confidence", *args, _stream())


def canvas_length(max_canvas, min_canvas, remaining, full_canvas=False):
    n = load().bd_canvas_length(int(max_canvas), int(min_canvas), int(remaining),
                                1 if full_canvas else 0)
    if n == 0:
        raise BdError("bd_canvas_length: invalid arguments")
    return n


def diffusion_canvas_init(canvas, prev_canvas, frozen, loop_state, vocab, seed, block):
    P = canvas.shape[0]
    _rows("diffusion_canvas_init", P, canvas=canvas, prev_canvas=prev_canvas, frozen=frozen)
    _at_least(loop_state, 4, "loop_state", "diffusion_canvas_init")
    return _invoke("diffusion_canvas_init", _ptr(canvas, torch.int32, "canvas"),
                   _ptr(prev_canvas, torch.int32, "prev_canvas"), _ptr(frozen, torch.uint8, "frozen"),
                   _ptr(loop_state, torch.int32, "loop_state"), P, int(vocab), int(seed), int(block),
                   _stream())


def diffusion_loop_update(tokens, canvas, prev_canvas, frozen, loop_state, stability_threshold,
                          max_steps, write_drafts=True):
    P = canvas.shape[0]
    _rows("diffusion_loop_update", P, tokens=tokens, canvas=canvas, prev_canvas=prev_canvas,
          frozen=frozen)
    _at_least(loop_state, 4, "loop_state", "diffusion_loop_update")
    return _invoke("diffusion_loop_update", _ptr(tokens, torch.int32, "tokens"),
                   _ptr(canvas, torch.int32, "canvas"), _ptr(prev_canvas, torch.int32, "prev_canvas"),
                   _ptr(frozen, torch.uint8, "frozen"), _ptr(loop_state, torch.int32, "loop_state"),
                   P, int(stability_threshold), int(max_steps), 1 if write_drafts else 0, _stream())


def hbm_copy(src, dst):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    return _invoke("bd_hbm_copy", _ptr(src, None, "src"), _ptr(dst, None, "dst"), n, _stream())


HBM_READ_WORDS = 2049


def hbm_read(src, checksum):
    """XOR of all 32-bit words of src into checksum[0]; checksum is an int32 device tensor of
    at least HBM_READ_WORDS elements (the rest is scratch)."""
    n = src.numel() * src.element_size()
    if checksum.numel() < HBM_READ_WORDS:
        raise ValueError(f"checksum needs {HBM_READ_WORDS} int32 elements")
    return _invoke("bd_hbm_read", _ptr(src, None, "src"), n, _ptr(checksum, torch.int32, "checksum"),
                   _stream())
