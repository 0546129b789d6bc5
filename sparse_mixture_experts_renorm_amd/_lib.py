"""ctypes binding of libmoe_mi355x.so (argument marshalling only).

Every function here has the name of the C entry point it calls, checks the
torch tensors it is given (device, dtype, shape, contiguity), allocates the
outputs the caller did not pass, and hands raw device pointers plus the
current HIP stream to the library. All arithmetic runs in the library's HIP
kernels; there is no fallback: if the shared library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_WORKSPACE_TOO_SMALL, MOE_HIP_ERROR = range(5)
MOE_F32, MOE_BF16 = 0, 1
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def _p(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run "
                "`python -m sparse_mixture_experts_renorm_amd.build` (hipcc, gfx950)")
        _lib = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        _p("moe_status_string", ctypes.c_char_p, i)
        _p("moe_workspace_size", sz, i, i, i, i, i, i)
        _p("moe_route", i, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp)
        _p("moe_route_logits", i, vp, i, i, i, vp, vp, vp, vp)
        _p("moe_permute_workspace_size", sz, i, i, i)
        _p("moe_permute", i, vp, vp, i, i, i, vp, vp, vp, vp, vp, vp, sz, vp)
        _p("moe_expert_ffn", i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, sz, vp)
        _p("moe_forward", i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, vp, vp, vp, sz, vp)
        _p("moe_forward_profiled", i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, vp, vp,
           vp, sz, vp, vp)
        _p("moe_forward_no_alloc", i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, vp, vp,
           vp)
        _p("moe_router_stats_workspace_size", sz, i, i)
        _p("moe_router_stats", i, vp, vp, i, i, vp, vp, vp, vp, sz, vp)
        _p("moe_forward_ext_workspace_size", sz, i, i, i, i, i, i, vp)
        _p("moe_forward_ext", i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, i, vp, vp, vp,
           vp, vp, sz, vp)
    return _lib


def declared_symbols() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|size_t|moe_status)\s+(moe_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoEError(status, fn)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def moe_workspace_size(T: int, d: int, ffn: int, E: int, k: int, dtype) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().moe_workspace_size(T, d, ffn, E, k, dt))


def workspace(T, d, ffn, E, k, dtype, device="cuda") -> torch.Tensor:
    """A device byte buffer large enough for moe_forward / moe_expert_ffn."""
    n = moe_workspace_size(T, d, ffn, E, k, dtype)
    if n == 0:
        raise ValueError("invalid or unsupported shape")
    return torch.empty(n + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws: torch.Tensor):
    p = ws.data_ptr()
    a = (p + 255) & ~255
    return ctypes.c_void_p(a), ws.numel() - (a - p)


def moe_route_logits(logits, k, probs=False, stream=None):
    """Routing from fp32 logits [T,E]. Returns (topk_idx int32 [T,k],
    topk_w f32 [T,k]) and probs f32 [T,E] as a third item if probs=True."""
    _dev(logits)
    assert logits.dtype == torch.float32 and logits.dim() == 2
    T, E = logits.shape
    dev = logits.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = torch.empty((T, E), dtype=torch.float32, device=dev) if probs else None
    _check(lib().moe_route_logits(_ptr(logits), T, E, k, _ptr(p), _ptr(idx), _ptr(w), _stream(stream)),
           "moe_route_logits")
    return (idx, w, p) if probs else (idx, w)


def moe_route(x, w_router, k, router_bias=None, want_logits=False, want_probs=False, stream=None):
    """Fused router. Returns dict(topk_idx, topk_w[, logits][, probs])."""
    _dev(x, w_router, router_bias)
    T, d = x.shape
    E = w_router.shape[0]
    assert w_router.shape == (E, d) and w_router.dtype == x.dtype
    dev = x.device
    out = {"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
           "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev)}
    if want_logits:
        out["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_probs:
        out["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check(lib().moe_route(_ptr(x), _ptr(w_router), _ptr(router_bias), T, d, E, k, _dt(x),
                           _ptr(out.get("logits")), _ptr(out.get("probs")), _ptr(out["topk_idx"]),
                           _ptr(out["topk_w"]), _stream(stream)), "moe_route")
    return out


def moe_permute(topk_idx, E, topk_w=None, stream=None):
    """Returns (counts [E], offsets [E+1], sorted_token [T*k], inv_pos [T*k]), all
    int32, and with topk_w (f32 [T,k]) also sorted_w (f32 [T*k]), the weights in
    permuted order."""
    _dev(topk_idx, topk_w)
    assert topk_idx.dtype == torch.int32 and topk_idx.dim() == 2
    T, k = topk_idx.shape
    if topk_w is not None:
        assert topk_w.dtype == torch.float32 and tuple(topk_w.shape) == (T, k)
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    sw = torch.empty(T * k, dtype=torch.float32, device=dev) if topk_w is not None else None
    n = int(lib().moe_permute_workspace_size(T, E, k))
    ws = torch.empty(n + 256, dtype=torch.uint8, device=dev) if n else None
    wp, wn = _ws_ptr(ws) if n else (None, 0)
    _check(lib().moe_permute(_ptr(topk_idx), _ptr(topk_w), T, E, k, _ptr(counts), _ptr(offsets),
                             _ptr(st), _ptr(inv), _ptr(sw), wp, wn, _stream(stream)),
           "moe_permute")
    return (counts, offsets, st, inv) if sw is None else (counts, offsets, st, inv, sw)


def moe_router_stats(probs, counts, stream=None):
    """Router statistics from probs f32 [T,E] and counts int32 [E]. Returns
    (mean_probs f32 [E], frac f32 [E], lb_loss f32 [1]) as device tensors."""
    _dev(probs, counts)
    assert probs.dtype == torch.float32 and probs.dim() == 2
    assert counts.dtype == torch.int32 and counts.dim() == 1
    T, E = probs.shape
    assert counts.shape[0] == E
    dev = probs.device
    mean = torch.empty(E, dtype=torch.float32, device=dev)
    frac = torch.empty(E, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    n = int(lib().moe_router_stats_workspace_size(T, E))
    ws = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device=dev)
    wp, wn = _ws_ptr(ws)
    _check(lib().moe_router_stats(_ptr(probs), _ptr(counts), T, E, _ptr(mean), _ptr(frac),
                                  _ptr(loss), wp, wn, _stream(stream)), "moe_router_stats")
    return mean, frac, loss


def _layer_shapes(x, w_gate, w_up, w_down):
    T, d = x.shape
    E, ffn, d2 = w_gate.shape
    assert d2 == d and w_up.shape == (E, ffn, d) and w_down.shape == (E, d, ffn)
    assert w_gate.dtype == w_up.dtype == w_down.dtype == x.dtype
    return T, d, ffn, E


def moe_expert_ffn(x, topk_idx, topk_w, w_gate, w_up, w_down, out_dtype=torch.float32, out=None,
                   ws=None, stream=None):
    """Expert half of the layer for a given routing; returns out [T, d]."""
    _dev(x, topk_idx, topk_w, w_gate, w_up, w_down, out, ws)
    T, d, ffn, E = _layer_shapes(x, w_gate, w_up, w_down)
    k = topk_idx.shape[1]
    assert topk_idx.dtype == torch.int32 and topk_w.dtype == torch.float32
    assert topk_idx.shape == (T, k) and topk_w.shape == (T, k)
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=x.device)
    if ws is None:
        ws = workspace(T, d, ffn, E, k, x.dtype, x.device)
    wp, wn = _ws_ptr(ws)
    _check(lib().moe_expert_ffn(_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(w_gate), _ptr(w_up),
                                _ptr(w_down), T, d, ffn, E, k, _dt(x), _ptr(out), _dt(out), wp, wn,
                                _stream(stream)), "moe_expert_ffn")
    return out


def stage_events():
    """Six timing events for moe_forward(stage_events=...): before the router,
    after it, after the permutation, the gate/up GEMM, the down GEMM and the
    combine. Each is recorded once here so its HIP event exists."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs


def moe_forward(x, w_router, w_gate, w_up, w_down, k, router_bias=None, out_dtype=torch.float32,
                out=None, ws=None, want_logits=False, want_probs=False, want_counts=False,
                stream=None, stage_events=None):
    """The whole layer. Returns out [T, d], or (out, extras) when any want_*
    flag is set (extras: logits [T,E], probs [T,E], counts [E]). With
    stage_events (from stage_events()) it calls moe_forward_profiled, which
    records them between the layer's kernels."""
    _dev(x, w_router, w_gate, w_up, w_down, router_bias, out, ws)
    T, d, ffn, E = _layer_shapes(x, w_gate, w_up, w_down)
    assert w_router.shape == (E, d) and w_router.dtype == x.dtype
    dev = x.device
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=dev)
    if ws is None:
        ws = workspace(T, d, ffn, E, k, x.dtype, dev)
    extras = {}
    if want_logits:
        extras["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_probs:
        extras["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_counts:
        extras["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    wp, wn = _ws_ptr(ws)
    args = [_ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(router_bias), T,
            d, ffn, E, k, _dt(x), _ptr(out), _dt(out), _ptr(extras.get("logits")),
            _ptr(extras.get("probs")), _ptr(extras.get("counts")), wp, wn, _stream(stream)]
    if stage_events is None:
        _check(lib().moe_forward(*args), "moe_forward")
    else:
        assert len(stage_events) == 6
        arr = (ctypes.c_void_p * 6)(*[e.cuda_event for e in stage_events])
        _check(lib().moe_forward_profiled(*args, arr), "moe_forward_profiled")
    return (out, extras) if extras else out


NO_ALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NO_ALLOC_SCRATCH_BYTES of include/moe.h


def moe_forward_no_alloc(x, w_router, w_gate, w_up, w_down, k, router_bias=None,
                         out_dtype=torch.float32, out=None, want_logits=False, want_probs=False,
                         want_counts=False, stream=None):
    """moe_forward with the library's own fixed scratch instead of a workspace
    argument (the C call allocates nothing; outputs the caller does not pass
    are allocated here by torch). Same returns as moe_forward."""
    _dev(x, w_router, w_gate, w_up, w_down, router_bias, out)
    T, d, ffn, E = _layer_shapes(x, w_gate, w_up, w_down)
    assert w_router.shape == (E, d) and w_router.dtype == x.dtype
    dev = x.device
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=dev)
    extras = {}
    if want_logits:
        extras["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_probs:
        extras["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_counts:
        extras["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    _check(lib().moe_forward_no_alloc(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(router_bias), T, d,
        ffn, E, k, _dt(x), _ptr(out), _dt(out), _ptr(extras.get("logits")),
        _ptr(extras.get("probs")), _ptr(extras.get("counts")), _stream(stream)),
        "moe_forward_no_alloc")
    return (out, extras) if extras else out


class MoeOptions(ctypes.Structure):
    """Mirror of the C struct moe_options (include/moe.h)."""
    _fields_ = [("capacity_factor", ctypes.c_float), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("residual", ctypes.c_int),
                ("n_shared", ctypes.c_int), ("shared_ffn", ctypes.c_int),
                ("shared_gate", ctypes.c_void_p), ("shared_up", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p)]


def _options(capacity_factor, norm_weight, norm_eps, residual, shared):
    o = MoeOptions()
    o.capacity_factor = float(capacity_factor)
    o.norm_weight = None if norm_weight is None else norm_weight.data_ptr()
    o.norm_eps = float(norm_eps)
    o.residual = 1 if residual else 0
    if shared is not None:
        sg, su, sd = shared
        o.n_shared, o.shared_ffn = sg.shape[0], sg.shape[1]
        o.shared_gate, o.shared_up, o.shared_down = sg.data_ptr(), su.data_ptr(), sd.data_ptr()
    return o


def moe_forward_ext_workspace_size(T, d, ffn, E, k, dtype, capacity_factor=0.0, norm_weight=None,
                                   norm_eps=1e-5, residual=False, shared=None) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    o = _options(capacity_factor, norm_weight, norm_eps, residual, shared)
    return int(lib().moe_forward_ext_workspace_size(T, d, ffn, E, k, dt, ctypes.byref(o)))


def moe_forward_ext(x, w_router, w_gate, w_up, w_down, k, router_bias=None, capacity_factor=0.0,
                    norm_weight=None, norm_eps=1e-5, residual=False, shared=None,
                    out_dtype=torch.float32, out=None, ws=None, want_logits=False,
                    want_probs=False, want_counts=False, want_routed_counts=False, stream=None):
    """The layer with the block options of moe_forward_ext: capacity factor,
    RMSNorm of the input (norm_weight [d]), residual add, shared experts
    (shared = (s_gate [S,ffn_s,d], s_up [S,ffn_s,d], s_down [S,d,ffn_s])).
    Returns out [T, d], or (out, extras) when any want_* flag is set."""
    _dev(x, w_router, w_gate, w_up, w_down, router_bias, norm_weight, out, ws)
    T, d, ffn, E = _layer_shapes(x, w_gate, w_up, w_down)
    assert w_router.shape == (E, d) and w_router.dtype == x.dtype
    if norm_weight is not None:
        assert norm_weight.shape == (d,) and norm_weight.dtype == x.dtype
    if shared is not None:
        _dev(*shared)
        sg, su, sd = shared
        S, sffn, d2 = sg.shape
        assert d2 == d and su.shape == (S, sffn, d) and sd.shape == (S, d, sffn)
        assert sg.dtype == su.dtype == sd.dtype == x.dtype
    dev = x.device
    o = _options(capacity_factor, norm_weight, norm_eps, residual, shared)
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=dev)
    if ws is None:
        n = int(lib().moe_forward_ext_workspace_size(T, d, ffn, E, k, _dt(x), ctypes.byref(o)))
        if n == 0:
            raise ValueError("invalid or unsupported shape or options")
        ws = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    extras = {}
    if want_logits:
        extras["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_probs:
        extras["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if want_counts:
        extras["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    if want_routed_counts:
        extras["routed_counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    wp, wn = _ws_ptr(ws)
    _check(lib().moe_forward_ext(_ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                 _ptr(router_bias), T, d, ffn, E, k, _dt(x), ctypes.byref(o),
                                 _ptr(out), _dt(out), _ptr(extras.get("logits")),
                                 _ptr(extras.get("probs")), _ptr(extras.get("counts")),
                                 _ptr(extras.get("routed_counts")), wp, wn, _stream(stream)),
           "moe_forward_ext")
    return (out, extras) if extras else out
