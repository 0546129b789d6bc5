"""Seeded synthetic workloads for the top-k routed MoE layer.

This module only makes inputs: shapes, seeded random draws and their rounding
to the storage dtype. It holds none of the layer's arithmetic (no routing, no
softmax, no expert math), so the CPU oracle and the HIP path can both be fed
from it without sharing any of the computation under test.

Workload shapes
---------------
The layer shape is the Mixtral block of the "Mixtral MoE Block" pages
(neurarch.com, structure table row ``block_sparse_moe`` and the exported
PyTorch module): hidden size 4096, 8 experts, top-2, expert FFN width 14336,
gate/up/down projections without bias. The other sizes follow the FFN sizing
rules of KempnerForge's ``ModelConfig`` (``computed_ffn_hidden_dim`` and
``computed_expert_ffn_hidden_dim``), reproduced by :func:`ffn_hidden_dim` and
:func:`expert_ffn_hidden_dim` so that the sizes below are checkable, not
typed in.

Random draws
------------
Every tensor is drawn from numpy's PCG64 with ``standard_normal`` in float32,
in chunks of ``CHUNK`` elements; chunk ``c`` of tensor ``tid`` uses the stream
``SeedSequence(seed, spawn_key=(tid, c))``. The value of an element therefore
depends only on (seed, tensor, position), never on thread count, which lets
the multi-GiB Mixtral weights be drawn by several threads at once.
Tensor ids: x=0, w_router=1, w_gate=2, w_up=3, w_down=4, and 16+ for the
synthetic logits / routings used by the routing and expert-only tests.
Weights are scaled by 0.02 (the ``init_std`` default of KempnerForge's
``ModelConfig``); x stays N(0, 1). bf16 workloads round each float32 draw to
bfloat16 with round-to-nearest-even and store the 16-bit patterns as uint16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22
WEIGHT_STD = 0.02

TID_X, TID_ROUTER, TID_GATE, TID_UP, TID_DOWN = 0, 1, 2, 3, 4
TID_LOGITS, TID_ROUTING_IDX, TID_ROUTING_W = 16, 17, 18
TID_NORM, TID_SHARED_GATE, TID_SHARED_UP, TID_SHARED_DOWN = 5, 6, 7, 8


def ffn_hidden_dim(dim: int, ffn_dim_multiplier: float = 1.0) -> int:
    """Llama-style dense FFN width: 4*dim*2/3*multiplier truncated to an int,
    then rounded UP to a multiple of 256 (KempnerForge ``ModelConfig``,
    ``computed_ffn_hidden_dim``; its docstring says "nearest" but the code
    takes the ceiling, and the code is followed here)."""
    raw = int(4 * dim * (2 / 3) * ffn_dim_multiplier)
    return 256 * math.ceil(raw / 256)


def expert_ffn_hidden_dim(dense_ffn: int, expert_multiplier: float = 1.0) -> int:
    """Per-expert width: dense width times the expert multiplier, rounded to a
    multiple of 16, at least 16 (KempnerForge ``ModelConfig``,
    ``computed_expert_ffn_hidden_dim``)."""
    raw = int(dense_ffn * expert_multiplier)
    return max(16, 16 * round(raw / 16))


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens (batch * sequence, flattened)
    d: int          # model width
    ffn: int        # expert hidden width
    E: int          # experts
    k: int          # experts per token
    dtype: str      # "f32" or "bf16": storage dtype of x and every weight
    zipf_bias: bool = False  # add the per-expert logit bias of the skewed workload

    @property
    def active_flops(self) -> int:
        """FLOPs the layer must do: k expert FFNs of 3 matrices per token plus
        the router projection (the top-k/N-of-the-compute statement of the
        axonml-nn ``MoELayer`` doc comment)."""
        return self.T * self.k * 6 * self.d * self.ffn + 2 * self.T * self.d * self.E


WORKLOADS = {
    # Tiny fp32 layer for exhaustive parity.
    "tiny": Workload("tiny", T=64, d=64, ffn=128, E=4, k=2, dtype="f32"),
    # Small bf16 layer: d=1024 and its Llama-style width 2816.
    "small": Workload("small", T=2048, d=1024, ffn=ffn_hidden_dim(1024), E=8, k=2, dtype="bf16"),
    # Mixtral-shaped prefill: one sequence of 4096 tokens, width 14336
    # (= Llama sizing of 4096 with multiplier 1.3).
    "prefill": Workload("prefill", T=4096, d=4096, ffn=ffn_hidden_dim(4096, 1.3), E=8, k=2,
                        dtype="bf16"),
    # Mixtral-shaped decode step: 32 tokens, weight streaming.
    "decode": Workload("decode", T=32, d=4096, ffn=ffn_hidden_dim(4096, 1.3), E=8, k=2,
                       dtype="bf16"),
    # Fine-grained experts (multiplier 0.25 of the d=2048 dense width), 64
    # experts, top-8, with a Zipf-shaped logit prior so loads are skewed.
    "skewed": Workload("skewed", T=8192, d=2048,
                       ffn=expert_ffn_hidden_dim(ffn_hidden_dim(2048), 0.25),
                       E=64, k=8, dtype="bf16", zipf_bias=True),
}


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------

def _stream(seed: int, tid: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, chunk))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tid: int, n: int, scale: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, scale^2) from the chunked stream of tensor tid."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        view = out[lo:hi]
        _stream(seed, tid, c).standard_normal(out=view, dtype=np.float32)
        if scale != 1.0:
            np.multiply(view, np.float32(scale), out=view)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as pool:
            list(pool.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the
    16-bit patterns as uint16. Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _tensor(seed: int, tid: int, shape, scale: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    f = normal_f32(seed, tid, n, scale).reshape(shape)
    if dtype == "bf16":
        return f32_to_bf16_bits(f).reshape(shape)
    return f


def zipf_logit_bias(E: int, s: float = 1.2) -> np.ndarray:
    """Per-expert additive router-logit bias for the skewed workload:
    b_e = -s * ln(e + 1), so that with no other signal the routing prior over
    expert rank e+1 is proportional to (e+1)^-s (Zipf with exponent s)."""
    return (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def make_layer_inputs(w: Workload, seed: int = 0, with_weights: bool = True) -> dict:
    """All inputs of one layer call, in the storage dtype of the workload.

    Returns a dict with x [T,d], w_router [E,d], w_gate [E,ffn,d],
    w_up [E,ffn,d], w_down [E,d,ffn] (uint16 bf16 bits or float32), and
    router_bias [E] float32 or None.
    """
    out = {
        "x": _tensor(seed, TID_X, (w.T, w.d), 1.0, w.dtype),
        "w_router": _tensor(seed, TID_ROUTER, (w.E, w.d), WEIGHT_STD, w.dtype),
        "router_bias": zipf_logit_bias(w.E) if w.zipf_bias else None,
    }
    if with_weights:
        out["w_gate"] = _tensor(seed, TID_GATE, (w.E, w.ffn, w.d), WEIGHT_STD, w.dtype)
        out["w_up"] = _tensor(seed, TID_UP, (w.E, w.ffn, w.d), WEIGHT_STD, w.dtype)
        out["w_down"] = _tensor(seed, TID_DOWN, (w.E, w.d, w.ffn), WEIGHT_STD, w.dtype)
    return out


def make_custom_inputs(T: int, d: int, ffn: int, E: int, dtype: str, seed: int = 0,
                       bias: bool = False) -> dict:
    """Same recipe as :func:`make_layer_inputs` for an arbitrary shape."""
    return make_layer_inputs(Workload("custom", T, d, ffn, E, 1, dtype, bias), seed)


def make_block_extras(d: int, n_shared: int, shared_ffn: int, dtype: str, seed: int = 0) -> dict:
    """Inputs of the block options: an RMSNorm weight [d] drawn around 1
    (1 + 0.1 N(0,1)) and n_shared shared experts' weights (0.02 N(0,1)):
    s_gate, s_up [n_shared, shared_ffn, d], s_down [n_shared, d, shared_ffn]."""
    g = 1.0 + normal_f32(seed, TID_NORM, d, 0.1)
    out = {"norm_weight": f32_to_bf16_bits(g) if dtype == "bf16" else g.astype(np.float32)}
    if n_shared > 0:
        out["s_gate"] = _tensor(seed, TID_SHARED_GATE, (n_shared, shared_ffn, d), WEIGHT_STD, dtype)
        out["s_up"] = _tensor(seed, TID_SHARED_UP, (n_shared, shared_ffn, d), WEIGHT_STD, dtype)
        out["s_down"] = _tensor(seed, TID_SHARED_DOWN, (n_shared, d, shared_ffn), WEIGHT_STD, dtype)
    return out


# --------------------------------------------------------------------------
# synthetic router logits (routing-only tests)
# --------------------------------------------------------------------------

LOGIT_KINDS = ("normal", "ties", "zeros", "huge", "subnormal", "mixed")


def make_logits(T: int, E: int, kind: str = "normal", seed: int = 0) -> np.ndarray:
    """float32 router logits [T, E] of a given structure.

    normal    : N(0, 1.28^2), the spread of x.W_r at d=4096 and std 0.02
    ties      : values from {-1, 0, 0.5, 1} so most rows hold exact ties
    zeros     : every entry +0.0 or -0.0 (sign at random)
    huge      : magnitudes up to 3e38 of both signs, with repeats
    subnormal : magnitudes around 1e-41 (denormal float32), with repeats
    mixed     : rows cycle through the kinds above
    """
    rng = _stream(seed, TID_LOGITS, LOGIT_KINDS.index(kind))
    if kind == "normal":
        return (rng.standard_normal((T, E), dtype=np.float32) * np.float32(1.28)).astype(np.float32)
    if kind == "ties":
        return rng.choice(np.array([-1.0, 0.0, 0.5, 1.0], np.float32), size=(T, E))
    if kind == "zeros":
        sign = rng.integers(0, 2, size=(T, E)).astype(bool)
        return np.where(sign, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    if kind == "huge":
        mags = np.array([3e38, 1e38, 1e30, 1e30, 2.5, 0.0], np.float32)
        v = rng.choice(mags, size=(T, E))
        s = rng.choice(np.array([-1.0, 1.0], np.float32), size=(T, E))
        return (v * s).astype(np.float32)
    if kind == "subnormal":
        bits = rng.choice(np.array([1, 2, 7000, 7000, 0x007FFFFF], np.uint32), size=(T, E))
        s = rng.integers(0, 2, size=(T, E)).astype(np.uint32) << np.uint32(31)
        return (bits | s).view(np.float32)
    if kind == "mixed":
        parts = [make_logits(T, E, kd, seed) for kd in LOGIT_KINDS[:-1]]
        rows = np.arange(T) % len(parts)
        out = np.empty((T, E), np.float32)
        for i, p in enumerate(parts):
            out[rows == i] = p[rows == i]
        return out
    raise ValueError(f"unknown logit kind {kind!r}")


# --------------------------------------------------------------------------
# synthetic routings (expert-only tests): k distinct experts per token
# --------------------------------------------------------------------------

ROUTING_KINDS = ("random", "all_same", "even_only", "one_heavy")


def make_routing(T: int, E: int, k: int, kind: str = "random", seed: int = 0):
    """(topk_idx int32 [T,k], topk_w float32 [T,k]) with k distinct experts per
    token and positive weights (not normalised: the expert path must not rely
    on it).

    random    : a uniformly random k-subset per token, random slot order
    all_same  : every token uses experts 0..k-1 (all other experts empty)
    even_only : subsets of the even experts only (odd experts empty); needs 2k <= E
    one_heavy : expert E-1 in every token's slot 0, the rest random
    """
    rng = _stream(seed, TID_ROUTING_IDX, ROUTING_KINDS.index(kind))
    idx = np.empty((T, k), np.int32)
    if kind == "random":
        for t in range(T):
            idx[t] = rng.permutation(E)[:k]
    elif kind == "all_same":
        idx[:] = np.arange(k, dtype=np.int32)
    elif kind == "even_only":
        evens = np.arange(0, E, 2)
        assert len(evens) >= k
        for t in range(T):
            idx[t] = rng.permutation(evens)[:k]
    elif kind == "one_heavy":
        rest = np.arange(E - 1)
        for t in range(T):
            idx[t, 0] = E - 1
            idx[t, 1:] = rng.permutation(rest)[:k - 1]
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    wr = _stream(seed, TID_ROUTING_W, ROUTING_KINDS.index(kind))
    w = wr.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return idx, w
