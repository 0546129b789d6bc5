"""CPU oracle for the forward pass of a top-k routed, renormalised MoE layer.

TEST INFRASTRUCTURE. This module is the parity reference for the HIP library.
Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import or run it; the product path never does. It shares no
code with the HIP path: it imports numpy only, and takes its inputs as plain
arrays (bf16 tensors arrive as uint16 bit patterns and are widened exactly).

Every step is the plain definition, computed in float64, one step after the
other in the order the pages give them, with no blocking or fusion:

  1. router logits  L = x W_r^T (+ b)          -- router Linear without bias
  2. probabilities  p = softmax(L) per token
  3. selection      S = the k experts with the largest logits, in descending
                    order, the lower expert index first among equal logits
  4. renormalise    w_j = p[S_j] / sum_i p[S_i]   (1/k if that sum were 0)
  5. counts / per-expert token lists in ascending token order
  6. each expert e: Y = (SiLU(X W_g^T) * (X W_u^T)) W_d^T on its rows
  7. combine        out[t] += w_j * Y_e[row of t]

Sources (page title, then the section / item):
  * axonml-nn ``layers/moe.rs`` (docs.rs): ``Expert`` forward (SwiGLU with
    the SiLU on the gate projection), ``MoERouter::route`` (Linear, softmax,
    stable sort by descending probability, take k, renormalise with a 1/k
    fallback), ``MoELayer::forward`` (expert counts, per-expert gather in
    token order, skip empty experts, weighted scatter-add), and
    ``load_balancing_loss`` (E * sum_i f_i P_i).
  * "Mixtral MoE Block" (neurarch.com, HTML and markdown pages), exported
    PyTorch ``_moe_forward``: softmax, topk, divide by the sum of the top-k
    weights, per-expert accumulation into a zero output.
  * "Model Architecture Patterns -- MoE, Router, FFN, LayerNorm": the
    ``SwiGLU`` FFN (silu(w1 x) * w3 x, then w2), ``TopKRouter`` (a Linear
    without bias).

Readings taken where the pages are silent or disagree (each is listed in the
design notes of the repository):
  * Selection compares logits, not rounded probabilities. Softmax is strictly
    increasing, so this is the pages' order by probability computed exactly;
    it differs only where rounding of exp() would merge two distinct values.
    Equal logits (including +0.0 and -0.0) keep the lower expert index first,
    as the stable sort of ``MoERouter::route`` does.
  * The layer renormalises (the axonml and Mixtral pages do; the skills
    page's ``TopKRouter`` does not, and is not followed).
  * The expert is gated SwiGLU with SiLU on gate_proj (axonml ``Expert``);
    the ungated two-matrix expert of the markdown Mixtral page and of the
    skills page's ``Expert`` is not followed (its parameter count cannot
    reach the 1.45B the Mixtral page states).
  * The combine weight of expert S_j for token t is w_j alone (axonml and
    Mixtral pages), not the sum of the token's gates (skills page's MoELayer).
  * No capacity limit: every token reaches its k experts.
  * Inputs must be finite (axonml's sort panics on NaN); asserted here.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "router_logits", "softmax", "select_top_k", "renormalise", "route",
    "expert_counts", "permute", "swiglu_expert", "combine", "expert_ffn",
    "moe_forward", "dense_bruteforce", "load_balancing_loss",
]


def widen(a) -> np.ndarray:
    """Any input array as float64. uint16 arrays are bfloat16 bit patterns:
    shifting them into the high half of a float32 is their exact value."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float64)


# ---------------------------------------------------------------- routing --

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] * W_r[e, i] (+ b[e]).

    The router is a Linear from the model width to E without bias
    (axonml ``MoERouter::new`` / ``route``; Mixtral page ``router``;
    skills page ``TopKRouter``). The optional bias is an input of the skewed
    workload only, added after the product."""
    L = widen(x) @ widen(w_router).T
    if bias is not None:
        L = L + widen(bias)[None, :]
    return L


def softmax(logits) -> np.ndarray:
    """p[t, e] = exp(L[t,e] - max_e L[t]) / sum_e exp(L[t,e] - max_e L[t])
    (axonml ``route``: softmax over the last axis; Mixtral ``_moe_forward``)."""
    L = widen(logits)
    assert np.all(np.isfinite(L)), "router logits must be finite"
    z = np.exp(L - L.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def select_top_k(logits, k: int) -> np.ndarray:
    """Indices [T, k] of each token's k largest logits, largest first.

    axonml ``MoERouter::route`` sorts the E (index, value) pairs by descending
    value with a stable sort and keeps the first k; a stable sort leaves equal
    values in ascending index order. A stable argsort of -L is that sort."""
    L = widen(logits)
    assert np.all(np.isfinite(L)), "router logits must be finite"
    E = L.shape[-1]
    assert 1 <= k <= E, "top_k must satisfy 1 <= k <= num_experts"
    order = np.argsort(-L, axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalise(probs, idx) -> np.ndarray:
    """w[t, j] = p[t, S_j] / sum_i p[t, S_i]; 1/k for a token whose selected
    probabilities sum to 0 (axonml ``route``; Mixtral ``_moe_forward`` divides
    the top-k weights by their sum)."""
    p = widen(probs)
    idx = np.asarray(idx)
    k = idx.shape[-1]
    top = np.take_along_axis(p, idx, axis=-1)
    s = top.sum(axis=-1, keepdims=True)
    out = np.full_like(top, 1.0 / k)
    pos = s[:, 0] > 0
    out[pos] = top[pos] / s[pos]
    return out


def route(logits, k: int):
    """(probs [T,E], topk_idx [T,k], topk_w [T,k]) from router logits: the three
    results ``MoERouter::route`` returns, in that order of computation."""
    p = softmax(logits)
    idx = select_top_k(logits, k)
    return p, idx, renormalise(p, idx)


# ---------------------------------------------------------------- dispatch --

def expert_counts(idx, E: int) -> np.ndarray:
    """Number of (token, slot) assignments per expert (axonml
    ``MoELayer::forward`` utilisation counts)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)[:E]


def permute(idx, E: int):
    """Per-expert token lists, as axonml ``MoELayer::forward`` builds them:
    experts in ascending order, and within an expert the tokens that chose it
    in ascending token order.

    Returns counts [E], offsets [E+1] (offsets[e] = start of expert e's rows),
    sorted_token [T*k] (token of each row), inv_pos [T*k] (row of assignment
    t*k + j)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = expert_counts(idx, E)
    offsets = np.zeros(E + 1, np.int64)
    sorted_token = np.empty(T * k, np.int64)
    inv_pos = np.empty(T * k, np.int64)
    row = 0
    for e in range(E):
        offsets[e] = row
        tok, slot = np.nonzero(idx == e)  # row-major: ascending token
        n = tok.size
        sorted_token[row:row + n] = tok
        inv_pos[tok * k + slot] = np.arange(row, row + n)
        row += n
    offsets[E] = row
    return counts, offsets, sorted_token, inv_pos


# ----------------------------------------------------------------- experts --

def swiglu_expert(X, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """down_proj(SiLU(gate_proj(X)) * up_proj(X)) with SiLU(z) = z / (1 + e^-z)
    (axonml ``Expert::forward``; skills page ``SwiGLU``). Weights are
    nn.Linear [out, in], so each projection multiplies by the transpose."""
    X = widen(X)
    G = X @ widen(w_gate_e).T
    U = X @ widen(w_up_e).T
    with np.errstate(over="ignore"):
        H = (G / (1.0 + np.exp(-G))) * U
    return H @ widen(w_down_e).T


def combine(T: int, d: int, idx, w, expert_rows) -> np.ndarray:
    """out[t] = sum over (e, t's slot j with S_j = e) of w[t, j] * Y_e[row],
    accumulated expert by expert into a zero output (axonml
    ``MoELayer::forward`` scatter-add; Mixtral ``out[rows] += w * expert(...)``).

    ``expert_rows[e]`` = (tokens [n], Y_e [n, d]) for each non-empty expert."""
    idx = np.asarray(idx)
    w = widen(w)
    out = np.zeros((T, d), np.float64)
    for e, (tok, Y) in expert_rows.items():
        # each token chooses e at most once, so this is its one weight
        wt = (w * (idx == e))[tok].sum(axis=-1)
        out[tok] += wt[:, None] * Y
    return out


def expert_ffn(x, idx, w, w_gate, w_up, w_down, E: int | None = None) -> np.ndarray:
    """Rows 5-7 of the layer for a given routing (idx, w): gather each expert's
    tokens, run its SwiGLU FFN, combine. Experts with no token are skipped."""
    idx = np.asarray(idx)
    xw = widen(x)
    T, d = xw.shape
    E = np.asarray(w_gate).shape[0] if E is None else E
    rows = {}
    for e in range(E):
        tok = np.nonzero((idx == e).any(axis=-1))[0]
        if tok.size == 0:
            continue
        rows[e] = (tok, swiglu_expert(xw[tok], w_gate[e], w_up[e], w_down[e]))
    return combine(T, d, idx, w, rows)


def moe_forward(x, w_router, w_gate, w_up, w_down, k: int, bias=None):
    """The whole layer on x [T, d]: router logits, route, counts, per-expert
    SwiGLU, weighted combine (axonml ``MoELayer::forward``).

    Returns (out [T,d], dict(logits, probs, idx, w, counts))."""
    L = router_logits(x, w_router, bias)
    probs, idx, w = route(L, k)
    E = np.asarray(w_router).shape[0]
    out = expert_ffn(x, idx, w, w_gate, w_up, w_down, E)
    return out, {"logits": L, "probs": probs, "idx": idx, "w": w,
                 "counts": expert_counts(idx, E)}


def dense_bruteforce(x, w_router, w_gate, w_up, w_down, k: int, bias=None) -> np.ndarray:
    """Self-check form of the layer: every expert on every token, then each
    token keeps the outputs of its selected experts with their renormalised
    weights and zero weight on the rest. Only for tiny inputs."""
    xw = widen(x)
    T, d = xw.shape
    E = np.asarray(w_router).shape[0]
    L = router_logits(x, w_router, bias)
    probs, idx, w = route(L, k)
    gate = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            gate[t, idx[t, j]] = w[t, j]
    out = np.zeros((T, d))
    for e in range(E):
        out += gate[:, e:e + 1] * swiglu_expert(xw, w_gate[e], w_up[e], w_down[e])
    return out


# -------------------------------------------------------------- statistics --

def load_balancing_loss(probs, counts) -> float:
    """E * sum_i f_i * P_i with f_i = counts_i / T (fraction of tokens sent to
    expert i; over all k slots these fractions sum to k) and P_i the mean
    routing probability of expert i over the T tokens; 0 for T = 0
    (axonml ``MoELayer::load_balancing_loss``)."""
    p = widen(probs)
    T, E = p.shape
    if T == 0:
        return 0.0
    f = np.asarray(counts, np.float64) / T
    P = p.sum(axis=0) / T
    return float(E * np.sum(f * P))
