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
  * No capacity limit by default: every token reaches its k experts. With a
    capacity factor cf > 0 (KempnerForge ``ModelConfig.moe_capacity_factor``:
    0 means no dropping, a positive value caps the tokens per expert) each
    expert keeps at most C = ceil(cf * T * k / E) assignments, the first C
    in token order; a dropped assignment adds nothing and the token's other
    weights are left as routed (not renormalised again).
  * RMSNorm before the layer follows the Mixtral page's ``nn.RMSNorm``:
    x / sqrt(mean(x^2) + eps) * weight (eps inside the root; the skills
    page's variant adds eps to the root instead and is not followed); the
    block adds the un-normalised input back (``moe_residual``).
  * When the layer's inputs are bf16, the normalised input is a bf16 tensor
    too (it is the input of a bf16 layer): the exact RMSNorm value is
    rounded once to the nearest bf16, ties to even (``round_to_bf16``).
  * Shared experts (KempnerForge ``moe_shared_experts``: experts that process
    all tokens) are SwiGLU FFNs applied to every token and added with
    weight 1.
  * Inputs must be finite (axonml's sort panics on NaN); asserted here.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "router_logits", "softmax", "select_top_k", "renormalise", "route",
    "expert_counts", "permute", "swiglu_expert", "combine", "expert_ffn",
    "moe_forward", "dense_bruteforce", "load_balancing_loss", "capacity", "rms_norm",
    "shared_experts", "round_to_bf16",
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


def capacity(T: int, E: int, k: int, capacity_factor: float):
    """Assignments each expert may keep: None (no limit) for a factor of 0,
    else ceil(cf * T * k / E) (KempnerForge ``moe_capacity_factor``, read as
    a multiple of the even share T * k / E)."""
    if capacity_factor < 0:
        raise ValueError("capacity_factor must be >= 0")
    if capacity_factor == 0:
        return None
    return int(np.ceil(capacity_factor * T * k / E))


def permute(idx, E: int, cap=None):
    """Per-expert token lists, as axonml ``MoELayer::forward`` builds them:
    experts in ascending order, and within an expert the tokens that chose it
    in ascending token order. With ``cap`` only the first ``cap`` tokens of
    each expert are kept.

    Returns counts [E] (rows kept per expert), offsets [E+1] (offsets[e] =
    start of expert e's rows), sorted_token [rows] (token of each row) and
    inv_pos [T*k] (row of assignment t*k + j, -1 if it was dropped)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    offsets = np.zeros(E + 1, np.int64)
    inv_pos = np.full(T * k, -1, np.int64)
    lists = []
    row = 0
    for e in range(E):
        offsets[e] = row
        tok, slot = np.nonzero(idx == e)  # row-major: ascending token
        if cap is not None:
            tok, slot = tok[:cap], slot[:cap]
        n = tok.size
        counts[e] = n
        lists.append(tok)
        inv_pos[tok * k + slot] = np.arange(row, row + n)
        row += n
    offsets[E] = row
    sorted_token = np.concatenate(lists) if lists else np.zeros(0, np.int64)
    return counts, offsets, sorted_token.astype(np.int64), inv_pos


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


def expert_ffn(x, idx, w, w_gate, w_up, w_down, E: int | None = None, cap=None) -> np.ndarray:
    """Rows 5-7 of the layer for a given routing (idx, w): gather each expert's
    tokens (the first ``cap`` of them if a capacity is set), run its SwiGLU
    FFN, combine. Experts with no token are skipped; a token an expert did
    not keep gets nothing from it."""
    idx = np.asarray(idx)
    xw = widen(x)
    T, d = xw.shape
    E = np.asarray(w_gate).shape[0] if E is None else E
    rows = {}
    for e in range(E):
        tok = np.nonzero((idx == e).any(axis=-1))[0]
        if cap is not None:
            tok = tok[:cap]
        if tok.size == 0:
            continue
        rows[e] = (tok, swiglu_expert(xw[tok], w_gate[e], w_up[e], w_down[e]))
    return combine(T, d, idx, w, rows)


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight over the last axis (the Mixtral
    page's ``nn.RMSNorm`` before the MoE layer)."""
    xw = widen(x)
    r = np.sqrt(np.mean(xw * xw, axis=-1, keepdims=True) + eps)
    return xw / r * widen(weight)


def round_to_bf16(a) -> np.ndarray:
    """Nearest bfloat16 value of each element (8 significant bits, ties to
    even), as float64. Normal range only (the values rounded here are
    normalised activations)."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                 # a = m * 2^e with 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # np.round: half to even


def shared_experts(x, s_gate, s_up, s_down) -> np.ndarray:
    """Sum over the shared experts of their SwiGLU FFN on every token
    (KempnerForge ``moe_shared_experts``); weights [S, ffn_s, d] and
    [S, d, ffn_s]."""
    xw = widen(x)
    out = np.zeros_like(xw)
    for i in range(np.asarray(s_gate).shape[0]):
        out += swiglu_expert(xw, s_gate[i], s_up[i], s_down[i])
    return out


def moe_forward(x, w_router, w_gate, w_up, w_down, k: int, bias=None, capacity_factor=0.0,
                norm_weight=None, norm_eps=1e-5, residual=False, shared=None):
    """The whole layer on x [T, d]: router logits, route, counts, per-expert
    SwiGLU, weighted combine (axonml ``MoELayer::forward``).

    Options (all off by default): ``capacity_factor`` (see ``capacity``);
    ``norm_weight``: the layer runs on rms_norm(x, norm_weight, norm_eps);
    ``residual``: x (not normalised) is added to the output (the Mixtral
    block's ``moe_residual``); ``shared`` = (s_gate, s_up, s_down): shared
    experts added to every token.

    Returns (out [T,d], dict(logits, probs, idx, w, counts, routed_counts)),
    counts being the rows each expert kept."""
    xin = widen(x)
    xl = xin if norm_weight is None else rms_norm(xin, norm_weight, norm_eps)
    if norm_weight is not None and np.asarray(x).dtype == np.uint16:
        xl = round_to_bf16(xl)  # a bf16 layer's normalised input is bf16
    L = router_logits(xl, w_router, bias)
    probs, idx, w = route(L, k)
    E = np.asarray(w_router).shape[0]
    T = xin.shape[0]
    cap = capacity(T, E, k, capacity_factor)
    out = expert_ffn(xl, idx, w, w_gate, w_up, w_down, E, cap)
    if shared is not None:
        out = out + shared_experts(xl, *shared)
    if residual:
        out = out + xin
    routed = expert_counts(idx, E)
    kept = routed if cap is None else np.minimum(routed, cap)
    return out, {"logits": L, "probs": probs, "idx": idx, "w": w, "counts": kept,
                 "routed_counts": routed}


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
