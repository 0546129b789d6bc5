"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each check comes from a
value a page prints, a closed form, a special case that reduces to a library
routine (scipy's softmax, torch's silu and matmul), an invariant, or brute
force on tiny inputs. The last test plants plausible mistakes in the oracle
and shows that each one fails at least one pin.
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import moe_workloads as wl
from oracle import moe_oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _layer(T, d, ffn, E, seed=0, scale=0.02):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) * scale
    wg = rng.standard_normal((E, ffn, d)) * scale
    wu = rng.standard_normal((E, ffn, d)) * scale
    wd = rng.standard_normal((E, d, ffn)) * scale
    return x, wr, wg, wu, wd


def _torch_ffn(x, wg, wu, wd):
    """Library SwiGLU: torch's silu and matmuls in float64 on the CPU."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    G = X @ torch.from_numpy(np.asarray(wg, np.float64)).T
    U = X @ torch.from_numpy(np.asarray(wu, np.float64)).T
    return ((torch.nn.functional.silu(G) * U) @ torch.from_numpy(np.asarray(wd, np.float64)).T).numpy()


# ----------------------------------------------------------------- pins --
# Each pin takes nothing and raises AssertionError (or any error) on failure.

def pin_page_router_weights_sum(golden=None):
    """axonml test_router_route: 4 tokens of 0.1, d=64, E=8, k=2 -> each
    token's 2 weights add to 1 within 1e-5 and both indices are < 8."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "axonml_unit_expectations.json")))["router_route"]
    x = np.full((g["T"], g["d"]), g["fill"])
    wr = _rand((g["E"], g["d"]), 1, 0.02)
    p, idx, w = O.route(O.router_logits(x, wr), g["k"])
    assert idx.shape == (g["T"], g["n_indices"])
    assert np.all(idx < g["index_below"]) and np.all(idx >= 0)
    assert np.all(np.abs(w.sum(-1) - g["weight_sum"]) < g["weight_sum_tol"])
    # and on spread-out random logits, to well below the page's bound
    L = _rand((500, 8), 2, 2.0)
    _, _, w2 = O.route(L, 3)
    assert np.all(np.abs(w2.sum(-1) - 1.0) < 1e-12)


def pin_router_onehot():
    """A token that is the i-th unit vector has logits equal to column i of
    W_r (plus the bias): the router is x W_r^T with W_r stored [E, d]."""
    E, d = 5, 7
    wr = _rand((E, d), 18)
    b = _rand((E,), 19)
    assert np.array_equal(O.router_logits(np.eye(d), wr), wr.T)
    assert np.allclose(O.router_logits(np.eye(d), wr, b), wr.T + b[None, :], rtol=0, atol=1e-15)


def pin_router_bias_forces_expert():
    """A bias far above every logit on expert 3 puts it in every token's
    first slot with weight ~1; a bias far below keeps it out of every top-k."""
    T, d, E = 25, 9, 6
    x, wr = _rand((T, d), 20), _rand((E, d), 21, 0.1)
    b = np.zeros(E); b[3] = 50.0
    _, idx, w = O.route(O.router_logits(x, wr, b), 2)
    assert np.all(idx[:, 0] == 3) and np.all(w[:, 0] > 0.999)
    b[3] = -50.0
    _, idx, _ = O.route(O.router_logits(x, wr, b), 5)
    assert not np.any(idx == 3)


def pin_k2_logistic():
    """k=2 closed form: w0 = 1 / (1 + exp(L_s1 - L_s0)) and w1 = 1 - w0."""
    L = _rand((300, 8), 3, 1.5)
    _, idx, w = O.route(L, 2)
    l0 = np.take_along_axis(L, idx[:, :1], -1)[:, 0]
    l1 = np.take_along_axis(L, idx[:, 1:2], -1)[:, 0]
    w0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.allclose(w[:, 0], w0, rtol=0, atol=1e-14)
    assert np.allclose(w[:, 1], 1.0 - w0, rtol=0, atol=1e-14)


def pin_kE_is_sorted_library_softmax():
    """k=E: the renormalised weights are the full softmax (scipy) in
    descending order, and the probabilities returned are scipy's softmax,
    also for logits near +-700 where exp() of the raw value overflows."""
    for scale in (1.0, 700.0):
        L = _rand((200, 6), 4, scale)
        p, idx, w = O.route(L, 6)
        ref = scipy.special.softmax(L, axis=-1)
        assert np.all(np.isfinite(p))
        assert np.allclose(p, ref, rtol=1e-12, atol=1e-300)
        assert np.allclose(w, -np.sort(-ref, axis=-1), rtol=1e-12, atol=1e-300)


def pin_zero_router_ties():
    """W_r = 0: every logit is 0, so all experts tie; the stable order keeps
    experts 0..k-1, each with weight 1/k, and experts >= k receive nothing."""
    T, d, E, k = 37, 16, 8, 3
    x = _rand((T, d), 5)
    _, idx, w = O.route(O.router_logits(x, np.zeros((E, d))), k)
    assert np.array_equal(idx, np.tile(np.arange(k), (T, 1)))
    assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-15)
    counts, offsets, st, inv = O.permute(idx, E)
    assert list(counts) == [T] * k + [0] * (E - k)
    assert list(offsets) == [min(e, k) * T for e in range(E + 1)]


def _rank_select(L, k):
    """Brute-force selection by counting: expert e goes to slot r where r is
    the number of experts with a larger logit plus the number of lower-index
    experts with an equal one."""
    T, E = L.shape
    out = np.empty((T, k), np.int64)
    for t in range(T):
        for e in range(E):
            r = sum(1 for i in range(E) if L[t, i] > L[t, e]) + \
                sum(1 for i in range(e) if L[t, i] == L[t, e])
            if r < k:
                out[t, r] = e
    return out


def pin_selection_bruteforce():
    """Selection equals rank counting on every logit structure of the
    workload generator (random, exact ties, signed zeros, |L| up to 3e38,
    subnormals)."""
    for kind in wl.LOGIT_KINDS:
        for E, k in ((8, 2), (5, 5), (13, 4), (1, 1)):
            L = wl.make_logits(40, E, kind, seed=E)
            assert np.array_equal(O.select_top_k(L, k), _rank_select(L.astype(np.float64), k)), (kind, E, k)


def pin_permute_library():
    """Per-expert lists equal a library stable argsort of the flattened
    assignments (assignment t*k+j sorts by its expert; ties keep the token
    order), counts sum to T*k, offsets are their running sum, and inv_pos
    inverts the permutation."""
    for kind in wl.ROUTING_KINDS:
        T, E, k = 97, 8, 3
        idx, _ = wl.make_routing(T, E, k, kind, seed=1)
        counts, offsets, st, inv = O.permute(idx, E)
        flat = idx.ravel()
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(st, order // k)
        assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(np.sort(inv), np.arange(T * k))
        assert np.array_equal(st[inv], np.repeat(np.arange(T), k))
        for e in range(E):
            assert np.all(flat[order[offsets[e]:offsets[e + 1]]] == e)


def pin_permute_loops():
    """Tiny case by the page's own loop structure: for each expert, walk the
    tokens in order and append the ones that chose it."""
    T, E, k = 9, 4, 2
    idx, _ = wl.make_routing(T, E, k, "random", seed=7)
    counts, offsets, st, inv = O.permute(idx, E)
    lists = [[t for t in range(T) if e in idx[t]] for e in range(E)]
    assert list(st) == [t for l in lists for t in l]
    assert list(counts) == [len(l) for l in lists]


def pin_single_expert_is_library_ffn():
    """E=1, k=1: the layer is one SwiGLU FFN; compare with torch's silu and
    matmuls in float64 (d != ffn, so a transposed operand cannot pass)."""
    x, wr, wg, wu, wd = _layer(23, 12, 20, 1, seed=8, scale=0.3)
    out, aux = O.moe_forward(x, wr, wg, wu, wd, 1)
    assert np.allclose(aux["w"], 1.0, rtol=0, atol=0)
    ref = _torch_ffn(x, wg[0], wu[0], wd[0])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def pin_identical_experts_are_dense():
    """All experts equal: for every k (1..E), the renormalised weights add up
    to one, so the layer equals the dense library FFN."""
    x, wr, wg, wu, wd = _layer(19, 10, 14, 4, seed=9, scale=0.3)
    wg[:] = wg[0]; wu[:] = wu[0]; wd[:] = wd[0]
    ref = _torch_ffn(x, wg[0], wu[0], wd[0])
    for k in range(1, 5):
        out, _ = O.moe_forward(x, wr, wg, wu, wd, k)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-13), k


def pin_token_permutation():
    """Tokens are independent: permuting the rows of x permutes the output
    rows and the routing, and leaves the counts unchanged."""
    x, wr, wg, wu, wd = _layer(31, 8, 12, 5, seed=10, scale=0.3)
    pi = np.random.default_rng(11).permutation(31)
    o1, a1 = O.moe_forward(x, wr, wg, wu, wd, 2)
    o2, a2 = O.moe_forward(x[pi], wr, wg, wu, wd, 2)
    assert np.allclose(o2, o1[pi], rtol=1e-13, atol=1e-15)
    assert np.array_equal(a2["idx"], a1["idx"][pi])
    assert np.array_equal(a2["counts"], a1["counts"])


def pin_dense_bruteforce():
    """Gather/scatter layer == every expert on every token, masked, <= 1e-12
    relative, on random tiny layers with and without a router bias."""
    for seed, (T, d, ffn, E, k) in enumerate(((17, 8, 12, 4, 2), (9, 6, 10, 6, 6), (12, 5, 7, 3, 1))):
        x, wr, wg, wu, wd = _layer(T, d, ffn, E, seed=20 + seed, scale=0.4)
        b = _rand((E,), 30 + seed) if seed == 1 else None
        out, _ = O.moe_forward(x, wr, wg, wu, wd, k, b)
        ref = O.dense_bruteforce(x, wr, wg, wu, wd, k, b)
        assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def pin_zero_and_scaling():
    """SiLU(0) = 0 and the layer is linear in W_up and in W_down: zero gate,
    up or down weights give an exact zero output; scaling W_up or W_down by a
    power of two scales the output by it exactly (routing is unchanged)."""
    x, wr, wg, wu, wd = _layer(15, 8, 12, 4, seed=12, scale=0.3)
    for which in range(3):
        ws = [wg.copy(), wu.copy(), wd.copy()]
        ws[which][:] = 0
        out, _ = O.moe_forward(x, wr, *ws, 2)
        assert np.all(out == 0)
    base, _ = O.moe_forward(x, wr, wg, wu, wd, 2)
    up4, _ = O.moe_forward(x, wr, wg, wu * 4, wd, 2)
    dn8, _ = O.moe_forward(x, wr, wg, wu, wd * 0.125, 2)
    assert np.array_equal(up4, base * 4)
    assert np.array_equal(dn8, base * 0.125)


def pin_constant_input_utilisation():
    """axonml test_moe_expert_utilization: a [2,5,64] input of 0.1 with 4
    experts, top-2 gives 4 counts totalling 20; every token routes the same
    way, so all output rows are equal and the two chosen experts get 10."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "axonml_unit_expectations.json")))["expert_utilization"]
    T = g["batch"] * g["seq"]
    x = np.full((T, g["d"]), g["fill"])
    _, wr, wg, wu, wd = _layer(T, g["d"], g["ffn"], g["E"], seed=13)
    out, aux = O.moe_forward(x, wr, wg, wu, wd, g["k"])
    assert len(aux["counts"]) == g["n_counts"] and aux["counts"].sum() == g["total"]
    assert sorted(aux["counts"])[-g["k"]:] == [T] * g["k"]
    assert np.all(out == out[0])


def pin_load_balancing_loss():
    """Closed forms: uniform probabilities give a loss of k for any counts
    (sum f_i = k); one token gives E times the sum of its selected
    probabilities; and the page's positive-loss test on the 0.1 input."""
    T, E, k = 40, 6, 2
    idx, _ = wl.make_routing(T, E, k, "random", seed=3)
    counts = O.expert_counts(idx, E)
    assert abs(O.load_balancing_loss(np.full((T, E), 1.0 / E), counts) - k) < 1e-12
    L = _rand((1, E), 4)
    p, idx1, _ = O.route(L, 3)
    c1 = O.expert_counts(idx1, E)
    assert abs(O.load_balancing_loss(p, c1) - E * p[0, idx1[0]].sum()) < 1e-12
    x = np.full((10, 64), 0.1)
    _, wr, *_ = _layer(10, 64, 8, 4, seed=14)
    p2, i2, _ = O.route(O.router_logits(x, wr), 2)
    assert O.load_balancing_loss(p2, O.expert_counts(i2, 4)) > 0.0
    assert O.load_balancing_loss(np.zeros((0, 4)), np.zeros(4)) == 0.0
    # full collapse: every token puts all probability on expert 2 and is
    # routed there (k = 1): f_2 = P_2 = 1, so the loss is E
    onehot = np.zeros((T, E))
    onehot[:, 2] = 1.0
    assert O.load_balancing_loss(onehot, np.eye(E)[2] * T) == E


def pin_bf16_widening():
    """bfloat16 bit patterns widen to their exact values."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x8000, 0x7F7F, 0x3EAB], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, -0.0, 3.3895313892515355e38, 0.333984375]
    got = O.widen(bits)
    assert list(got) == want
    assert np.signbit(got[3])


def pin_capacity_bruteforce():
    """Each expert keeps the first C tokens (ascending) that chose it, found
    by walking the tokens with a counter per expert; the kept rows are laid
    out expert by expert. C = ceil(cf * T * k / E); a factor of 0 means no
    limit (KempnerForge: 0 = no drop)."""
    T, E, k = 50, 5, 2
    idx, _ = wl.make_routing(T, E, k, "one_heavy", seed=2)
    assert O.capacity(T, E, k, 0.0) is None
    assert O.capacity(T, E, k, 1.0) == 20 and O.capacity(T, E, k, 0.26) == 6
    for cf in (0.26, 0.5, 1.0, 1.25):
        cap = O.capacity(T, E, k, cf)
        counts, offsets, st, inv = O.permute(idx, E, cap)
        seen = [0] * E
        want_rows = [[] for _ in range(E)]
        kept = np.zeros((T, k), bool)
        for t in range(T):
            for j in range(k):
                e = int(idx[t, j])
                if seen[e] < cap:
                    kept[t, j] = True
                    want_rows[e].append(t)
                seen[e] += 1
        assert [len(r) for r in want_rows] == list(counts)
        assert list(st) == [t for r in want_rows for t in r]
        assert offsets[-1] == kept.sum() == len(st)
        for t in range(T):
            for j in range(k):
                p = inv[t * k + j]
                if kept[t, j]:
                    assert st[p] == t and offsets[idx[t, j]] <= p < offsets[idx[t, j] + 1]
                else:
                    assert p == -1
    # a cap at or above every count changes nothing
    big = O.capacity(T, E, k, 10.0)
    for a, b in zip(O.permute(idx, E, big), O.permute(idx, E)):
        assert np.array_equal(a, b)


def pin_capacity_constant_input():
    """Identical tokens all choose the same k experts, so with capacity C
    exactly the first C tokens keep their outputs and the rest get zero."""
    T, d, ffn, E, k = 24, 32, 16, 4, 2
    x = np.full((T, d), 0.1)
    _, wr, wg, wu, wd = _layer(T, d, ffn, E, seed=21)
    full, _ = O.moe_forward(x, wr, wg, wu, wd, k)
    cf = 0.5                      # C = ceil(0.5 * 24 * 2 / 4) = 6
    out, aux = O.moe_forward(x, wr, wg, wu, wd, k, capacity_factor=cf)
    assert O.capacity(T, E, k, cf) == 6
    assert np.array_equal(out[:6], full[:6]) and not out[6:].any()
    assert sorted(aux["counts"][aux["counts"] > 0]) == [6, 6]
    assert sorted(aux["routed_counts"][aux["routed_counts"] > 0]) == [T, T]


def pin_rms_norm_library():
    """The norm equals torch's rms_norm (float64, CPU), is invariant to
    scaling the input when eps = 0, and maps a constant row c to
    c / sqrt(c^2 + eps) times the weight."""
    x = _rand((7, 48), 31) * 3.0
    g = _rand((48,), 32)
    for eps in (1e-5, 1e-2, 0.0):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g),
                                            eps).numpy()
        np.testing.assert_allclose(O.rms_norm(x, g, eps), want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O.rms_norm(8.0 * x, g, 0.0), O.rms_norm(x, g, 0.0), rtol=1e-14)
    c = np.full((1, 16), 0.5)
    np.testing.assert_allclose(O.rms_norm(c, np.ones(16), 0.04), np.full((1, 16), 0.5 / 0.53851648071345),
                               rtol=1e-12)


def pin_round_to_bf16():
    """Rounding to bf16 equals torch's float32 -> bfloat16 conversion on
    float32 values (one rounding either way), and ties go to even."""
    a = (_rand((4000,), 51) * np.exp(_rand((4000,), 52) * 4.0)).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(a.astype(np.float64)), want)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(2 + 2.0 ** -7), 0.0, 2.0 ** -130 * 0])
    assert list(O.round_to_bf16(ties)) == [1.0, 1 + 2.0 ** -6, -2.0, 0.0, 0.0]


def pin_residual_and_shared():
    """With W_down = 0 the block returns its input exactly; shared experts
    add torch's SwiGLU of the normalised input; the residual is the
    un-normalised input."""
    T, d, ffn, E, k = 20, 32, 24, 4, 2
    x, wr, wg, wu, wd = _layer(T, d, ffn, E, seed=41)
    g = 1.0 + _rand((d,), 42, 0.1)
    out, _ = O.moe_forward(x, wr, wg, wu, np.zeros_like(wd), k, norm_weight=g, norm_eps=1e-5,
                           residual=True)
    assert np.array_equal(out, x)
    rng = np.random.default_rng(43)
    sg, su = rng.standard_normal((2, 12, d)) * 0.02, rng.standard_normal((2, 12, d)) * 0.02
    sd = rng.standard_normal((2, d, 12)) * 0.02
    base, _ = O.moe_forward(x, wr, wg, wu, wd, k, norm_weight=g, norm_eps=1e-5)
    withs, _ = O.moe_forward(x, wr, wg, wu, wd, k, norm_weight=g, norm_eps=1e-5, residual=True,
                             shared=(sg, su, sd))
    xn = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), 1e-5).numpy()
    want = base + x + _torch_ffn(xn, sg[0], su[0], sd[0]) + _torch_ffn(xn, sg[1], su[1], sd[1])
    np.testing.assert_allclose(withs, want, rtol=1e-12, atol=1e-14)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_page_values_shapes(golden):
    """Shapes and counts the pages print: [2,5,64] in and out, 25 weight
    tensors for 8 experts, the Mixtral block's 1.45B parameters (only reached
    with 3-matrix gated experts), and the expert widths of the sizing rules."""
    g = golden("axonml_unit_expectations.json")
    s = g["layer_shape"]
    B, S, d = s["in_shape"]
    x = np.full((B * S, d), 0.1)
    _, wr, wg, wu, wd = _layer(B * S, d, s["ffn"], s["E"], seed=15)
    out, _ = O.moe_forward(x, wr, wg, wu, wd, s["k"])
    assert list(out.reshape(B, S, d).shape) == s["out_shape"]
    pc = g["parameter_count"]
    assert pc["router_tensors"] + pc["E"] * pc["tensors_per_expert"] == pc["total"]

    m = golden("mixtral_block.json")
    D, F, E = m["dim"], m["expert_ffn"], m["experts"]
    attn = 2 * D * m["q_out"] + 2 * D * m["kv_out"]
    gated = attn + E * 3 * D * F + D * E + m["norms"] * D
    ungated = attn + E * 2 * D * F + D * E + m["norms"] * D
    assert round(gated / 1e9, 2) == m["params_billions_rounded"]
    assert round(ungated / 1e9, 2) != m["params_billions_rounded"]
    p = wl.WORKLOADS["prefill"]
    assert (p.d, p.ffn, p.E, p.k) == (D, F, E, m["top_k"])
    assert p.T == m["io_shape"][1]

    f = golden("kempnerforge_ffn_sizes.json")
    for c in f["cases"]:
        got = wl.expert_ffn_hidden_dim(wl.ffn_hidden_dim(c["dim"], c["ffn_dim_multiplier"]),
                                       c["expert_multiplier"])
        assert got == c["expert_ffn"], c
    assert wl.WORKLOADS["small"].ffn == 2816 and wl.WORKLOADS["skewed"].ffn == 1408


def test_invalid_top_k_rejected():
    """ModelConfig validation and MoERouter::new: k must be in 1..E."""
    L = _rand((3, 4), 16)
    for k in (0, 5):
        with pytest.raises(AssertionError):
            O.select_top_k(L, k)


def test_nonfinite_rejected():
    """axonml's sort cannot order NaN; the oracle refuses non-finite logits."""
    L = _rand((3, 4), 17)
    L[1, 2] = np.nan
    with pytest.raises(AssertionError):
        O.route(L, 2)


# ------------------------------------------------------ planted mistakes --

def _m_no_renorm(p, idx):
    return np.take_along_axis(O.widen(p), np.asarray(idx), -1)


def _m_gate_sum_combine(T, d, idx, w, rows):
    out = np.zeros((T, d))
    for e, (tok, Y) in rows.items():
        out[tok] += O.widen(w)[tok].sum(-1, keepdims=True) * Y
    return out


def _m_silu_on_up(X, wg, wu, wd):
    X = O.widen(X)
    G = X @ O.widen(wg).T
    U = X @ O.widen(wu).T
    return (G * (U / (1 + np.exp(-U)))) @ O.widen(wd).T


def _m_sigmoid_sign(X, wg, wu, wd):
    X = O.widen(X)
    G = X @ O.widen(wg).T
    return ((G / (1 + np.exp(G))) * (X @ O.widen(wu).T)) @ O.widen(wd).T


def _m_ties_high_index(L, k):
    L = O.widen(L)
    E = L.shape[-1]
    o = np.argsort(-L[:, ::-1], axis=-1, kind="stable")
    return (E - 1 - o)[:, :k]


def _m_ascending(L, k):
    return np.argsort(O.widen(L), axis=-1, kind="stable")[:, :k]


def _m_softmax_no_shift(L):
    z = np.exp(O.widen(L))
    return z / z.sum(-1, keepdims=True)


def _m_permute_desc(idx, E):
    c, off, st, inv = _REAL["permute"](idx, E)
    k = np.asarray(idx).shape[1]
    st2 = st.copy()
    for e in range(E):
        st2[off[e]:off[e + 1]] = st[off[e]:off[e + 1]][::-1]
    return c, off, st2, inv


def _m_bias_sign(x, wr, bias=None):
    L = O.widen(x) @ O.widen(wr).T
    return L if bias is None else L - O.widen(bias)[None]


def _m_router_transposed_scale(x, wr, bias=None):
    L = O.widen(x) @ O.widen(wr).T
    return L / np.sqrt(L.shape[-1])


def _m_offsets_inclusive(idx, E):
    c, off, st, inv = _REAL["permute"](idx, E)
    return c, np.concatenate([np.cumsum(c), [c.sum()]]), st, inv


_REAL = {"permute": O.permute}

def _m_round_half_up(a):
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.floor(m * 256.0 + 0.5) / 256.0, e)


_orig_capacity, _orig_permute, _orig_rms, _orig_shared, _orig_ffn = (
    O.capacity, O.permute, O.rms_norm, O.shared_experts, O.expert_ffn)


def _m_capacity_floor(T, E, k, cf):
    return None if cf == 0 else int(np.floor(cf * T * k / E))


def _m_capacity_plus_one(T, E, k, cf):
    c = _orig_capacity(T, E, k, cf)
    return None if c is None else c + 1


def _m_permute_keeps_last(idx, E, cap=None):
    if cap is None:
        return _orig_permute(idx, E)
    # keep the last cap tokens of each expert instead of the first
    idx = np.asarray(idx)
    T, k = idx.shape
    rev = idx[::-1]
    counts, offsets, st, inv = _orig_permute(rev, E, cap)
    st = (T - 1 - st)
    return counts, offsets, st, inv


def _m_rms_eps_outside(x, weight, eps):
    xw = O.widen(x)
    return xw / (np.sqrt(np.mean(xw * xw, axis=-1, keepdims=True)) + eps) * O.widen(weight)


def _m_shared_half(x, a, b, c):
    return 0.5 * _orig_shared(x, a, b, c)


def _m_ffn_ignores_cap(x, idx, w, wg, wu, wd, E=None, cap=None):
    return _orig_ffn(x, idx, w, wg, wu, wd, E)


MUTANTS = {
    "capacity_floor": ("capacity", _m_capacity_floor),
    "capacity_plus_one": ("capacity", _m_capacity_plus_one),
    "permute_keeps_last": ("permute", _m_permute_keeps_last),
    "rms_eps_outside_root": ("rms_norm", _m_rms_eps_outside),
    "shared_half_weight": ("shared_experts", _m_shared_half),
    "ffn_ignores_capacity": ("expert_ffn", _m_ffn_ignores_cap),
    "bf16_round_half_up": ("round_to_bf16", _m_round_half_up),
    "no_renormalisation": ("renormalise", _m_no_renorm),
    "gate_sum_combine": ("combine", _m_gate_sum_combine),
    "silu_on_up": ("swiglu_expert", _m_silu_on_up),
    "sigmoid_sign": ("swiglu_expert", _m_sigmoid_sign),
    "ties_to_high_index": ("select_top_k", _m_ties_high_index),
    "ascending_topk": ("select_top_k", _m_ascending),
    "softmax_no_shift": ("softmax", _m_softmax_no_shift),
    "permute_descending_tokens": ("permute", _m_permute_desc),
    "router_bias_sign": ("router_logits", _m_bias_sign),
    "router_scaled": ("router_logits", _m_router_transposed_scale),
    "offsets_inclusive": ("permute", _m_offsets_inclusive),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # any failure of a pin counts
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
