"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Bars (written in each test): routing indices, counts, offsets and the
permutation bit-exact when both sides get the same fp32 logits; gate weights
and probabilities within 1e-6; layer outputs within 1e-4 x RMS (fp32
workloads) or 2e-2 x RMS (bf16 workloads) of the fp64 oracle, max-abs over
every compared element; bit-identical results on repeated calls.
"""
import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as O
from parity_util import (check_slot_order, compare_layer, dev_tensor, host, logit_tolerance,
                         routing_alternatives, say)

pytestmark = pytest.mark.gpu

REL_TOL = {"f32": 1e-4, "bf16": 2e-2}
# bf16 layers narrower than 1024 in d or ffn carry h into the down pass as two
# bf16 terms (include/moe.h); rounding h then no longer moves the output, and
# the rest (fp32 sums, the SiLU's ulps) stays far inside this bound
TWO_TERM_TOL = 1e-3


def two_term(d, ffn, dtype):
    return dtype == "bf16" and (d < 1024 or ffn < 1024)


def layer_tol(d, ffn, dtype):
    return TWO_TERM_TOL if two_term(d, ffn, dtype) else REL_TOL[dtype]


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_renorm_amd as m
    m.lib()
    return m


# ------------------------------------------------------------ routing --

ROUTE_SHAPES = [(1, 1, 1), (37, 4, 2), (300, 8, 2), (129, 13, 5), (77, 64, 8), (33, 256, 16),
                (64, 8, 8), (1000, 2, 1)]


@pytest.mark.parametrize("kind", wl.LOGIT_KINDS)
@pytest.mark.parametrize("T,E,k", ROUTE_SHAPES)
def test_route_logits_bitexact(M, kind, T, E, k):
    say(f"moe_route_logits kind={kind} T={T} E={E} k={k}")
    L = wl.make_logits(T, E, kind, seed=T + E)
    idx, w, p = M.moe_route_logits(dev_tensor(L), k, probs=True)
    torch.cuda.synchronize()
    p_ref, idx_ref, w_ref = O.route(L, k)
    assert np.array_equal(host(idx), idx_ref), "indices differ"
    assert np.max(np.abs(host(w) - w_ref)) <= 1e-6
    assert np.max(np.abs(host(p) - p_ref)) <= 1e-6


@pytest.mark.parametrize("kind", wl.ROUTING_KINDS)
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (513, 8, 2), (3000, 64, 8),
                                   (100, 256, 16), (700, 6, 3), (5000, 1, 1), (8192, 64, 8),
                                   (70000, 8, 2), (300000, 4, 1),
                                   # around the one-pass kernel's limits (4096
                                   # assignments, 64 experts)
                                   (2048, 8, 2), (2049, 8, 2), (512, 64, 8), (500, 65, 8),
                                   (100, 32, 16)])
def test_permute_bitexact(M, kind, T, E, k):
    if kind == "even_only" and 2 * k > E:
        pytest.skip("needs 2k <= E")
    if kind == "one_heavy" and E < 2 and k > 1:
        pytest.skip("needs E >= 2")
    say(f"moe_permute kind={kind} T={T} E={E} k={k}")
    idx, w = wl.make_routing(T, E, k, kind, seed=T)
    counts, offsets, st, inv, sw = M.moe_permute(dev_tensor(idx), E, topk_w=dev_tensor(w))
    torch.cuda.synchronize()
    c_ref, o_ref, st_ref, inv_ref = O.permute(idx, E)
    assert np.array_equal(host(counts), c_ref)
    assert np.array_equal(host(offsets), o_ref)
    assert np.array_equal(host(st), st_ref)
    assert np.array_equal(host(inv), inv_ref)
    # the weights in permuted order, bit for bit: row inv_ref[i] holds w[i]
    sw_ref = np.empty(T * k, np.float32)
    sw_ref[inv_ref] = w.reshape(-1)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,E,k,bias", [(64, 64, 4, 2, False), (300, 256, 8, 2, False),
                                          (1000, 2048, 64, 8, True), (31, 4096, 8, 2, False),
                                          (20, 112, 200, 16, True),
                                          # one workgroup per token (at most 64 tokens and
                                          # 16 experts): minimal width, widths past one load
                                          # round, k = E, and the first batch above the limit
                                          (1, 16, 16, 4, True), (64, 8192, 12, 3, True),
                                          (33, 2080, 16, 16, False), (65, 512, 8, 2, False)])
def test_route_fused(M, dtype, T, d, E, k, bias):
    say(f"moe_route dtype={dtype} T={T} d={d} E={E} k={k} bias={bias}")
    inp = wl.make_custom_inputs(T, d, 16, E, dtype, seed=3, bias=bias)
    x, wr, b = inp["x"], inp["w_router"], inp["router_bias"]
    r = M.moe_route(dev_tensor(x), dev_tensor(wr), k, router_bias=dev_tensor(b),
                    want_logits=True, want_probs=True)
    torch.cuda.synchronize()
    L_ref = O.router_logits(x, wr, b)
    tol = logit_tolerance(x, wr)
    L_gpu = host(r["logits"]).astype(np.float64)
    assert np.all(np.abs(L_gpu - L_ref) <= tol), f"max logit err {np.abs(L_gpu - L_ref).max():.3e}"
    # routing: the oracle's own logits decide; tokens whose k-th and (k+1)-th
    # logits are within the tolerance band may take either expert
    alts = routing_alternatives(L_ref, k, tol)
    gi = host(r["topk_idx"])
    check_slot_order(gi, L_ref, tol)
    p_ref, idx_ref, w_ref = O.route(L_ref, k)
    for t in range(T):
        assert tuple(sorted(gi[t].tolist())) in alts[t], (t, gi[t], alts[t])
    # weights and probabilities: fp32 rounding plus the logit error
    # (d p / d L is at most 1/2 per unit of logit), on unambiguous tokens
    sure = [t for t in range(T) if len(alts[t]) == 1 and np.array_equal(gi[t], idx_ref[t])]
    slack = 1e-6 + tol.max(axis=1)[sure, None]
    assert np.all(np.abs(host(r["topk_w"])[sure] - w_ref[sure]) <= slack)
    assert np.all(np.abs(host(r["probs"])[sure] - p_ref[sure]) <= slack)


# ------------------------------------------------------- expert path --

EXPERT_SHAPES = [
    # T, d, ffn, E, k, dtype, routing kind
    (64, 64, 128, 4, 2, "f32", "random"),
    # fp32 MFMA tiles (128 x 128): several row and column tiles with ragged
    # ends in both passes, long reductions, empty and light experts
    (700, 272, 336, 5, 2, "f32", "random"),
    (300, 1040, 2064, 3, 2, "f32", "one_heavy"),
    (50, 128, 64, 8, 1, "f32", "even_only"),
    (300, 256, 320, 8, 2, "bf16", "random"),
    (257, 272, 336, 8, 2, "bf16", "random"),      # ragged K and N tails
    (200, 128, 192, 8, 3, "bf16", "all_same"),    # experts 3..7 empty
    (333, 128, 256, 8, 2, "bf16", "even_only"),   # odd experts empty
    (150, 192, 160, 6, 3, "bf16", "one_heavy"),   # one expert takes every token
    (1, 64, 64, 4, 2, "bf16", "random"),
    (40, 64, 96, 1, 1, "bf16", "random"),
    (90, 96, 112, 5, 5, "bf16", "random"),       # k = E
    # at most 32 rows per expert on average: the weight-streaming kernels
    (40, 272, 336, 4, 2, "bf16", "random"),      # ragged K tails on both passes
    (60, 128, 192, 4, 2, "bf16", "all_same"),    # 60 rows on experts 0 and 1 (two row blocks)
    (16, 64, 96, 8, 1, "bf16", "one_heavy"),     # k = 1, every token on expert 7
    # streaming path with an expert above 64 rows: that expert goes to a tile
    # launch after the streaming one (instead of reading its weights once per
    # 32 rows)
    (256, 64, 96, 8, 1, "bf16", "one_heavy"),    # all 256 rows on expert 7
    (128, 256, 320, 8, 2, "bf16", "one_heavy"),  # expert 7 tiled (two-term h), the rest streamed
    (100, 1024, 1024, 4, 1, "bf16", "all_same"),  # one-term h, all 100 rows on expert 0
    (32, 4096, 14336, 8, 2, "bf16", "random"),   # decode shape
    # at least 768 rows per expert on average: the tall-tile kernels
    (3200, 256, 320, 4, 1, "bf16", "random"),
    (1600, 272, 336, 2, 2, "bf16", "random"),    # ragged K and N tails on both passes
    (1700, 128, 192, 3, 3, "bf16", "one_heavy"),  # k = E
    (2000, 128, 256, 4, 2, "bf16", "all_same"),  # 2000 rows on experts 0 and 1, the rest empty
    # long reductions with a tail (6160 = 96 * 64 + 16): the down pass splits its
    # reduction and the last step of each part reads past K
    (1600, 256, 6160, 2, 1, "bf16", "random"),   # tall tiles
    (600, 128, 6160, 2, 1, "bf16", "random"),    # 256 x 256 tiles
    # many experts: the tile map's prefix over up to 256 experts (four per lane)
    (4000, 64, 128, 256, 4, "bf16", "random"),   # 256 x 256 tiles, E at the limit
    (3000, 64, 96, 130, 8, "bf16", "random"),    # E not a multiple of four
    (9600, 64, 96, 100, 8, "bf16", "random"),    # tall tiles
    # widths of 1024 and more: h as one bf16 term (the shapes above use two),
    # with reduction tails (1040 = 16 * 64 + 16) in both passes
    (40, 1040, 1040, 4, 2, "bf16", "random"),    # weight-streaming kernels
    (600, 1040, 1104, 4, 2, "bf16", "random"),   # 256 x 256 tiles
    (2000, 1040, 1040, 2, 1, "bf16", "random"),  # tall tiles
    (1500, 1024, 1024, 2, 2, "bf16", "one_heavy"),  # tall tiles, no tails, one expert empty
    # tall down tiles with a part table: a reduction long enough to split and
    # so few tiles that every one runs as two halves (2064 = 32 * 64 + 16:
    # the second half ends in a tail)
    (800, 1024, 2064, 2, 2, "bf16", "random"),
]


@pytest.mark.parametrize("T,d,ffn,E,k,dtype,kind", EXPERT_SHAPES)
def test_expert_ffn_parity(M, T, d, ffn, E, k, dtype, kind):
    say(f"moe_expert_ffn T={T} d={d} ffn={ffn} E={E} k={k} {dtype} {kind}")
    inp = wl.make_custom_inputs(T, d, ffn, E, dtype, seed=5)
    idx, w = wl.make_routing(T, E, k, kind, seed=6)
    args = [dev_tensor(inp[n]) for n in ("w_gate", "w_up", "w_down")]
    out = M.moe_expert_ffn(dev_tensor(inp["x"]), dev_tensor(idx), dev_tensor(w), *args)
    torch.cuda.synchronize()
    ref = O.expert_ffn(inp["x"], idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], E)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(host(out).astype(np.float64) - ref).max()
    assert err <= layer_tol(d, ffn, dtype) * rms, f"max err {err / rms:.3e} x RMS"


# Row counts per expert around the tile heights: the grouped GEMMs cut an
# expert's rows into ceil(rows / tile height) row tiles of nearly equal height
# (whole 32-row blocks), and a wave skips the MFMAs of blocks past the tile's
# rows. k = 1, so each token's output is its one expert's row.
ROW_SPLITS = [
    # counts per expert, d, ffn
    ([769, 1537], 128, 192),                 # tall tiles: 8/8/9 and 9/10/10/10/10 blocks
    ([384, 385, 1151, 1153], 64, 96),        # tall tiles: exactly one tile, one row more, 3 and 4 tiles
    ([257, 511, 512, 513, 31, 33], 64, 96),  # 256 x 256 tiles
    ([1, 32, 33, 800], 64, 96),              # tiny experts beside a large one
    # tall tiles with light experts beside a heavy one (tiles of 1 to 129 rows)
    ([5000, 100, 20, 1, 128, 129], 64, 128),
    ([4000, 1, 65, 128, 129], 1040, 1024),   # one-term h, reduction tails
]


@pytest.mark.parametrize("counts,d,ffn", ROW_SPLITS)
def test_expert_ffn_row_splits(M, counts, d, ffn):
    E, T = len(counts), sum(counts)
    say(f"moe_expert_ffn row splits counts={counts} d={d} ffn={ffn}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=8)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(9).shuffle(idx)
    idx = idx.reshape(T, 1)
    w = np.ones((T, 1), dtype=np.float32)
    args = [dev_tensor(inp[n]) for n in ("w_gate", "w_up", "w_down")]
    out = M.moe_expert_ffn(dev_tensor(inp["x"]), dev_tensor(idx), dev_tensor(w), *args)
    torch.cuda.synchronize()
    ref = O.expert_ffn(inp["x"], idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], E)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(host(out).astype(np.float64) - ref).max()
    assert err <= layer_tol(d, ffn, "bf16") * rms, f"max err {err / rms:.3e} x RMS"


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 13, 16, 32, 64]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([rng.integers(1, 40), rng.integers(40, 600)]))
        yield (T, int(16 * rng.integers(1, 17)), int(16 * rng.integers(1, 17)), E, k)


@pytest.mark.parametrize("T,d,ffn,E,k", list(_random_shapes(30, 2024)))
def test_expert_ffn_random_shapes_f32(M, T, d, ffn, E, k):
    say(f"moe_expert_ffn f32 random shape T={T} d={d} ffn={ffn} E={E} k={k}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "f32", seed=T + d)
    idx, w = wl.make_routing(T, E, k, "random", seed=ffn + E)
    args = [dev_tensor(inp[n]) for n in ("w_gate", "w_up", "w_down")]
    out = M.moe_expert_ffn(dev_tensor(inp["x"]), dev_tensor(idx), dev_tensor(w), *args)
    torch.cuda.synchronize()
    ref = O.expert_ffn(inp["x"], idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], E)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(host(out).astype(np.float64) - ref).max()
    assert err <= REL_TOL["f32"] * rms, f"max err {err / rms:.3e} x RMS"


@pytest.mark.parametrize("T,d,ffn,E,k", list(_random_shapes(40, 4048)))
def test_expert_ffn_random_shapes_bf16(M, T, d, ffn, E, k):
    """Random bf16 shapes (widths 16-256, so h goes to the down pass as two
    bf16 terms), element by element against the oracle: every element within
    2e-2 x RMS, and within the two-term bound."""
    say(f"moe_expert_ffn bf16 random shape T={T} d={d} ffn={ffn} E={E} k={k}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=T + d)
    idx, w = wl.make_routing(T, E, k, "random", seed=ffn + E)
    args = [dev_tensor(inp[n]) for n in ("w_gate", "w_up", "w_down")]
    out = M.moe_expert_ffn(dev_tensor(inp["x"]), dev_tensor(idx), dev_tensor(w), *args)
    torch.cuda.synchronize()
    ref = O.expert_ffn(inp["x"], idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], E)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(host(out).astype(np.float64) - ref)
    assert np.all(err <= REL_TOL["bf16"] * rms), f"max err {err.max() / rms:.3e} x RMS"
    assert np.all(err <= layer_tol(d, ffn, "bf16") * rms), f"max err {err.max() / rms:.3e} x RMS"


def _wide_random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        E = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 600))
        yield (T, int(16 * rng.integers(64, 129)), int(16 * rng.integers(64, 129)), E, k)


@pytest.mark.parametrize("T,d,ffn,E,k", list(_wide_random_shapes(12, 77)))
def test_expert_ffn_random_wide_shapes_bf16(M, T, d, ffn, E, k):
    """Random bf16 shapes with both widths 1024-2048 (h as one bf16 term):
    every element within 2e-2 x RMS of the oracle."""
    say(f"moe_expert_ffn bf16 wide random shape T={T} d={d} ffn={ffn} E={E} k={k}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=T + d)
    idx, w = wl.make_routing(T, E, k, "random", seed=ffn + E)
    args = [dev_tensor(inp[n]) for n in ("w_gate", "w_up", "w_down")]
    out = M.moe_expert_ffn(dev_tensor(inp["x"]), dev_tensor(idx), dev_tensor(w), *args)
    torch.cuda.synchronize()
    ref = O.expert_ffn(inp["x"], idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], E)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(host(out).astype(np.float64) - ref)
    assert np.all(err <= REL_TOL["bf16"] * rms), f"max err {err.max() / rms:.3e} x RMS"


# -------------------------------------------------------- whole layer --

@pytest.mark.parametrize("name", ["tiny", "small"])
def test_forward_parity_workload(M, name):
    w = wl.WORKLOADS[name]
    say(f"moe_forward workload={name} T={w.T} d={w.d} ffn={w.ffn} E={w.E} k={w.k}")
    inp = wl.make_layer_inputs(w, seed=0)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out, ex = M.moe_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k,
                            router_bias=dv["router_bias"], want_counts=True)
    torch.cuda.synchronize()
    st = compare_layer(host(out), inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                       inp["w_down"], w.k, inp["router_bias"], REL_TOL[w.dtype])
    say(f"  {name}: max err {st['max_rel_err']:.3e} x RMS, near-ties {st['near_ties']}")
    # expert counts: exact unless a near-tie token moved between experts
    diff = np.abs(host(ex["counts"]).astype(np.int64) - O.expert_counts(st["ref_idx"], w.E))
    assert diff.sum() <= 2 * st["near_ties"]


@pytest.mark.parametrize("T,d,ffn,E,k,bias", [(1, 64, 64, 4, 2, False), (129, 128, 176, 8, 2, True),
                                              (700, 256, 512, 16, 4, True)])
def test_forward_parity_shapes(M, T, d, ffn, E, k, bias):
    say(f"moe_forward T={T} d={d} ffn={ffn} E={E} k={k} bias={bias}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=9, bias=bias)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out = M.moe_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], k,
                        router_bias=dv["router_bias"])
    torch.cuda.synchronize()
    compare_layer(host(out), inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                  k, inp["router_bias"], layer_tol(d, ffn, "bf16"))


# Decode-sized bf16 batches (at most 256 assignments on the weight-streaming
# path): the gate/up stream kernel ranks each expert's assignments itself and
# writes the permutation that the down pass and the combine read; the counts
# come from the same place. Around it: 264 assignments (separate permutation
# kernel), E at its limit, and experts above 64 rows, whose tile launch reads
# the permutation the stream kernel wrote.
DECODE_SIZED = [
    # T, d, ffn, E, k, router bias (None, or (expert, bias) pairs)
    (32, 128, 192, 8, 2, None),
    (128, 64, 96, 8, 2, None),          # 256 assignments, the limit
    (132, 64, 96, 16, 2, None),         # 264: streamed, permutation kernel
    (40, 64, 96, 64, 6, None),
    (16, 64, 96, 256, 16, None),        # E = 256, 256 assignments
    (128, 64, 96, 8, 2, ((3, 60.0), (5, 30.0))),  # every token on experts 3 and 5: both tiled
    (100, 1024, 1024, 4, 1, ((2, 60.0),)),        # one-term h, all 100 rows on expert 2
]


@pytest.mark.parametrize("T,d,ffn,E,k,bias", DECODE_SIZED)
def test_forward_decode_sized(M, T, d, ffn, E, k, bias):
    say(f"moe_forward decode-sized T={T} d={d} ffn={ffn} E={E} k={k} bias={bias}")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=11)
    if bias is not None:
        b = np.zeros(E, dtype=np.float32)
        for e, v in bias:
            b[e] = v
        inp["router_bias"] = b
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out, ex = M.moe_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], k,
                            router_bias=dv["router_bias"], want_counts=True)
    torch.cuda.synchronize()
    st = compare_layer(host(out), inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                       inp["w_down"], k, inp["router_bias"], layer_tol(d, ffn, "bf16"))
    diff = np.abs(host(ex["counts"]).astype(np.int64) - O.expert_counts(st["ref_idx"], E))
    assert diff.sum() <= 2 * st["near_ties"]
    if bias is not None and st["near_ties"] == 0:
        assert all(host(ex["counts"])[e] == T for e, _ in bias)


def test_forward_zero_tokens(M):
    say("moe_forward T=0")
    inp = wl.make_custom_inputs(4, 64, 64, 4, "bf16")
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    x0 = dv["x"][:0]
    out = M.moe_forward(x0, dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], 2)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_forward_deterministic_and_permutation(M):
    """Two calls are bit-identical; permuting the tokens permutes the output
    rows bit-exactly (tokens are independent, combine sums in slot order)."""
    w = wl.WORKLOADS["small"]
    say("moe_forward determinism / token permutation (small workload)")
    inp = wl.make_layer_inputs(w, seed=1)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    args = (dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k)
    o1 = M.moe_forward(dv["x"], *args)
    o2 = M.moe_forward(dv["x"], *args)
    pi = torch.from_numpy(np.random.default_rng(0).permutation(w.T)).cuda()
    o3 = M.moe_forward(dv["x"][pi].contiguous(), *args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o3, o1[pi])


def test_forward_bf16_output(M):
    """bf16 output = the fp32 output rounded once (within 1 bf16 ulp)."""
    w = wl.WORKLOADS["small"]
    say("moe_forward bf16 output (small workload)")
    inp = wl.make_layer_inputs(w, seed=2)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    args = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k)
    o32 = M.moe_forward(*args).double()
    o16 = M.moe_forward(*args, out_dtype=torch.bfloat16).double()
    torch.cuda.synchronize()
    ulp = torch.abs(o32) * 2.0 ** -7 + 1e-30
    assert torch.all(torch.abs(o16 - o32) <= ulp)


def test_constant_input_identical_rows(M):
    """The pages' unit-test input (every entry 0.1): every token routes the
    same way, all k chosen experts get T rows, and all output rows match."""
    T, d, ffn, E, k = 10, 64, 256, 4, 2
    say("moe_forward constant 0.1 input")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=4)
    x = wl.f32_to_bf16_bits(np.full((T, d), 0.1, np.float32))
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out, ex = M.moe_forward(dev_tensor(x), dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                            k, want_counts=True)
    torch.cuda.synchronize()
    c = host(ex["counts"])
    assert c.sum() == T * k and sorted(c)[-k:] == [T] * k
    o = host(out)
    assert np.all(o == o[0])
