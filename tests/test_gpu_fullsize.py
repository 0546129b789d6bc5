"""Parity at the full workload sizes, in the launch configuration the
benchmark times (bf16 inputs, fp32 output, one caller workspace).

The layer test evaluates every token with the oracle (a few seconds of
numpy at these sizes), with the same near-tie protocol as the small tests;
the block-option and largest-batch tests evaluate seeded samples of tokens
(tokens are independent: no capacity limit reached). Whole-batch properties are checked exactly: the expert counts
add up to T*k and match the oracle's counts except where a near-tie token
moved, and two calls give bit-identical outputs.
"""
import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as O
from parity_util import compare_layer, dev_tensor, host, logit_tolerance, routing_alternatives, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_renorm_amd as m
    m.lib()
    return m


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill", "skewed"])
def test_fullsize_parity(M, name):
    w = wl.WORKLOADS[name]
    say(f"full-size {name}: T={w.T} d={w.d} ffn={w.ffn} E={w.E} k={w.k}; generating inputs")
    inp = wl.make_layer_inputs(w, seed=0)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    ws = M.workspace(w.T, w.d, w.ffn, w.E, w.k, torch.bfloat16)
    args = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k)
    say(f"full-size {name}: moe_forward x2")
    o1, ex = M.moe_forward(*args, router_bias=dv["router_bias"], out=out, ws=ws, want_counts=True)
    o1 = o1.clone()
    o2 = M.moe_forward(*args, router_bias=dv["router_bias"], out=out, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "two calls differ"
    got = host(o1)
    counts = host(ex["counts"]).astype(np.int64)
    assert counts.sum() == w.T * w.k

    # whole-batch routing from the oracle's own logits
    L = O.router_logits(inp["x"], inp["w_router"], inp["router_bias"])
    tol = logit_tolerance(inp["x"], inp["w_router"])
    _, idx, _ = O.route(L, w.k)
    near = sum(1 for a in routing_alternatives(L, w.k, tol) if len(a) > 1)
    diff = np.abs(counts - O.expert_counts(idx, w.E)).sum()
    say(f"full-size {name}: counts {counts.tolist()[:16]}..., near-ties {near}, count diff {diff}")
    assert diff <= 2 * near

    say(f"full-size {name}: oracle on all {w.T} tokens")
    st = compare_layer(got, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                       inp["w_down"], w.k, inp["router_bias"], 2e-2)
    say(f"full-size {name}: max err {st['max_rel_err']:.3e} x RMS (bar 2e-2), "
        f"near-ties {st['near_ties']}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fullsize_block_options(M, name):
    """The extended forward in the configuration the benchmark's extras time
    (capacity factor 1.25, RMSNorm, residual, one shared expert as wide as
    the routed ones), on sampled tokens. At this balance no expert reaches
    its capacity, which the test asserts, so every token's output depends on
    its own routing only and near-tie tokens may take any valid routing."""
    import test_gpu_ext as X
    w = wl.WORKLOADS[name]
    say(f"full-size block options {name}: generating inputs")
    inp = wl.make_layer_inputs(w, seed=0)
    ext = wl.make_block_extras(w.d, 1, w.ffn, w.dtype, seed=0)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    shared = (dev_tensor(ext["s_gate"]), dev_tensor(ext["s_up"]), dev_tensor(ext["s_down"]))
    say(f"full-size block options {name}: moe_forward_ext")
    out, ex = M.moe_forward_ext(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                                w.k, router_bias=dv["router_bias"], capacity_factor=1.25,
                                norm_weight=dev_tensor(ext["norm_weight"]), residual=True,
                                shared=shared, want_counts=True, want_routed_counts=True)
    torch.cuda.synchronize()
    got = host(out)
    kept, routed = host(ex["counts"]), host(ex["routed_counts"])
    cap = O.capacity(w.T, w.E, w.k, 1.25)
    assert routed.max() <= cap and np.array_equal(kept, routed), "an expert reached its capacity"
    rng = np.random.default_rng(99)
    tok = np.sort(rng.choice(w.T, size=min(48, w.T), replace=False))
    say(f"full-size block options {name}: oracle on {len(tok)} tokens")
    sub = dict(inp, x=inp["x"][tok])
    ref, _ = O.moe_forward(sub["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                           w.k, inp["router_bias"], norm_weight=ext["norm_weight"],
                           residual=True, shared=(ext["s_gate"], ext["s_up"], ext["s_down"]))
    worst, amb = X._compare(got[tok], ref, None, sub, ext, w.k, 0.0, True, True, 1, True)
    say(f"full-size block options {name}: worst {worst:.3e} x RMS, near-ties {amb}")


@pytest.mark.timeout(900)
def test_largest_batch_byte_offsets(M):
    """The largest batch the ABI accepts at the prefill widths: T*k*ffn*2 bytes
    of h just under 2^32 (T = 74898, 4.29e9 bytes), so the down pass's 32-bit
    byte offsets into h reach the top of their range. The sample holds the
    last tokens of the last expert by the oracle's own routing (the highest
    permuted rows, hence the highest offsets) and a few random ones."""
    T, d, ffn, E, k = 74898, 4096, 14336, 8, 2
    assert T * k * ffn * 2 < 2 ** 32 <= (T + 1) * k * ffn * 2
    say(f"largest batch T={T}: generating inputs")
    inp = wl.make_custom_inputs(T, d, ffn, E, "bf16", seed=0)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    say("largest batch: moe_forward")
    out = M.moe_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], k)
    torch.cuda.synchronize()
    got = host(out)
    del dv, out
    torch.cuda.empty_cache()
    say("largest batch: oracle routing of every token")
    L = O.router_logits(inp["x"], inp["w_router"], None)
    _, idx, _ = O.route(L, k)
    last = np.flatnonzero((idx == E - 1).any(axis=1))[-8:]
    rng = np.random.default_rng(7)
    tok = np.unique(np.concatenate([last, rng.choice(T, size=8, replace=False)]))
    say(f"largest batch: oracle on {len(tok)} tokens")
    st = compare_layer(got[tok], inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                       inp["w_down"], k, None, 2e-2, tokens=tok)
    say(f"largest batch: max err {st['max_rel_err']:.3e} x RMS, near-ties {st['near_ties']}")
