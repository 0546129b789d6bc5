"""Router statistics on the GPU (moe_router_stats) against the oracle's
load_balancing_loss and its per-expert terms.

Inputs come from the seeded generators and the oracle only: probabilities
are the oracle's softmax of seeded logits, stored as fp32, and the counts
its expert counts; both sides read those same fp32 values.
- frac[e] = counts[e] / T is one correctly rounded fp32 division: bit-exact.
- mean_probs and the loss are fp32 sums of up to T terms of [0, 1]: within
  a relative 1e-5 (about 80 ulp, far above the rounding of a few hundred
  fp32 additions in a fixed order).
- The end-to-end case feeds moe_forward's own probs_out and counts_out and
  compares against the oracle's statistics from its own fp64 routing; there
  the counts may differ where a near-tie token moved, which the bound
  accounts for.
"""
import numpy as np
import pytest
import torch

import moe_workloads as wl
from oracle import moe_oracle as O
from parity_util import dev_tensor, host, logit_tolerance, routing_alternatives, say

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (37, 8, 2), (1000, 8, 2), (65, 3, 3), (8192, 64, 8), (4096, 256, 4),
          (20000, 16, 1)]


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_renorm_amd as m
    m.lib()
    return m


def _inputs(T, E, k, seed, kind="normal"):
    L = wl.make_logits(T, E, kind, seed)
    p, idx, _ = O.route(L, k)
    return p.astype(np.float32), O.expert_counts(idx, E).astype(np.int32)


def _oracle_stats(p32, counts):
    T, E = p32.shape
    P = p32.astype(np.float64).sum(axis=0) / T
    return P, O.load_balancing_loss(p32, counts)


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_router_stats_parity(M, T, E, k):
    say(f"router_stats T={T} E={E} k={k}")
    p32, counts = _inputs(T, E, k, seed=T + E)
    mean, frac, loss = M.moe_router_stats(dev_tensor(p32), dev_tensor(counts))
    torch.cuda.synchronize()
    P, want_loss = _oracle_stats(p32, counts)
    assert np.array_equal(host(frac), np.float32(counts) / np.float32(T))
    np.testing.assert_allclose(host(mean), P, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(host(loss)[0], want_loss, rtol=1e-5)


def test_router_stats_closed_forms(M):
    """Uniform probabilities give a loss of k; full collapse onto one expert
    with k = 1 gives E (the same closed forms that pin the oracle)."""
    T, E, k = 3000, 8, 2
    idx, _ = wl.make_routing(T, E, k, "random", seed=5)
    counts = O.expert_counts(idx, E).astype(np.int32)
    uni = np.full((T, E), 1.0 / E, np.float32)
    _, _, loss = M.moe_router_stats(dev_tensor(uni), dev_tensor(counts))
    assert abs(host(loss)[0] - k) < 1e-5
    one = np.zeros((T, E), np.float32)
    one[:, 5] = 1.0
    c1 = np.zeros(E, np.int32)
    c1[5] = T
    mean, frac, loss = M.moe_router_stats(dev_tensor(one), dev_tensor(c1))
    assert host(loss)[0] == E and host(mean)[5] == 1.0 and host(frac)[5] == 1.0


def test_router_stats_zero_tokens(M):
    p = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    c = torch.zeros(8, dtype=torch.int32, device="cuda")
    mean, frac, loss = M.moe_router_stats(p, c)
    assert host(loss)[0] == 0.0 and not host(mean).any() and not host(frac).any()


def test_router_stats_deterministic(M):
    p32, counts = _inputs(8192, 64, 8, seed=9)
    a = M.moe_router_stats(dev_tensor(p32), dev_tensor(counts))
    b = M.moe_router_stats(dev_tensor(p32), dev_tensor(counts))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_router_stats_after_forward(M):
    """Statistics of moe_forward's own probs_out / counts_out against the
    oracle's from its own routing of the same inputs."""
    w = wl.WORKLOADS["small"]
    inp = wl.make_layer_inputs(w, seed=0)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    out, ex = M.moe_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k,
                            router_bias=dv["router_bias"], want_probs=True, want_counts=True)
    mean, frac, loss = M.moe_router_stats(ex["probs"], ex["counts"])
    torch.cuda.synchronize()
    L = O.router_logits(inp["x"], inp["w_router"], inp["router_bias"])
    p, idx, _ = O.route(L, w.k)
    counts = O.expert_counts(idx, w.E)
    near = sum(1 for a in routing_alternatives(L, w.k, logit_tolerance(inp["x"], inp["w_router"]))
               if len(a) > 1)
    P = p.sum(axis=0) / w.T
    np.testing.assert_allclose(host(mean), P, rtol=1e-4, atol=1e-6)
    dc = np.abs(host(ex["counts"]).astype(np.int64) - counts).sum()
    assert dc <= 2 * near
    want = O.load_balancing_loss(p, counts)
    # a moved assignment changes one f_e by 1/T in each of two experts
    bound = 1e-4 * want + w.E * dc / w.T * P.max()
    say(f"lb loss gpu {host(loss)[0]:.6f} oracle {want:.6f} near-ties {near}")
    assert abs(host(loss)[0] - want) <= bound
