"""The layer call captured into a HIP graph (torch.cuda.graph) gives, on
every replay, bit-identical results to the eager call, with other eager GPU
work and synchronisations between the replays. The library records no
memset or allocation on the call path, so the captured graph holds only its
kernels."""
import numpy as np
import pytest
import torch

import moe_workloads as wl
from parity_util import dev_tensor, say

pytestmark = pytest.mark.gpu

CASES = [(32, 4096, 14336, 8, 2, "bf16", False), (300, 256, 320, 8, 2, "bf16", True),
         (64, 64, 128, 4, 2, "f32", False)]


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_renorm_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("T,d,ffn,E,k,dtype,bias", CASES)
def test_graph_replays_match_eager(M, T, d, ffn, E, k, dtype, bias):
    say(f"graph T={T} d={d} ffn={ffn} E={E} k={k} {dtype}")
    inp = wl.make_custom_inputs(T, d, ffn, E, dtype, seed=7, bias=bias)
    dv = {n: dev_tensor(v) for n, v in inp.items()}
    lay = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], k)
    ws = M.workspace(T, d, ffn, E, k, dv["x"].dtype)
    eager = M.moe_forward(*lay, router_bias=dv["router_bias"], ws=ws).clone()
    out = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.moe_forward(*lay, router_bias=dv["router_bias"], ws=ws, out=out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            M.moe_forward(*lay, router_bias=dv["router_bias"], ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float(r + 1))                       # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        del junk
