"""Host-side checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

import moe_workloads as wl


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even to bfloat16 equals torch's float32->bfloat16 cast."""
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, -2.5, 3e38, 1e-40, 65504.0], np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)[:30000],  # exact ties
    ])
    f = f[np.isfinite(f)]
    ours = wl.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(f).to(torch.bfloat16).float().numpy())


def test_draws_independent_of_chunking_and_threads():
    n = wl.CHUNK * 2 + 1234
    a = wl.normal_f32(0, 5, n)
    # each chunk is its own stream, so chunk 1 alone reproduces the middle part
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=(5, 1))))
    mid = g.standard_normal(wl.CHUNK, dtype=np.float32)
    assert np.array_equal(a[wl.CHUNK:2 * wl.CHUNK], mid)
    assert np.array_equal(a, wl.normal_f32(0, 5, n))
    assert not np.array_equal(a[:1000], wl.normal_f32(1, 5, 1000))


def test_layer_inputs_shapes_and_scale():
    w = wl.WORKLOADS["tiny"]
    inp = wl.make_layer_inputs(w)
    assert inp["x"].shape == (64, 64) and inp["x"].dtype == np.float32
    assert inp["w_gate"].shape == (4, 128, 64) and inp["w_down"].shape == (4, 64, 128)
    assert abs(inp["w_up"].std() - 0.02) < 0.002 and abs(inp["x"].std() - 1) < 0.05
    assert inp["router_bias"] is None
    s = wl.make_custom_inputs(8, 32, 48, 3, "bf16")
    assert s["x"].dtype == np.uint16 and s["w_up"].shape == (3, 48, 32)


def test_zipf_bias_prior():
    b = wl.zipf_logit_bias(64)
    p = np.exp(b) / np.exp(b).sum()
    r = np.arange(1, 65, dtype=np.float64) ** -1.2
    assert np.allclose(p, r / r.sum(), rtol=1e-6)


def test_routings_have_distinct_experts():
    for kind in wl.ROUTING_KINDS:
        idx, w = wl.make_routing(50, 8, 3, kind, seed=2)
        assert idx.dtype == np.int32 and w.dtype == np.float32
        assert all(len(set(r)) == 3 for r in idx.tolist())
        assert idx.min() >= 0 and idx.max() < 8 and np.all(w > 0)


def test_logit_kinds():
    for kind in wl.LOGIT_KINDS:
        L = wl.make_logits(30, 8, kind)
        assert L.shape == (30, 8) and L.dtype == np.float32 and np.all(np.isfinite(L))
    z = wl.make_logits(30, 8, "zeros")
    assert np.all(z == 0) and np.any(np.signbit(z)) and np.any(~np.signbit(z))
