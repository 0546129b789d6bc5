"""Helpers of the GPU parity tests: moving seeded inputs to the device and
comparing HIP results with the oracle.

Routing near-ties. The HIP router computes fp32 logits; the oracle computes
them in fp64. Where a token's k-th and (k+1)-th largest logits are closer
than the logit tolerance, either expert is a correct choice. Such tokens
are found from the oracle's own logits; the HIP result must then be one of
the oracle's valid alternatives (all of them are computed by the oracle),
and every other token must match the oracle's choice exactly.
"""
from __future__ import annotations

import itertools
import os
import sys

import numpy as np
import torch

from oracle import moe_oracle as O


def say(msg: str):
    """Progress line that bypasses pytest's capture (names the case before a GPU step)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def dev_tensor(a, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def logit_tolerance(x, w_router):
    """Per-(token, expert) bound on |fp32 logit - exact logit|: 1e-5 times the
    sum of |x_i W_r[e,i]| (fp32 accumulation of exact bf16 products), plus
    an absolute floor for all-zero rows."""
    return 1e-5 * (np.abs(O.widen(x)) @ np.abs(O.widen(w_router)).T) + 1e-30


def routing_alternatives(L, k, tol):
    """For each token, the k-subsets of experts that are a correct top-k
    within the tolerance band: every expert whose logit is above the k-th
    largest by more than the band must be in, and the rest are chosen from
    those within the band of the k-th largest."""
    T, E = L.shape
    alts = []
    for t in range(T):
        srt = np.sort(L[t])[::-1]
        kth = srt[k - 1]
        band = 2.0 * tol[t].max()
        sure = [e for e in range(E) if L[t, e] > kth + band]
        cand = [e for e in range(E) if abs(L[t, e] - kth) <= band and e not in sure]
        need = k - len(sure)
        alts.append([tuple(sorted(sure + list(c))) for c in itertools.combinations(cand, need)])
    return alts


def check_slot_order(gpu_idx, L, tol):
    """Slots must be in descending logit order within the band."""
    T, k = gpu_idx.shape
    for t in range(T):
        band = 2.0 * tol[t].max()
        v = L[t, gpu_idx[t]]
        assert np.all(v[:-1] >= v[1:] - band), (t, gpu_idx[t], v)
        assert len(set(gpu_idx[t].tolist())) == k


def compare_layer(out_gpu, x, w_router, w_gate, w_up, w_down, k, bias, rel_tol, gpu_idx=None,
                  tokens=None):
    """Compare the GPU layer output (fp32, rows `tokens` of the batch, or all)
    with the oracle. Returns a dict of statistics; raises on mismatch."""
    xs = x if tokens is None else x[tokens]
    L = O.router_logits(xs, w_router, bias)
    tol = logit_tolerance(xs, w_router)
    probs, idx, w = O.route(L, k)
    E = np.asarray(w_router).shape[0]
    ref = O.expert_ffn(xs, idx, w, w_gate, w_up, w_down, E)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = rel_tol * rms
    alts = routing_alternatives(L, k, tol)
    ambiguous = [t for t, a in enumerate(alts) if len(a) > 1]
    got = np.asarray(out_gpu, np.float64)
    err = np.abs(got - ref).max(axis=1)
    bad = [t for t in range(len(xs)) if err[t] > bound and t not in ambiguous]
    assert not bad, f"{len(bad)} tokens exceed {rel_tol}*RMS; worst {err.max() / rms:.3e}*RMS"
    for t in ambiguous:
        ok = False
        for s in alts[t]:
            sel = np.array(s)[np.argsort(-L[t, list(s)], kind="stable")]
            pw = probs[t, sel] / probs[t, sel].sum()
            o = np.zeros(got.shape[1])
            for e, we in zip(sel, pw):
                o += we * O.swiglu_expert(O.widen(xs[t:t + 1]), w_gate[e], w_up[e], w_down[e])[0]
            if np.abs(got[t] - o).max() <= bound:
                ok = True
                break
        assert ok, f"near-tie token {t}: output matches none of the valid routings"
    if gpu_idx is not None:
        gi = np.asarray(gpu_idx)
        check_slot_order(gi, L, tol)
        for t in range(len(xs)):
            assert tuple(sorted(gi[t].tolist())) in alts[t], (t, gi[t], alts[t])
    unamb = [t for t in range(len(xs)) if t not in ambiguous]
    worst = float(err[unamb].max() / rms) if unamb else 0.0
    return {"rms": rms, "max_rel_err": worst, "near_ties": len(ambiguous), "ref_idx": idx}
