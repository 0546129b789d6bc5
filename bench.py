#!/usr/bin/env python3
"""Benchmark of the top-k routed MoE layer forward on one MI355X.

One step = one moe_forward call (router, softmax/top-k/renorm, permutation,
grouped gate/up GEMM with SiLU*mul, grouped down GEMM, combine) over the
whole batch, inputs resident in HBM. Default workload: the Mixtral-shaped
prefill layer (T=4096, d=4096, ffn=14336, E=8, top-2, bf16 weights and
activations, fp32 accumulation, fp32 output).

Prints one JSON line: tokens/s for the layer, plus
  roofline     -- the gate/up GEMM (the dominant kernel): its algorithmic
                  FLOPs (4*T*k*d*ffn) per launch over its mean duration, timed
                  with HIP events recorded between the layer's kernels on its
                  stream, against the bf16 dense MFMA peak (prefill-like
                  workloads) or its algorithmic bytes against HBM (decode);
  cpu_baseline -- the CPU oracle timed on this host on a bounded token sample;
  extras       -- the calls beyond the layer itself, timed the same way on the
                  same inputs: moe_router_stats on the layer's probabilities
                  and counts (bytes read against HBM), and moe_forward_ext
                  with each block option (capacity factor 1.25; RMSNorm and
                  residual; one shared expert of the routed experts' width;
                  all together), each as a whole-layer step against the
                  layer's bound (active FLOPs, or bytes for decode); and,
                  under extras.workloads, the decode, small and skewed
                  configurations of the layer, each measured like the
                  headline (ms/step, tokens/s, stage times, the gate/up
                  kernel's roofline, the layer's fraction of the bf16 peak or,
                  for decode, of HBM bandwidth over its algorithmic bytes).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA (fp32 layers)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE layer tokens/sec + % bf16 MFMA peak (active FLOPs), d4096/ffn14336/E8/top2"
CPU_SAMPLE = {"tiny": 64, "small": 2048, "prefill": 4096, "decode": 32, "skewed": 8192}
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {  # the files whose text defines each dominant kernel
    "expert_gemm_bf16_kernel": ["expert_gemm.hip", "common.h"],
    "expert_stream_kernel": ["expert_stream.hip", "common.h"],
    "expert_gemm_f32_kernel": ["expert_gemm.hip", "common.h"],
}


def code_text(text: str) -> str:
    """Source text without comments and blank space, so that only a change
    of the code itself changes its hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha256(kernel: str, read=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        path = os.path.join("sparse_mixture_experts_renorm_amd", "csrc", f)
        if read is None:
            with open(os.path.join(ROOT, path)) as fh:
                text = fh.read()
        else:
            text = read(path)
        h.update(code_text(text).encode())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a plain copy of known size), or None when there are none for
    this workload or the kernel's source has changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    r = t.get("kernels", {}).get(workload)
    if not r or r.get("source_sha256") != source_sha256(kernel):
        return None
    c = t["calibration"]
    return (r["fetch_kib"] * 1024 * c["fetch_scale"] + r["write_kib"] * 1024 * c["write_scale"])


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clock takes a few tens of milliseconds of load to settle
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill",
                    choices=["tiny", "small", "prefill", "decode", "skewed"])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the router-statistics and block-option timings")
    ap.add_argument("--no-workloads", action="store_true",
                    help="with the prefill workload, skip the decode, small and skewed "
                         "measurements reported under extras.workloads")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timing of the layer call replayed from a captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = COPY_BYTES // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)
        return

    import moe_workloads as wl
    import sparse_mixture_experts_renorm_amd as moe

    w = wl.WORKLOADS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    log(f"workload {w}: generating seeded inputs")
    t0 = time.time()
    inp = wl.make_layer_inputs(w, seed=0)
    log(f"inputs ready in {time.time() - t0:.1f}s; copying to the GPU")

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    dv = {n: to_dev(v) for n, v in inp.items()}
    out = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
    ws = moe.workspace(w.T, w.d, w.ffn, w.E, w.k, dv["x"].dtype, dev)
    call = dict(router_bias=dv["router_bias"], out=out, ws=ws)
    lay = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k)

    m = measure_layer(moe, w, dv, args.steps, args.warmup)
    ms_per_step = m["ms_per_step"]
    roof = m["roofline"]
    roof["traffic"] = measured_traffic(w.name, roof.pop("kernel_family"))

    active = w.active_flops
    layer_s = ms_per_step / 1e3
    result = {
        "metric": METRIC,
        "value": w.T / layer_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "ffn": w.ffn, "E": w.E, "k": w.k,
                   "out_dtype": "f32", "router_bias": w.zipf_bias},
        "active_tflops": active / layer_s / 1e12,
        "mfma_peak_frac": active / layer_s / 1e12 / PEAK_BF16_TFLOPS,
        "stages_ms": m["stages_ms"],
        "step_ms_events": m["step_ms_events"],
        "expert_counts": m["expert_counts"],
        "roofline": roof,
        "cpu_baseline": None,
    }
    if "layer_hbm_frac" in m:
        result["layer_hbm_frac"] = m["layer_hbm_frac"]

    if not args.no_graph:
        # the same call captured once into a HIP graph and replayed: the
        # kernels are identical, only the launches are batched
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            moe.moe_forward(*lay, **call)          # warm the caching allocator on this stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s_cap):
                moe.moe_forward(*lay, **call)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        gms = _timed(g.replay, args.steps, args.warmup)
        result["graph"] = {"ms_per_step": gms, "tokens/s": w.T / gms * 1e3,
                           "note": "same layer call replayed from a captured HIP graph"}
        log(f"graph replay: {gms:.3f} ms/step")

    if not args.no_extras:
        result["extras"] = extras(args, w, moe, wl, dv, lay, call, to_dev, log)
    if not args.no_workloads and w.name == "prefill":
        result.setdefault("extras", {})["workloads"] = other_workloads(args, moe, wl, dv, to_dev, log)

    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        S = min(w.T, CPU_SAMPLE[w.name])
        log(f"CPU oracle on the first {S} tokens")
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        t = time.perf_counter()
        O.moe_forward(inp["x"][:S], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                      w.k, inp["router_bias"])
        dt = time.perf_counter() - t
        result["cpu_baseline"] = {
            "value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {S} of the {w.T} tokens of the same seeded workload, fp64 numpy "
                      f"oracle, all experts' weights widened, {dt:.1f}s"}
    print(json.dumps(result), flush=True)


def gate_up_kernel(w, rows):
    """Name and family of the gate/up kernel the library launches for this
    shape (its own switches: fp32 layers on the fp32 MFMA tiles; bf16 layers
    weight streaming for at most 32 rows per expert on average, 384-row tiles
    from 768, 256-row tiles between)."""
    kmask = "true" if w.d % 64 else "false"
    if w.dtype == "f32":
        return "expert_gemm_f32_kernel<true>", "expert_gemm_f32_kernel", "mfma"
    if rows <= 32 * w.E:
        nb = 1 if rows <= 16 * w.E else 2
        # bf16 batches of at most 256 assignments derive their permutation
        # inside this kernel (its last template argument)
        self_perm = "true" if w.dtype == "bf16" and rows <= 256 else "false"
        return (f"expert_stream_kernel<true, 1, {nb}, false, {self_perm}>", "expert_stream_kernel",
                "hbm")
    if rows >= 2 * 384 * w.E:
        return f"expert_gemm_tall_kernel<true, {kmask}>", "expert_gemm_bf16_kernel", "mfma"
    return f"expert_gemm_bf16_kernel<true, 8, {kmask}, false>", "expert_gemm_bf16_kernel", "mfma"


def measure_layer(moe, w, dv, steps, warmup):
    """Time moe_forward on resident inputs: `warmup` untimed calls, `steps`
    timed calls between two events, then `steps` calls of
    moe_forward_profiled whose events (recorded on the layer's stream between
    its kernels) give each stage's time. Returns the figures of one workload:
    ms per step, stage times, expert counts and the roofline of the gate/up
    kernel (algorithmic FLOPs, or bytes when it streams weights, over its
    mean event-timed duration)."""
    import numpy as np
    import torch
    dev = dv["x"].device
    out = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
    ws = moe.workspace(w.T, w.d, w.ffn, w.E, w.k, dv["x"].dtype, dev)
    call = dict(router_bias=dv["router_bias"], out=out, ws=ws)
    lay = (dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"], w.k)
    log(f"{w.name}: warmup x{warmup}")
    for _ in range(warmup):
        moe.moe_forward(*lay, **call)
    torch.cuda.synchronize()
    # ---- timed region: `steps` whole-layer steps, events around the loop ----
    log(f"{w.name}: timed x{steps}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        moe.moe_forward(*lay, **call)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps
    # ---- per-kernel times: events between the layer's kernels, same stream ----
    log(f"{w.name}: per-kernel timing x{steps}")
    evs = [moe.stage_events() for _ in range(steps)]
    for s in range(steps):
        _, ex = moe.moe_forward(*lay, **call, want_counts=True, stage_events=evs[s])
    torch.cuda.synchronize()
    names = ["router", "permute", "gate_up", "down", "combine"]
    stage_ms = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
                for i, n in enumerate(names)}
    per_step = np.array([evs[s][0].elapsed_time(evs[s][-1]) for s in range(steps)])
    cnt = ex["counts"].cpu().numpy()

    rows = w.T * w.k
    touched = int(np.count_nonzero(cnt))
    es = 2 if w.dtype == "bf16" else 4
    gu_flops = 4.0 * rows * w.d * w.ffn
    gu_bytes = touched * 2 * w.ffn * w.d * es + rows * w.d * es + rows * w.ffn * es
    gu_s = stage_ms["gate_up"] / 1e3
    kname, family, bound = gate_up_kernel(w, rows)
    if bound == "mfma":
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        roof = {"kernel": kname, "bound": "mfma", "achieved": gu_flops / gu_s / 1e12,
                "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": kname, "bound": "hbm", "achieved": gu_bytes / gu_s / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["mean_ms"] = stage_ms["gate_up"]
    roof["algorithmic_per_launch"] = gu_flops if bound == "mfma" else gu_bytes
    roof["kernel_family"] = family
    layer_s = ms_per_step / 1e3
    res = {"ms_per_step": ms_per_step, "tokens/s": w.T / layer_s,
           "active_tflops": w.active_flops / layer_s / 1e12,
           "mfma_peak_frac": w.active_flops / layer_s / 1e12 / PEAK_BF16_TFLOPS,
           "stages_ms": stage_ms,
           "stage_tflops": {"gate_up": gu_flops / gu_s / 1e12,
                            "down": 2.0 * rows * w.d * w.ffn / (stage_ms["down"] / 1e3) / 1e12},
           "step_ms_events": {"median": float(np.median(per_step)), "min": float(per_step.min()),
                              "max": float(per_step.max()),
                              "note": "per-call spread from the per-kernel timing loop"},
           "expert_counts": cnt.tolist(), "roofline": roof}
    if bound == "hbm":
        # the layer's algorithmic bytes: every touched expert's three weight
        # matrices, the router weights, x read and out written (fp32)
        layer_bytes = touched * 3.0 * w.d * w.ffn * es + w.E * w.d * es + w.T * w.d * (es + 4)
        res["layer_bytes"] = layer_bytes
        res["layer_hbm_GB/s"] = layer_bytes / layer_s / 1e9
        res["layer_hbm_frac"] = layer_bytes / layer_s / 1e9 / PEAK_HBM_GBS
    return res


def other_workloads(args, moe, wl, dv, to_dev, log):
    """The other configurations of the layer, each timed like the headline
    (warmup, then `steps` timed whole-layer calls and `steps` profiled ones):
    decode (its 32 tokens are the first rows of the prefill draw and its
    weights the prefill weights, so the resident tensors are reused), small
    and skewed (drawn here)."""
    res = {}
    dec = wl.WORKLOADS["decode"]
    ddv = dict(dv, x=dv["x"][:dec.T].contiguous())
    r = measure_layer(moe, dec, ddv, args.steps, args.warmup)
    r["roofline"].pop("kernel_family")
    res["decode"] = r
    log(f"decode: {r['ms_per_step']:.3f} ms/step, layer {r.get('layer_hbm_frac', 0):.3f} of HBM")
    for name in ("small", "skewed"):
        w = wl.WORKLOADS[name]
        log(f"{name}: generating seeded inputs")
        inp = wl.make_layer_inputs(w, seed=0)
        wdv = {n: to_dev(v) for n, v in inp.items()}
        del inp
        r = measure_layer(moe, w, wdv, args.steps, args.warmup)
        r["roofline"].pop("kernel_family")
        res[name] = r
        log(f"{name}: {r['ms_per_step']:.3f} ms/step, {r['mfma_peak_frac']:.3f} of bf16 peak")
        del wdv
    return res


def _timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def extras(args, w, moe, wl, dv, lay, call, to_dev, log):
    """Timings of the calls beyond the plain layer (see the module docstring)."""
    import numpy as np
    steps, warm = max(1, min(args.steps, 20)), max(1, args.warmup)
    out = {}
    _, ex = moe.moe_forward(*lay, **call, want_probs=True, want_counts=True)
    probs, counts = ex["probs"], ex["counts"]
    ms = _timed(lambda: moe.moe_router_stats(probs, counts), steps, warm)
    nbytes = w.T * w.E * 4 + w.E * 4
    out["router_stats"] = {"ms": ms, "bytes": nbytes, "GB/s": nbytes / ms / 1e6,
                           "hbm_frac": nbytes / ms / 1e6 / PEAK_HBM_GBS}
    log("block options: generating the norm weight and one shared expert")
    blk = wl.make_block_extras(w.d, 1, w.ffn, w.dtype, seed=0)
    g = to_dev(blk["norm_weight"])
    shared = (to_dev(blk["s_gate"]), to_dev(blk["s_up"]), to_dev(blk["s_down"]))
    es = 2 if w.dtype == "bf16" else 4
    variants = {
        "capacity_1.25": dict(capacity_factor=1.25),
        "rmsnorm_residual": dict(norm_weight=g, residual=True),
        f"shared_1x{w.ffn}": dict(shared=shared),
        "all_options": dict(capacity_factor=1.25, norm_weight=g, residual=True, shared=shared),
    }
    import torch
    ext_out = call["out"]
    for name, opt in variants.items():
        n = moe.moe_forward_ext_workspace_size(w.T, w.d, w.ffn, w.E, w.k, dv["x"].dtype, **opt)
        wsb = torch.empty(n + 256, dtype=torch.uint8, device=dv["x"].device)
        kw = dict(router_bias=dv["router_bias"], out=ext_out, ws=wsb, **opt)
        _, ex = moe.moe_forward_ext(*lay, **kw, want_counts=True)
        kept = ex["counts"].cpu().numpy().astype(np.int64)
        ms = _timed(lambda: moe.moe_forward_ext(*lay, **kw), steps, warm)
        n_sh = 1 if "shared" in opt else 0
        flops = (6.0 * kept.sum() * w.d * w.ffn + 2.0 * w.T * w.d * w.E
                 + n_sh * 6.0 * w.T * w.d * w.ffn)
        wbytes = (np.count_nonzero(kept) + n_sh) * 3.0 * w.d * w.ffn * es
        r = {"ms": ms, "tokens/s": w.T / ms * 1e3, "kept_rows": int(kept.sum()),
             "active_tflops": flops / ms / 1e9, "mfma_peak_frac": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
             "weight_GB/s": wbytes / ms / 1e6, "hbm_frac": wbytes / ms / 1e6 / PEAK_HBM_GBS}
        out[name] = r
        log(f"{name}: {ms:.3f} ms")
    return out


if __name__ == "__main__":
    main()
