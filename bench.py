#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward pass on one MI355X.

One step = one ``moe_forward`` call (noisy top-k gating, routing, expert FFNs,
weighted sum, Importance/Load and both losses, training mode) over a batch of
65536 tokens, d_model 512, 4096 experts 512-1024-512, k = 4, bf16 storage with
fp32 accumulation and fp32 gate math. Inputs are synthetic (seeded Philox
normals, weights ~ N(0, 1/fan_in)) and resident in HBM before timing starts.

Prints one JSON line: tokens/s from the median of the timed steps (HIP events
around each step on the stream the library launches on); the expert-FFN
kernel against its own roof (HBM bandwidth where streaming the experts'
weights bounds it, the MFMA peak of its dtype where its arithmetic does; its
duration from timing events the library records around that kernel inside
the timed steps); every stage, each entry point called on its own, against
its own roof (gate and Load passes: MFMA; expert FFN: the larger of its two
ideal times; combine: HBM; route: latency, in microseconds); and the oracle's
CPU throughput on a bounded sample of the same workload (all host threads),
plus on one thread for the two fp32 workloads.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer forward tokens/sec at 4096 experts k=4; % MFMA peak and % HBM BW"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_device(a, torch, np):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def time_steps(step, steps, torch):
    """Times `steps` calls of step() with a pair of HIP events around each one
    on the current stream (the stream the library launches on), the events of
    consecutive steps back to back. Returns (per-step ms list, total ms from
    the first event to the last)."""
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for i in range(steps):
        step()
        ev[i + 1].record(st)
    ev[-1].synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[-1])


def median(v):
    v = sorted(v)
    m = len(v) // 2
    return v[m] if len(v) % 2 else 0.5 * (v[m - 1] + v[m])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def roof(name, ms, flops=0.0, nbytes=0.0, flops_peak=None, bound=None):
    """A stage's time against its own roof: achieved TFLOP/s over the MFMA
    peak of its dtype and achieved GB/s over the HBM peak; `bound` names the
    roof that limits it (by default the larger of the two ideal times)."""
    r = {"ms": ms}
    t_mfma = flops / (flops_peak * 1e12) * 1e3 if flops and flops_peak else 0.0
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3 if nbytes else 0.0
    if flops:
        r.update(alg_flops=flops, tflops=flops / (ms * 1e-3) / 1e12, mfma_peak_tflops=flops_peak,
                 mfma_frac=flops / (ms * 1e-3) / (flops_peak * 1e12))
    if nbytes:
        r.update(alg_bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                 hbm_frac=nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9))
    r["bound"] = bound or ("latency" if not (flops or nbytes) else
                           "mfma" if t_mfma >= t_hbm else "hbm")
    r["roof_ms"] = max(t_mfma, t_hbm)
    r["frac"] = r["roof_ms"] / ms if r["roof_ms"] else None
    return r


def time_calls(fn, iters, torch):
    """Average device time of fn() over iters calls, bracketed by HIP events on
    the current stream (the stream the library launches on)."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


# HBM bytes per ffn_kernel launch from the calibrated FETCH_SIZE + WRITE_SIZE
# counters of the committed rocprofv3 summary of that workload; valid only
# while the kernel's sources are byte-identical to those the counters were
# taken on.
FFN_SOURCES = ["sparsely_gated_mixture_moe_amd/csrc/ffn.hip",
               "sparsely_gated_mixture_moe_amd/csrc/device_common.h"]


def profiled_traffic(workload):
    import hashlib

    TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", f"ffn_kernel_{workload}_hbm_traffic.txt")
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        key, sep, val = line.partition(":")
        if sep and key in ("traffic_bytes_per_launch", "sources_sha256"):
            fields[key] = val.strip()
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("sources_sha256") != h.hexdigest():
        log("ffn sources changed since the traffic counters were taken: traffic = null")
        return None
    return int(fields["traffic_bytes_per_launch"])


def library_gemms(torch, iters=20):
    """The vendor GEMM (torch.matmul -> hipBLASLt) on dense versions of the
    layer's products: the gate's x [B, d] times [W_g | W_noise] at the
    4096-expert workload, and the two expert products over all routed rows of
    the Zipf 256-expert workload (131072 rows) and of its most popular expert
    (21504 rows). Reference points only: the fused kernels also add the noise,
    the top-k and the routing, and write no [B, 2n] logits."""
    shapes = [
        ("gate product 65536 x 8192 x 512 (bf16 out)", 65536, 8192, 512, torch.bfloat16),
        ("Zipf expert-0 first product 21504 x 1024 x 512", 21504, 1024, 512, torch.bfloat16),
        ("Zipf expert-0 second product 21504 x 512 x 1024", 21504, 512, 1024, torch.bfloat16),
        ("all routed rows, first product 131072 x 1024 x 512", 131072, 1024, 512, torch.bfloat16),
        ("all routed rows, second product 131072 x 512 x 1024", 131072, 512, 1024, torch.bfloat16),
        ("square 8192 x 8192 x 8192", 8192, 8192, 8192, torch.bfloat16),
        ("fp32 32768 x 1024 x 512", 32768, 1024, 512, torch.float32),
    ]
    for name, m, n, kk, dt in shapes:
        a = torch.randn(m, kk, device="cuda", dtype=dt)
        b = torch.randn(n, kk, device="cuda", dtype=dt).t()
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        peak = BF16_PEAK_TFLOPS if dt == torch.bfloat16 else FP32_PEAK_TFLOPS
        tf = 2.0 * m * n * kk / ms / 1e9
        print(json.dumps({"gemm": name, "dtype": str(dt).replace("torch.", ""), "ms": ms,
                          "tflops": tf, "frac": tf / peak}), flush=True)
        del a, b, c


def cpu_baseline(w, inp, target_s):
    """The oracle's whole forward pass on the first S tokens of the workload,
    S grown until one run takes about target_s seconds."""
    import numpy as np

    import datagen as dg
    import oracle

    def run(S):
        sub = dict(inp)
        sub["x"] = inp["x"][:S]
        sub["eps"] = inp["eps"][:S]
        t0 = time.perf_counter()
        oracle.forward(sub, w.k)
        return time.perf_counter() - t0

    S = 256
    t = run(S)
    # grow the sample until one run takes at least 80 % of the target (fixed
    # costs make the small-sample estimates low)
    while t < 0.8 * target_s and S < w.tokens:
        S = int(min(w.tokens, max(2 * S, S * 1.05 * target_s / max(t, 1e-3))))
        t = run(S)
    threads = oracle.threads()
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"oracle forward pass (fp64, {threads} OpenMP threads) on the first {S} "
                      f"tokens of the same workload: gating over all {w.n_experts} experts, "
                      f"expert FFNs, weighted sum, Importance/Load and losses; {t:.1f} s"}


def cpu_single_thread(target_s):
    """The oracle's forward pass on one host thread for the two fp32
    workloads (256 tokens over 16 experts; 8192 tokens over 32 experts),
    median of three runs on the whole batch or on its first S tokens, S grown
    until one run takes about target_s seconds."""
    import datagen as dg
    import oracle

    all_threads = oracle.threads()
    oracle.set_threads(1)
    res = {}
    try:
        for name in ("tiny_fp32", "flat_fp32_n32"):
            w = dg.WORKLOADS[name]
            inp = dg.make_inputs(w)

            def run(S):
                sub = dict(inp, x=inp["x"][:S], eps=inp["eps"][:S])
                t0 = time.perf_counter()
                oracle.forward(sub, w.k)
                return time.perf_counter() - t0

            S = min(w.tokens, 64)
            t = run(S)
            while t < 0.8 * target_s and S < w.tokens:
                S = int(min(w.tokens, max(2 * S, S * 1.05 * target_s / max(t, 1e-3))))
                t = run(S)
            ts = sorted([t, run(S), run(S)])
            res[name] = {"value": S / ts[1], "unit": "tokens/s", "cores": 1, "tokens": S,
                         "median_of": 3, "seconds": ts[1]}
    finally:
        oracle.set_threads(all_threads)
    return res


def upload(w, name, shape, torch, dg, chunk=1 << 27):
    """Tensor `name` of workload `w` generated in chunks straight into device memory."""
    import numpy as np

    probe = dg.gen(w, name, 0, 1)
    bf16 = probe.dtype == np.uint16
    total = int(np.prod(shape))
    t = torch.empty(total, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    for i, off in enumerate(range(0, total, chunk)):
        cnt = min(chunk, total - off)
        if i % 16 == 15:
            log(f"  {name}: {off / total:.0%}")
        a = dg.gen(w, name, off, cnt)
        src = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        t[off:off + cnt].copy_(src)
    return t.view(*shape)


def bench_hier(a, w):
    """The hierarchical layer ("Hierarchical MoE"): one step = one moe_hier_forward
    call (both gate levels, leaf routing, expert FFNs, weighted sum, both levels'
    Load and the losses, training mode)."""
    import numpy as np
    import torch

    import datagen as dg
    import sparsely_gated_mixture_moe_amd as moe

    B, d, h = w.tokens, w.d_model, w.d_hidden
    ga, gb, k1, k2 = w.groups, w.group_experts, w.k1, w.k2
    n, K = ga * gb, k1 * k2
    log(f"generating {w.name} on the device: {w.description}")
    t0 = time.time()
    g = {"x": upload(w, "x", (B, d), torch, dg), "w_gate": upload(w, "w_gate", (ga, d), torch, dg),
         "w_noise": upload(w, "w_noise", (ga, d), torch, dg),
         "eps": upload(w, "eps", (B, ga), torch, dg),
         "w_gate2": upload(w, "w_gate2", (ga, gb, d), torch, dg),
         "w_noise2": upload(w, "w_noise2", (ga, gb, d), torch, dg),
         "eps2": upload(w, "eps2", (B, k1, gb), torch, dg),
         "w1": upload(w, "w1", (n, h, d), torch, dg), "w2": upload(w, "w2", (n, d, h), torch, dg)}
    torch.cuda.synchronize()
    log(f"inputs resident after {time.time() - t0:.1f} s")
    layout = 1 if a.expert_layout == "packed" else 0
    if layout:  # a one-time conversion of the leaf weights, outside the timed steps
        g["w1"], g["w2"] = moe.moe_pack_expert_weights(g["w1"], g["w2"])
        torch.cuda.synchronize()
    f = moe.MoeHierForward((B, d), g["w_gate"], g["w_noise"], g["w_gate2"], g["w_noise2"],
                           g["w1"], g["w2"], k1, k2, train=True, expert_layout=layout)
    dev = g["x"].device
    y = torch.empty((B, d), dtype=g["x"].dtype, device=dev)
    leaf_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    leaf_gate = torch.empty((B, K), dtype=torch.float32, device=dev)

    def step():
        f(g["x"], g["eps"], g["eps2"], y, topk_idx=leaf_idx, topk_gate=leaf_gate)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    per_step, total_ms = time_steps(step, a.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = median(per_step)
    log(f"{ms_step:.3f} ms/step median, {total_ms / a.steps:.3f} mean")
    # the leaf FFN on its own, on the step's routing
    dims = moe.make_dims(B, d, h, n, K, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16)
    ws = moe.workspace(dims, moe.make_opts(), dev)
    route = moe.moe_route(leaf_idx, leaf_gate, n, d_model=d, ws=ws)
    eo = torch.empty((B * K, d), dtype=g["x"].dtype, device=dev)
    it = a.stage_iters
    stages = {
        "route_leaves": time_calls(lambda: moe.moe_route(leaf_idx, leaf_gate, n, d_model=d, ws=ws),
                                   it, torch),
        "expert_ffn": time_calls(lambda: moe.moe_expert_ffn(
            g["x"], route["offsets"], route["perm_token"], g["w1"], g["w2"], K, ws=ws, out=eo,
            expert_layout=layout),
            it, torch),
    }
    log("stages (ms): " + ", ".join(f"{k_}={v:.3f}" for k_, v in stages.items()))
    cnt = route["counts"].cpu().numpy()
    used, rows = int((cnt > 0).sum()), int(cnt.sum())
    ffn_bytes = used * 2 * d * h * 2 + 2 * rows * d * 2
    ffn_ms = ffn_total / ffn_n  # the FFN kernel inside the timed steps
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    gate_flops = 2.0 * B * d * 2 * ga + 2.0 * B * k1 * d * 2 * gb
    step_flops = gate_flops + 4.0 * rows * d * h  # both gate levels once + FFN
    step_bytes = (B * d * 2 + B * ga * 4 + B * k1 * gb * 4 + 2 * ga * d * 2 + 2 * n * d * 2
                  + used * 2 * d * h * 2 + B * d * 2)
    result = {
        "metric": "hierarchical MoE-layer forward tokens/sec (128 x 128 = 16384 leaves, k1 = k2 = 2)",
        "value": B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "d_model": d, "d_hidden": h, "groups": ga,
                   "group_experts": gb, "k1": k1, "k2": k2, "train": 1,
                   "expert_layout": a.expert_layout},
        "roofline": {"kernel": "ffn_kernel (expert FFN over the leaves)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": ffn_bytes, "avg_launch_ms": ffn_ms,
                     "timed_launches": ffn_n,
                     "mfma_frac": 4.0 * rows * d * h / (ffn_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)},
        "step": {"alg_bytes": step_bytes, "alg_flops": step_flops,
                 "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": step_flops / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                 "mean_ms": total_ms / a.steps},
        "stages_ms": stages, "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def bench_batchwise(a, w, g, moe, torch, layout=0):
    """Batchwise gating (section "What the paper measured"): one step = one
    moe_batchwise_forward call (expert-major scores, each expert's top m =
    k B / n rows, token lists, expert FFNs, softmax and weighted sum,
    Importance and the losses)."""
    B, d, h, n, k = w.tokens, w.d_model, w.d_hidden, w.n_experts, w.k
    m = max(1, k * B // n)
    f = moe.MoeBatchwiseForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], m,
                                gate_bias=g.get("gate_bias"), train=bool(a.train),
                                expert_layout=layout)
    y = torch.empty((B, d), dtype=g["x"].dtype, device=g["x"].device)

    def step():
        f(g["x"], g["eps"], y)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    per_step, total_ms = time_steps(step, a.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = median(per_step)
    log(f"{ms_step:.3f} ms/step median, {total_ms / a.steps:.3f} mean")
    cnt = f.counts.cpu().numpy()
    used, rows = int((cnt > 0).sum()), int(cnt.sum())
    ffn_bytes = used * 2 * d * h * 2 + 2 * rows * d * 2
    ffn_ms = ffn_total / ffn_n
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    gate_flops = 2.0 * B * d * n * (2 if a.train else 1)
    step_flops = gate_flops + 4.0 * rows * d * h
    # x, eps, gate weights, the fp32 score matrix written and read back, the
    # expert weights, the rows in and out, y
    step_bytes = (B * d * 2 + (B * n * 4 if a.train else 0) + 2 * n * d * 2 + 2 * B * n * 4
                  + used * 2 * d * h * 2 + 2 * rows * d * 2 + B * d * 2)
    result = {
        "metric": "batchwise-gated MoE-layer forward tokens/sec (4096 experts, m = k B / n rows each)",
        "value": B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.act_dtype == 1 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "d_model": d, "d_hidden": h, "n_experts": n,
                   "k": k, "gating": "batchwise", "rows_per_expert": m, "train": a.train,
                   "expert_layout": a.expert_layout},
        "roofline": {"kernel": "ffn_kernel (expert FFN)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": ffn_bytes, "avg_launch_ms": ffn_ms,
                     "timed_launches": ffn_n},
        "step": {"alg_bytes": step_bytes, "alg_flops": step_flops,
                 "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": step_flops / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                 "mean_ms": total_ms / a.steps},
        "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def bench_backward(a, w, g, moe, torch, np, dg):
    """The backward pass (moe_backward): one step = one call computing the
    gradients of sum dy . y + the weighted losses for x, the gate weights and
    bias and every expert's weights and biases, from one forward pass's
    selection, thresholds, Importance and Load (recomputing the experts'
    hidden activations)."""
    B, d, h, n, k = w.tokens, w.d_model, w.d_hidden, w.n_experts, w.k
    fwd = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], k,
                          gate_bias=g.get("gate_bias"), train=True, return_routing=True)
    dy = torch.empty_like(g["x"]).normal_()
    dims = moe.make_dims(B, d, h, n, k, moe._binding._dt(g["x"]), moe._binding._dt(g["w1"]),
                         moe._binding._dt(g["w_gate"]))
    nbytes = int(moe.lib().moe_backward_workspace_size(ctypes_byref(dims),
                                                        ctypes_byref(moe.make_opts())))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=g["x"].device)

    def step():
        moe.moe_backward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], k,
                         fwd["topk_idx"], fwd["topk_gate"], fwd["thresh"], fwd["importance"],
                         fwd["load"], dy, gate_bias=g.get("gate_bias"), ws=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    per_step, total_ms = time_steps(step, a.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = median(per_step)
    log(f"backward {ms_step:.3f} ms/step median")
    cnt = fwd["counts"].cpu().numpy()
    rows = int(cnt.sum())
    used = int((cnt > 0).sum())
    esize = 2 if w.expert_dtype == dg.BF16 else 4
    # expert products: hidden recompute, dA, dW2, dW1, dx rows (2 d h flops per routed row
    # each; dy . E needs no recompute of E); gate: c and u, dW_g and dW_noise, dx (2 d n flops
    # per token each, twice)
    flops = 5 * 2.0 * rows * d * h + 3 * 2 * 2.0 * B * d * n
    # expert weights read, their fp32 gradients written; the dense [B, 2n] fp32 logit
    # gradients written and read twice; x, dy, dx
    nbytes_alg = (used * 2 * d * h * (esize + 4) + 3 * B * 2 * n * 4
                  + 2 * B * d * esize + B * d * 4)
    t = ms_step * 1e-3
    # bf16 storage: the products run on the bf16 matrix cores (fp32 operands split into
    # two bf16 parts); fp32 storage: on the fp32 matrix cores
    peak = BF16_PEAK_TFLOPS if esize == 2 else FP32_PEAK_TFLOPS
    mfma_frac = flops / t / 1e12 / peak
    hbm_frac = nbytes_alg / t / (HBM_PEAK_GBS * 1e9)
    # the roof the call is nearer to bounds it: HBM for the 4096-expert workload (the
    # fp32 weight gradients alone are 17 GB), the matrix cores for the few-expert ones
    if hbm_frac > mfma_frac:
        roof = {"bound": "hbm", "achieved": nbytes_alg / t / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": hbm_frac, "mfma_frac": mfma_frac}
    else:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": peak, "unit": "TFLOP/s",
                "frac": mfma_frac, "hbm_frac": hbm_frac}
    result = {
        "metric": "MoE-layer backward tokens/sec (4096 experts, k = 4)",
        "value": B / t, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if esize == 2 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "d_model": d, "d_hidden": h, "n_experts": n,
                   "k": k, "pass": "backward", "storage": "bf16" if esize == 2 else "f32"},
        "roofline": dict({"kernel": "moe_backward (all kernels of one call)"}, **roof,
                         traffic=None, alg_flops_per_launch=flops,
                         alg_bytes_per_launch=nbytes_alg),
        "step": {"mean_ms": total_ms / a.steps, "min_ms": min(per_step), "max_ms": max(per_step)},
        "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def ctypes_byref(o):
    import ctypes
    return ctypes.byref(o)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flat_bf16_n4096")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the oracle CPU-baseline run (0 skips it)")
    ap.add_argument("--stage-iters", type=int, default=10,
                    help="calls of each entry point on its own for the stage times (0 skips them)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="batch size instead of the workload's (same model), e.g. 1 for the "
                         "latency of a single token")
    ap.add_argument("--capacity-factor", type=float, default=0.0, metavar="F",
                    help="fixed expert capacity ceil(F * tokens * k / n) rows (GShard variant; "
                         "0: no limit, the pages' layer)")
    ap.add_argument("--gate-order", type=int, default=0, choices=(0, 1),
                    help="0: softmax over the kept k (the pages); 1: softmax over all n, then "
                         "the kept k (Switch's order)")
    ap.add_argument("--expert-layout", default="packed", choices=("natural", "packed"),
                    help="packed (default): the expert weights are converted once, before timing, to "
                         "the matrix-core operand layout (moe_pack_expert_weights, "
                         "expert_layout=1); the hierarchical, batchwise and backward lines read "
                         "the natural layout")
    ap.add_argument("--gating", default="topk", choices=("topk", "batchwise"),
                    help="batchwise: every expert takes its k B / n best rows of the batch "
                         "(moe_batchwise_forward) instead of every token its k best experts")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (moe_backward) instead of the forward")
    ap.add_argument("--train", type=int, default=1, choices=(0, 1),
                    help="1: noisy gating with the Load pass (the headline step); 0: inference")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes three times "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="only time the vendor GEMM (torch.matmul, hipBLASLt) on the layer's "
                         "product shapes, as a reference point for the fused kernels")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if a.copy_calibration:
        nbytes = a.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)
        return

    if a.library_gemms:
        library_gemms(torch)
        return

    import datagen as dg
    import sparsely_gated_mixture_moe_amd as moe

    w = dg.WORKLOADS[a.workload]
    if a.tokens > 0:
        w = dg.workload(a.workload, tokens=a.tokens)
    if a.backward:
        a.expert_layout = "natural"  # the packed layout is read by the forward passes only
    if w.hierarchical:
        bench_hier(a, w)
        return
    B, d, h, n, k = w.tokens, w.d_model, w.d_hidden, w.n_experts, w.k
    log(f"generating {w.name}: {w.description}")
    t0 = time.time()
    inp = dg.make_inputs(w)
    log(f"inputs generated in {time.time() - t0:.1f} s; uploading")
    g = {key: to_device(v, torch, np) for key, v in inp.items()}
    torch.cuda.synchronize()

    layout = 1 if a.expert_layout == "packed" else 0
    if layout:  # a one-time conversion of the weights, outside the timed steps
        g["w1"], g["w2"] = moe.moe_pack_expert_weights(g["w1"], g["w2"])
        torch.cuda.synchronize()
    if a.gating == "batchwise":
        bench_batchwise(a, w, g, moe, torch, layout)
        return
    if a.backward:
        bench_backward(a, w, g, moe, torch, np, dg)
        return
    cap = int(np.ceil(a.capacity_factor * B * k / n)) if a.capacity_factor > 0 else 0
    f = moe.MoeForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], k,
                       gate_bias=g.get("gate_bias"), train=bool(a.train), capacity=cap,
                       gate_order=a.gate_order, expert_layout=layout)
    dev = g["x"].device
    y = torch.empty((B, d), dtype=g["x"].dtype, device=dev)
    topk_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    topk_gate = torch.empty((B, k), dtype=torch.float32, device=dev)
    thresh = torch.empty((B, 2), dtype=torch.float32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)

    def step():
        f(g["x"], g["eps"], y, topk_idx=topk_idx, topk_gate=topk_gate, thresh=thresh,
          counts=counts)

    log(f"warmup {a.warmup} steps")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {a.steps} steps")
    torch.cuda.synchronize()
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    per_step, total_ms = time_steps(step, a.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = median(per_step)
    log(f"{ms_step:.3f} ms/step median, {total_ms / a.steps:.3f} mean "
        f"(wall {1000 * wall / a.steps:.3f} ms/step)")

    # Stage times: each entry point on its own, on the routing of the step above.
    it = a.stage_iters
    route = moe.moe_route(topk_idx, topk_gate, n, d_model=d)
    ws = moe.workspace(f.dims, f.opts, dev)
    eo = torch.empty((B * k, d), dtype=g["x"].dtype, device=dev)
    stage_ms = {} if it <= 0 else {
        "gate": time_calls(lambda: moe.moe_gate(g["x"], g["w_gate"], g["w_noise"],
                                                g["eps"] if a.train else None, k,
                                                train=bool(a.train), gate_bias=g.get("gate_bias"),
                                                ws=ws, gate_order=a.gate_order), it, torch),
        "route": time_calls(lambda: moe.moe_route(topk_idx, topk_gate, n, d_model=d, ws=ws,
                                                  capacity=cap), it, torch),
        "expert_ffn": time_calls(lambda: moe.moe_expert_ffn(
            g["x"], route["offsets"], route["perm_token"], g["w1"], g["w2"], k, ws=ws, out=eo,
            capacity=cap, expert_layout=layout), it, torch),
        "combine": time_calls(lambda: moe.moe_combine(eo, route["slot_pos"], topk_gate,
                                                      n_experts=n, out=y), it, torch),
    }
    if it > 0 and a.train:
        stage_ms["aux_losses"] = time_calls(lambda: moe.moe_aux_losses(
            g["x"], g["w_gate"], g["w_noise"], thresh, route["offsets"], route["perm_token"],
            route["importance"], k, gate_bias=g.get("gate_bias"), ws=ws), it, torch)
    torch.cuda.synchronize()
    log("stages (ms): " + ", ".join(f"{k_}={v:.3f}" for k_, v in stage_ms.items()))

    # Algorithmic work (the selected experts only; the gate GEMM once for the
    # step, and once more for the Load pass as a stage of its own).
    cnt = counts.cpu().numpy()
    esize = 2 if w.expert_dtype == dg.BF16 else 4
    asize = 2 if w.act_dtype == dg.BF16 else 4
    gsize = 2 if w.gate_dtype == dg.BF16 else 4
    if cap:  # the rows the experts serve
        cnt = np.minimum(cnt, cap)
    used = int((cnt > 0).sum())
    rows = int(cnt.sum())
    expert_peak = BF16_PEAK_TFLOPS if w.expert_dtype == dg.BF16 else FP32_PEAK_TFLOPS
    gate_peak = BF16_PEAK_TFLOPS if w.gate_dtype == dg.BF16 else FP32_PEAK_TFLOPS
    gate_mats = 2 if a.train else 1  # W_g and W_noise, or W_g alone without noise
    gate_flops = 2.0 * B * d * n * gate_mats
    gate_bytes = B * d * asize + (B * n * 4 if a.train else 0) + gate_mats * n * d * gsize \
        + B * k * 8 + B * 8
    ffn_bytes = used * 2 * d * h * esize + 2 * rows * d * asize
    ffn_flops = 4.0 * rows * d * h
    comb_bytes = B * k * d * asize + B * d * asize + B * k * 8
    load_flops = 2.0 * B * d * n * 2
    load_bytes = B * d * asize + 2 * n * d * gsize + B * 8
    ffn_ms = ffn_total / ffn_n  # the FFN kernel inside the timed steps
    stages = {}
    if stage_ms:
        stages = {
            "gate": roof("gate", stage_ms["gate"], gate_flops, gate_bytes, gate_peak, "mfma"),
            "route": roof("route", stage_ms["route"]),
            "expert_ffn": roof("expert_ffn", stage_ms["expert_ffn"], ffn_flops, ffn_bytes,
                               expert_peak),
            "combine": roof("combine", stage_ms["combine"], 0.0, comb_bytes, None, "hbm"),
        }
        stages["route"]["us"] = stage_ms["route"] * 1e3
        if "aux_losses" in stage_ms:
            stages["aux_losses"] = roof("aux_losses", stage_ms["aux_losses"], load_flops,
                                        load_bytes, gate_peak, "mfma")
    ffn_roof = roof("ffn", ffn_ms, ffn_flops, ffn_bytes, expert_peak)
    if ffn_roof["bound"] == "mfma":
        rl = {"kernel": "ffn_kernel (expert FFN)", "bound": "mfma",
              "achieved": ffn_roof["tflops"], "peak": expert_peak, "unit": "TFLOP/s",
              "frac": ffn_roof["mfma_frac"], "hbm_frac": ffn_roof["hbm_frac"]}
    else:
        rl = {"kernel": "ffn_kernel (expert FFN)", "bound": "hbm",
              "achieved": ffn_roof["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": ffn_roof["hbm_frac"], "mfma_frac": ffn_roof["mfma_frac"]}
    rl.update(traffic=profiled_traffic(w.name), alg_bytes_per_launch=ffn_bytes,
              alg_flops_per_launch=ffn_flops, avg_launch_ms=ffn_ms, timed_launches=ffn_n)
    # x, eps, the gate matrices, the used experts' weights, y; gate GEMM once + FFN
    step_bytes = B * d * asize + (B * n * 4 if a.train else 0) + gate_mats * n * d * gsize \
        + used * 2 * d * h * esize + B * d * asize
    step_flops = gate_flops + ffn_flops
    step_gate_ms = gate_flops / (gate_peak * 1e12) * 1e3
    step_ffn_ms = ffn_flops / (expert_peak * 1e12) * 1e3
    alg_roof_ms = max(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, step_gate_ms + step_ffn_ms)
    step = {"alg_bytes": step_bytes, "alg_flops": step_flops,
            "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "mfma_frac": (step_gate_ms + step_ffn_ms) / ms_step,
            "alg_roofline_ms": alg_roof_ms, "alg_roofline_frac": alg_roof_ms / ms_step,
            "mean_ms": total_ms / a.steps, "min_ms": min(per_step), "max_ms": max(per_step)}
    if stages:
        serial = sum(v["roof_ms"] for v in stages.values())
        step.update(stage_roofs_ms=serial, stage_roofs_frac=serial / ms_step)

    result = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act_dtype == dg.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "d_model": d, "d_hidden": h, "n_experts": n,
                   "k": k, "train": a.train, "capacity": cap, "gate_order": a.gate_order,
                   "expert_layout": a.expert_layout,
                   "act_dtype": "bf16" if w.act_dtype == dg.BF16 else "f32",
                   "expert_dtype": "bf16" if w.expert_dtype == dg.BF16 else "f32",
                   "gate_dtype": "bf16" if w.gate_dtype == dg.BF16 else "f32"},
        "roofline": rl,
        "step": step,
        "stages": stages,
        # rows per expert of the timed steps' routing (the load balance the FFN sees)
        "routing": {"rows": rows, "used_experts": used,
                    "rows_per_expert_mean": float(cnt.mean()),
                    "rows_per_expert_max": int(cnt.max()),
                    "rows_per_expert_min": int(cnt.min())},
        "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    if a.cpu_seconds > 0:
        log("timing the oracle on the host cores")
        cb = cpu_baseline(w, inp, a.cpu_seconds)
        log("timing the oracle on one host thread (256-token and 8192-token fp32 workloads)")
        cb["single_thread"] = cpu_single_thread(min(4.0, a.cpu_seconds / 3))
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
