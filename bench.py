#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward pass on one MI355X.

One step = one ``moe_forward`` call (noisy top-k gating, routing, expert FFNs,
weighted sum, Importance/Load and both losses, training mode) over a batch of
65536 tokens, d_model 512, 4096 experts 512-1024-512, k = 4, bf16 storage with
fp32 accumulation and fp32 gate math. Inputs are synthetic (seeded Philox
normals, weights ~ N(0, 1/fan_in)) and resident in HBM before timing starts.

Prints one JSON line: tokens/s, the expert-FFN kernel's achieved HBM bandwidth
against the 8 TB/s peak (its duration from timing events the library records
around that kernel inside the timed steps, on the step's stream), per-stage
times of each entry point called on its own, and the oracle's CPU throughput
on a bounded sample of the same workload.

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
# counters of the committed rocprofv3 summary; valid only while the kernel's
# sources are byte-identical to those the counters were taken on.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ffn_kernel_flat_bf16_n4096_hbm_traffic.txt")
FFN_SOURCES = ["sparsely_gated_mixture_moe_amd/csrc/ffn.hip",
               "sparsely_gated_mixture_moe_amd/csrc/device_common.h"]


def profiled_traffic(workload):
    import hashlib

    if workload != "flat_bf16_n4096" or not os.path.exists(TRAFFIC_PROFILE):
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
            "sample": f"oracle forward pass (fp64, {threads} OpenMP threads) on the first {S} "
                      f"tokens of the same workload: gating over all {w.n_experts} experts, "
                      f"expert FFNs, weighted sum, Importance/Load and losses; {t:.1f} s"}


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
    f = moe.MoeHierForward((B, d), g["w_gate"], g["w_noise"], g["w_gate2"], g["w_noise2"],
                           g["w1"], g["w2"], k1, k2, train=True)
    dev = g["x"].device
    y = torch.empty((B, d), dtype=g["x"].dtype, device=dev)
    leaf_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    leaf_gate = torch.empty((B, K), dtype=torch.float32, device=dev)

    def step():
        f(g["x"], g["eps"], g["eps2"], y, topk_idx=leaf_idx, topk_gate=leaf_gate)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    e0.record(st)
    for _ in range(a.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = e0.elapsed_time(e1) / a.steps
    log(f"{ms_step:.3f} ms/step")
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
            g["x"], route["offsets"], route["perm_token"], g["w1"], g["w2"], K, ws=ws, out=eo),
            it, torch),
    }
    log("stages (ms): " + ", ".join(f"{k_}={v:.3f}" for k_, v in stages.items()))
    cnt = route["counts"].cpu().numpy()
    used, rows = int((cnt > 0).sum()), int(cnt.sum())
    ffn_bytes = used * 2 * d * h * 2 + 2 * rows * d * 2
    ffn_ms = ffn_total / ffn_n  # the FFN kernel inside the timed steps
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    gate_flops = 2.0 * B * d * 2 * ga + 2.0 * B * k1 * d * 2 * gb
    step_flops = 2 * gate_flops + 4.0 * rows * d * h  # both gates twice (selection, Load) + FFN
    step_bytes = (B * d * 2 + B * ga * 4 + B * k1 * gb * 4 + 2 * ga * d * 2 + 2 * n * d * 2
                  + used * 2 * d * h * 2 + B * d * 2)
    result = {
        "metric": "hierarchical MoE-layer forward tokens/sec (128 x 128 = 16384 leaves, k1 = k2 = 2)",
        "value": B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "d_model": d, "d_hidden": h, "groups": ga,
                   "group_experts": gb, "k1": k1, "k2": k2, "train": 1},
        "roofline": {"kernel": "ffn_kernel (expert FFN over the leaves)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": ffn_bytes, "avg_launch_ms": ffn_ms,
                     "timed_launches": ffn_n,
                     "mfma_frac": 4.0 * rows * d * h / (ffn_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)},
        "step": {"alg_bytes": step_bytes, "alg_flops": step_flops,
                 "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": step_flops / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)},
        "stages_ms": stages, "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def bench_batchwise(a, w, g, moe, torch):
    """Batchwise gating (section "What the paper measured"): one step = one
    moe_batchwise_forward call (expert-major scores, each expert's top m =
    k B / n rows, token lists, expert FFNs, softmax and weighted sum,
    Importance and the losses)."""
    B, d, h, n, k = w.tokens, w.d_model, w.d_hidden, w.n_experts, w.k
    m = max(1, k * B // n)
    f = moe.MoeBatchwiseForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], m,
                                gate_bias=g.get("gate_bias"), train=bool(a.train))
    y = torch.empty((B, d), dtype=g["x"].dtype, device=g["x"].device)

    def step():
        f(g["x"], g["eps"], y)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    e0.record(st)
    for _ in range(a.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = e0.elapsed_time(e1) / a.steps
    log(f"{ms_step:.3f} ms/step")
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
                   "k": k, "gating": "batchwise", "rows_per_expert": m, "train": a.train},
        "roofline": {"kernel": "ffn_kernel (expert FFN)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": ffn_bytes, "avg_launch_ms": ffn_ms,
                     "timed_launches": ffn_n},
        "step": {"alg_bytes": step_bytes, "alg_flops": step_flops,
                 "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": step_flops / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)},
        "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


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
    ap.add_argument("--gating", default="topk", choices=("topk", "batchwise"),
                    help="batchwise: every expert takes its k B / n best rows of the batch "
                         "(moe_batchwise_forward) instead of every token its k best experts")
    ap.add_argument("--train", type=int, default=1, choices=(0, 1),
                    help="1: noisy gating with the Load pass (the headline step); 0: inference")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes three times "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
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

    import datagen as dg
    import sparsely_gated_mixture_moe_amd as moe

    w = dg.WORKLOADS[a.workload]
    if a.tokens > 0:
        w = dg.workload(a.workload, tokens=a.tokens)
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

    if a.gating == "batchwise":
        bench_batchwise(a, w, g, moe, torch)
        return
    cap = int(np.ceil(a.capacity_factor * B * k / n)) if a.capacity_factor > 0 else 0
    f = moe.MoeForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], k,
                       gate_bias=g.get("gate_bias"), train=bool(a.train), capacity=cap,
                       gate_order=a.gate_order)
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
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    moe.moe_ffn_timing(True)
    w0 = time.perf_counter()
    e0.record(st)
    for _ in range(a.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_ffn_timing(False)
    ffn_n, ffn_total = moe.moe_ffn_timing_read()
    ms_step = e0.elapsed_time(e1) / a.steps
    log(f"{ms_step:.3f} ms/step (wall {1000 * wall / a.steps:.3f} ms/step)")

    # Stage times: each entry point on its own, on the routing of the step above.
    it = a.stage_iters
    route = moe.moe_route(topk_idx, topk_gate, n, d_model=d)
    ws = moe.workspace(f.dims, f.opts, dev)
    eo = torch.empty((B * k, d), dtype=g["x"].dtype, device=dev)
    stages = {} if it <= 0 else {
        "gate": time_calls(lambda: moe.moe_gate(g["x"], g["w_gate"], g["w_noise"],
                                                g["eps"] if a.train else None, k,
                                                train=bool(a.train), gate_bias=g.get("gate_bias"),
                                                ws=ws, gate_order=a.gate_order), it, torch),
        "route": time_calls(lambda: moe.moe_route(topk_idx, topk_gate, n, d_model=d, ws=ws,
                                                  capacity=cap), it, torch),
        "expert_ffn": time_calls(lambda: moe.moe_expert_ffn(
            g["x"], route["offsets"], route["perm_token"], g["w1"], g["w2"], k, ws=ws, out=eo,
            capacity=cap), it, torch),
        "combine": time_calls(lambda: moe.moe_combine(eo, route["slot_pos"], topk_gate,
                                                      n_experts=n, out=y), it, torch),
    }
    if it > 0 and a.train:
        stages["aux_losses"] = time_calls(lambda: moe.moe_aux_losses(
            g["x"], g["w_gate"], g["w_noise"], thresh, route["offsets"], route["perm_token"],
            route["importance"], k, gate_bias=g.get("gate_bias"), ws=ws), it, torch)
    torch.cuda.synchronize()
    log("stages (ms): " + ", ".join(f"{k_}={v:.3f}" for k_, v in stages.items()))

    # Roofline of the dominant kernel, the expert FFN: algorithmic bytes per launch =
    # the weights of every expert that received rows (2 d h elements each) + the
    # gathered input rows + the written output rows.
    cnt = counts.cpu().numpy()
    esize = 2 if w.expert_dtype == dg.BF16 else 4
    asize = 2 if w.act_dtype == dg.BF16 else 4
    if cap:  # the rows the experts serve
        cnt = np.minimum(cnt, cap)
    used = int((cnt > 0).sum())
    rows = int(cnt.sum())
    ffn_bytes = used * 2 * d * h * esize + 2 * rows * d * asize
    ffn_flops = 4.0 * rows * d * h
    ffn_ms = ffn_total / ffn_n  # the FFN kernel inside the timed steps
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    gsize = 2 if w.gate_dtype == dg.BF16 else 4
    if a.train:  # x, eps, both gate matrices, the used experts, y; gate GEMM twice + FFN
        step_bytes = (B * d * asize + B * n * 4 + 2 * n * d * gsize + used * 2 * d * h * esize
                      + B * d * asize)
        step_flops = 2.0 * B * d * 2 * n * 2 + ffn_flops
    else:  # no noise: x, W_g, the used experts, y; one clean-logit GEMM + FFN
        step_bytes = B * d * asize + n * d * gsize + used * 2 * d * h * esize + B * d * asize
        step_flops = 2.0 * B * d * n + ffn_flops
    mfma_peak = BF16_PEAK_TFLOPS if w.expert_dtype == dg.BF16 else FP32_PEAK_TFLOPS

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
                   "act_dtype": "bf16" if w.act_dtype == dg.BF16 else "f32",
                   "gate_dtype": "bf16" if w.gate_dtype == dg.BF16 else "f32"},
        "roofline": {"kernel": "ffn_kernel (expert FFN)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(w.name),
                     "alg_bytes_per_launch": ffn_bytes, "avg_launch_ms": ffn_ms,
                     "timed_launches": ffn_n,
                     "mfma_frac": ffn_flops / (ffn_ms * 1e-3) / (mfma_peak * 1e12)},
        "step": {"alg_bytes": step_bytes, "alg_flops": step_flops,
                 "hbm_frac": step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": step_flops / (ms_step * 1e-3) / (mfma_peak * 1e12)},
        "stages_ms": stages,
        "wall_ms_per_step": 1000 * wall / a.steps,
        "cpu_baseline": None,
    }
    if a.cpu_seconds > 0:
        log("timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
