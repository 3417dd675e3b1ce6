"""GPU parity of the backward pass (``moe_backward`` through the C ABI) against
the oracle's backward.

Each case runs the GPU forward pass, checks its selection against the oracle
(the same on every row that is not a near tie, a valid top k within the margin
on near-tie rows), runs the GPU backward on that forward's selection,
thresholds, Importance and Load, and compares every gradient with the oracle's
backward evaluated on the same selection (forced, as the forward tests do on
near-tie rows): dx, dW_g, dW_noise, the gate bias, dW1, db1, dW2, db2, each at
the workload's bar (1e-4 for fp32, 2e-2 for bf16 storage) with the error
metric of the forward tests. A hidden pre-activation within rounding of
ReLU's kink has two valid gradients; the oracle takes the GPU's side there
(resolve_kinks), as it takes the GPU's valid selection on a near-tie row. The reading (which parameters receive gradients, selection and
eq 9's thresholds held fixed) is the one the oracle's pins fix.
"""
import numpy as np
import pytest

import datagen as dg
import oracle
from parity import announce, check_gating, gpu_inputs, out_tol, rel_err, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsely_gated_mixture_moe_amd as moe  # noqa: E402

FLOOR = 1e-2

# (workload, overrides, train, expert and gate biases, loss weights (w_imp, w_load), aux_scale)
CASES = [
    ("tiny_fp32", {}, True, True, (0.1, 0.1), 1.0),
    ("tiny_fp32", {}, False, True, (0.1, 0.1), 1.0),
    ("tiny_fp32", {"tokens": 300, "n_experts": 37, "k": 3, "d_model": 128}, True, True,
     (0.3, 1.0), 2.0),
    ("tiny_fp32", {"tokens": 130, "n_experts": 5, "k": 5}, True, False, (0.1, 0.1), 1.0),
    ("tiny_fp32", {"tokens": 257, "n_experts": 9, "k": 1}, True, False, (0.1, 0.1), 1.0),
    ("flat_fp32_n32", {}, True, False, (0.1, 0.1), 1.0),
    ("flat_fp32_n32", {"tokens": 1000}, False, True, (0.1, 0.1), 1.0),
    ("zipf_bf16_n256", {"tokens": 2048}, True, False, (0.1, 0.1), 1.0),
    ("flat_bf16_n4096", {"tokens": 2048, "n_experts": 512}, True, False, (0.1, 0.1), 1.0),
    ("flat_bf16_n4096", {"tokens": 700, "n_experts": 96, "k": 6, "d_model": 256}, False, True,
     (0.1, 0.1), 1.0),
    # segments over 2048 rows: the experts' weight gradients in row chunks whose partial
    # sums are added afterwards (fp32 kernel; bf16 with 128- and 256-wide tiles)
    ("tiny_fp32", {"tokens": 6000, "n_experts": 3, "k": 2}, True, True, (0.1, 0.1), 1.0),
    ("flat_bf16_n4096", {"tokens": 8192, "n_experts": 4, "k": 2, "d_model": 256,
                         "d_hidden": 256}, True, True, (0.1, 0.1), 1.0),
    ("zipf_bf16_n256", {"tokens": 4000, "n_experts": 64, "d_hidden": 256}, True, False,
     (0.1, 0.1), 1.0),
    # bf16 gates in training mode take the gate's gradient pass (blocked pair gradients,
    # selected pairs rewritten): with a gate bias and a ragged last tile, one 16-expert
    # chunk, and k = 8
    ("flat_bf16_n4096", {"tokens": 1000, "n_experts": 48, "k": 3, "d_model": 128}, True, True,
     (0.3, 1.0), 2.0),
    ("flat_bf16_n4096", {"tokens": 333, "n_experts": 16, "k": 2, "d_model": 256,
                         "d_hidden": 128}, True, True, (0.1, 0.1), 1.0),
    ("flat_bf16_n4096", {"tokens": 520, "n_experts": 32, "k": 8, "d_model": 256,
                         "d_hidden": 256}, True, False, (0.1, 0.1), 1.0),
]


def _id(c):
    name, kw, train, bias, wts, aux = c
    return name + "".join(f"-{k}{v}" for k, v in kw.items()) + f"-train{int(train)}-bias{int(bias)}"


def make_dy(w, seed):
    """Upstream gradient [B, d] in the activations' storage type."""
    dy = dg.normal(w.seed, 50 + seed, 0, w.tokens * w.d_model, 1.0, w.act_dtype)
    return dy.reshape(w.tokens, w.d_model)


KINK_REL = 1e-5


def resolve_kinks(inp, sel, gates, dy, ob, got_dw1):
    """ReLU's derivative is undefined at 0, and a hidden pre-activation within
    rounding of 0 can take either side on the GPU (fp32 accumulation) and in
    the oracle (fp64). Like a near tie in the selection, such an element
    ("near kink": |pre| <= KINK_REL * max(1, RMS(pre))) has two valid
    gradients: with the mask open, dA[p][j] = dHid[p][j] (the gradient that
    reaches the hidden unit), closed 0. For each near-kink element this takes
    the GPU's side (the one that makes its dW1 row agree better with the
    oracle's) and moves the oracle's dW1[e][j], db1[e][j] and dx[t] to it, in
    place. Returns the number of near-kink elements, asserted to be rare."""
    x = dg.as_f32(inp["x"]).astype(np.float64)
    W1 = dg.as_f32(inp["w1"]).astype(np.float64)
    W2 = dg.as_f32(inp["w2"]).astype(np.float64)
    b1 = dg.as_f32(inp["b1"]).astype(np.float64) if "b1" in inp else None
    B, k = sel.shape
    found = []
    sumsq, count = 0.0, 0
    for e in np.unique(sel):
        ts, js = np.nonzero(sel == e)
        pre = x[ts] @ W1[e].T + (b1[e] if b1 is not None else 0.0)
        sumsq += float((pre * pre).sum())
        count += pre.size
        found.append((e, ts, js, pre))
    tau = KINK_REL * max(1.0, np.sqrt(sumsq / max(count, 1)))
    n_kink = 0
    for e, ts, js, pre in found:
        for r, j in zip(*np.nonzero(np.abs(pre) <= tau)):
            n_kink += 1
            t, slot = ts[r], js[r]
            dO = gates[t, slot] * dy[t]
            dhid = float(dO @ W2[e][:, j])
            sign = -1.0 if pre[r, j] > 0 else 1.0  # a flip closes an open mask, opens a closed one
            delta_w1 = sign * dhid * x[t]
            before = np.abs(got_dw1[e, j] - ob["dw1"][e, j]).max()
            after = np.abs(got_dw1[e, j] - ob["dw1"][e, j] - delta_w1).max()
            if after < before:  # the GPU took the other side
                ob["dw1"][e, j] += delta_w1
                ob["db1"][e, j] += sign * dhid
                ob["dx"][t] += sign * dhid * W1[e][j]
    assert n_kink <= max(16, 1e-4 * count), f"{n_kink} near-kink pre-activations of {count}"
    return n_kink


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_backward_parity(case):
    name, kw, train, bias, (wi, wl), aux = case
    w = dg.workload(name, **kw)
    announce(f"moe_backward {w.name} {kw} train={train} bias={bias}")
    inp = dg.make_inputs(w, with_bias=bias)
    if bias and "gate_bias" not in inp:
        inp["gate_bias"] = (0.2 * dg.normal(w.seed, 60, 0, w.n_experts)).astype(np.float32)
    g = gpu_inputs(inp)
    fwd = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                          train=train, noise_floor=FLOOR, w_importance=wi, w_load=wl,
                          return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.gate(inp, w.k, train=train, noise_floor=FLOOR, want_logits=True)
    sel = to_host(fwd["topk_idx"])
    check_gating(ref, ref["H"], sel, to_host(fwd["topk_gate"]), to_host(fwd["thresh"]))
    dy = make_dy(w, 1)
    grads = moe.moe_backward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                             fwd["topk_idx"], fwd["topk_gate"], fwd["thresh"], fwd["importance"],
                             fwd["load"], to_device(dy), b1=g.get("b1"), b2=g.get("b2"),
                             gate_bias=g.get("gate_bias"), train=train, noise_floor=FLOOR,
                             w_importance=wi, w_load=wl, aux_scale=aux)
    torch.cuda.synchronize()
    ob = oracle.backward(inp, w.k, dg.as_f32(dy), aux_scale=aux, train=train, noise_floor=FLOOR,
                         w_importance=wi, w_load=wl, force_idx=sel)
    got_dw1 = to_host(grads["dw1"])
    nk = resolve_kinks(inp, sel, to_host(fwd["topk_gate"]), dg.as_f32(dy), ob, got_dw1)
    tol = out_tol(w.act_dtype == dg.BF16)
    errs, worst = {}, {}
    for key in ("dx", "dw_gate", "dw_noise", "dgate_bias", "dw1", "db1", "dw2", "db2"):
        if key not in grads:
            continue
        got = to_host(grads[key])
        if key == "dw_noise" and not train:
            assert np.all(got == 0.0)
            continue
        r = ob[key]
        errs[key] = rel_err(got, r)
        den = np.maximum(np.abs(r), np.sqrt(np.mean(r * r)))
        at = np.unravel_index(np.argmax(np.abs(got - r) / np.where(den == 0, 1, den)), r.shape)
        worst[key] = (tuple(int(i) for i in at), float(got[at]), float(r[at]))
    print(w.name, kw, train, {k: f"{v:.2e}" for k, v in errs.items()}, "near-kink", nk)
    bad = {k: (v, worst[k]) for k, v in errs.items() if v > tol}
    assert not bad, f"errors above {tol} (index, gpu, oracle): {bad}"


def test_backward_is_deterministic():
    w = dg.workload("flat_bf16_n4096", tokens=1000, n_experts=64, d_hidden=256)
    announce("moe_backward determinism")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    fwd = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          return_routing=True)
    dy = to_device(make_dy(w, 2))
    args = (g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k, fwd["topk_idx"],
            fwd["topk_gate"], fwd["thresh"], fwd["importance"], fwd["load"], dy)
    a = moe.moe_backward(*args)
    a = {k: v.clone() for k, v in a.items()}
    b = moe.moe_backward(*args)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_backward_empty_batch():
    w = dg.workload("tiny_fp32", tokens=0)
    announce("moe_backward empty batch")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    fwd = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          return_routing=True)
    dy = torch.empty((0, w.d_model), dtype=torch.float32, device="cuda")
    gr = moe.moe_backward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          fwd["topk_idx"], fwd["topk_gate"], fwd["thresh"], fwd["importance"],
                          fwd["load"], dy)
    torch.cuda.synchronize()
    assert to_host(gr["dx"]).shape == (0, w.d_model)
    for key in ("dw_gate", "dw_noise", "dw1", "dw2"):
        assert np.all(to_host(gr[key]) == 0.0), key


def resolve_kinks_sampled(inp, sel, gates, dy, ob, experts, tokens, got_dw1):
    """resolve_kinks for the sampled oracle: the near-kink pre-activations of
    the sampled experts' routed rows move the oracle's dW1 rows of those
    experts, and the sampled tokens' dx, to the GPU's side."""
    x = dg.as_f32(inp["x"]).astype(np.float64)
    W1 = dg.as_f32(inp["w1"]).astype(np.float64)
    W2 = dg.as_f32(inp["w2"]).astype(np.float64)
    b1 = dg.as_f32(inp["b1"]).astype(np.float64) if "b1" in inp else None
    tpos = {int(t): q for q, t in enumerate(tokens)}
    # (expert, rows): the sampled experts' routed rows and the sampled tokens' experts
    pairs = {}
    for q, e in enumerate(experts):
        ts, js = np.nonzero(sel == e)
        pairs.setdefault(int(e), set()).update(zip(ts.tolist(), js.tolist()))
    for t in tokens:
        for j in range(sel.shape[1]):
            pairs.setdefault(int(sel[t, j]), set()).add((int(t), j))
    found, sumsq, count = [], 0.0, 0
    for e, tj in pairs.items():
        tj = sorted(tj)
        ts = np.array([a for a, _ in tj], dtype=np.int64)
        js = np.array([b for _, b in tj], dtype=np.int64)
        pre = x[ts] @ W1[e].T + (b1[e] if b1 is not None else 0.0)
        sumsq += float((pre * pre).sum())
        count += pre.size
        found.append((e, ts, js, pre))
    tau = KINK_REL * max(1.0, np.sqrt(sumsq / max(count, 1)))
    eq = {int(e): q for q, e in enumerate(experts)}
    n_kink = 0
    for e, ts, js, pre in found:
        for r, j in zip(*np.nonzero(np.abs(pre) <= tau)):
            n_kink += 1
            t, slot = int(ts[r]), int(js[r])
            dhid = float((gates[t, slot] * dy[t]) @ W2[e][:, j])
            sign = -1.0 if pre[r, j] > 0 else 1.0
            took_other = False
            if e in eq:  # decide from the GPU's dW1 row of this expert
                q = eq[e]
                delta = sign * dhid * x[t]
                before = np.abs(got_dw1[q, j] - ob["dw1"][q, j]).max()
                after = np.abs(got_dw1[q, j] - ob["dw1"][q, j] - delta).max()
                took_other = after < before
                if took_other:
                    ob["dw1"][q, j] += delta
                    if "db1" in ob and ob["db1"].size:
                        ob["db1"][q, j] += sign * dhid
            if t in tpos and (took_other or e not in eq):
                # a sampled token whose expert is not sampled: take the side that agrees
                # with the GPU's dx (checked below against the bar either way)
                ob.setdefault("_dx_alt", {})[(tpos[t], e, j)] = sign * dhid * W1[e][j]
    assert n_kink <= max(16, 1e-4 * count), f"{n_kink} near-kink pre-activations of {count}"
    return n_kink


@pytest.mark.parametrize("name", ["flat_bf16_n4096", "zipf_bf16_n256"])
def test_backward_full_size_sampled(name):
    """The backward at full size in the launch configuration bench.py times
    (moe_backward with its own workspace, after moe_forward): 65536 tokens x 4096
    experts, and the Zipf-skewed 32768 tokens x 256 experts with its gate bias
    (about 21K rows on expert 0, whose weight gradients run in row chunks), both
    512-1024-512, k 4, bf16. Against the oracle's sampled backward with the GPU's
    selection forced: dW1, dW2 of six experts (the most and least popular, random
    ones), the gate-weight, noise-weight and gate-bias gradients of the same experts
    (sums over the whole batch, Importance and Load over the whole batch), and dx
    of 46 tokens (both ends, tile edges, random)."""
    w = dg.workload(name)
    B, d, n, k = w.tokens, w.d_model, w.n_experts, w.k
    announce(f"moe_backward full size {w.name}: generating inputs")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    fwd = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], k,
                          gate_bias=g.get("gate_bias"), train=True, noise_floor=FLOOR,
                          return_routing=True)
    dy = make_dy(w, 3)
    announce("moe_backward full size: GPU call")
    grads = moe.moe_backward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], k,
                             fwd["topk_idx"], fwd["topk_gate"], fwd["thresh"], fwd["importance"],
                             fwd["load"], to_device(dy), gate_bias=g.get("gate_bias"), train=True,
                             noise_floor=FLOOR)
    torch.cuda.synchronize()
    sel = to_host(fwd["topk_idx"])
    counts = np.bincount(sel.ravel(), minlength=n)
    rng = np.random.default_rng(11)
    nz = np.nonzero(counts)[0]
    experts = np.unique(np.concatenate([[int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])],
                                        rng.choice(n, 4, replace=False)])).astype(np.int32)
    edges = [0, 1, 63, 64, 255, 256, B // 2, B - 257, B - 2, B - 1]
    tokens = np.unique(np.concatenate([edges, rng.choice(B, 36, replace=False)])).astype(np.int64)
    announce(f"moe_backward full size: oracle gating on {tokens.size} rows")
    ref = oracle.gate(inp, k, train=True, noise_floor=FLOOR, rows=tokens, want_logits=True)
    check_gating(ref, ref["H"], sel, to_host(fwd["topk_gate"]), to_host(fwd["thresh"]), rows=tokens)
    announce(f"moe_backward full size: oracle sampled backward ({experts.size} experts, "
             f"{tokens.size} tokens)")
    ob = oracle.backward_sampled(inp, k, dg.as_f32(dy), gate_experts=experts, experts=experts,
                                 tokens=tokens, train=True, noise_floor=FLOOR, force_idx=sel)
    got = {"dw1": to_host(grads["dw1"])[experts], "dw2": to_host(grads["dw2"])[experts],
           "dw_gate": to_host(grads["dw_gate"])[experts],
           "dw_noise": to_host(grads["dw_noise"])[experts], "dx": to_host(grads["dx"])[tokens]}
    if "dgate_bias" in grads:
        got["dgate_bias"] = to_host(grads["dgate_bias"])[experts]
    nk = resolve_kinks_sampled(inp, sel, to_host(fwd["topk_gate"]), dg.as_f32(dy), ob, experts,
                               tokens, got["dw1"])
    for (q, e, j), delta in ob.pop("_dx_alt", {}).items():  # per token, the side nearer the GPU
        if np.abs(got["dx"][q] - ob["dx"][q] - delta).max() < np.abs(got["dx"][q] - ob["dx"][q]).max():
            ob["dx"][q] += delta
    tol = out_tol(True)
    errs = {}
    for key in ("dw1", "dw2", "dw_gate", "dw_noise"):
        errs[key] = max(rel_err(got[key][q], ob[key][q]) for q in range(experts.size))
    errs["dx"] = max(rel_err(got["dx"][q], ob["dx"][q]) for q in range(tokens.size))
    if "dgate_bias" in got:
        errs["dgate_bias"] = rel_err(got["dgate_bias"], ob["dgate_bias"])
    print(w.name, "full size: experts", experts.tolist(), "counts", counts[experts].tolist(),
          {kk: f"{v:.2e}" for kk, v in errs.items()}, "near-kink", nk)
    bad = {kk: v for kk, v in errs.items() if v > tol}
    assert not bad, f"errors above {tol}: {bad}"
