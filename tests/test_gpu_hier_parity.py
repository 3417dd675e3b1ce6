"""GPU parity of the hierarchical layer (section "Hierarchical MoE" of the
explainer; ``moe_hier_forward`` through the C ABI) against the oracle.

Each gate level is compared with the oracle's: the same selections on every
row that is not a near tie, and a valid top-k within the margin on near-tie
rows. The oracle is then re-run with the GPU's selections forced at both
levels (so the secondary gates see the same groups in the same rank order),
and every output is compared with it: leaf ids bit-exactly, gates, y,
Importance, both levels' Load and the leaf Load, and the losses within the
stated tolerances. The hierarchy's losses are this library's own reading
(the pages give none); the oracle's version is pinned at its limits (the
flat layer, the dense mixture, hard counts at train = 0 and with vanishing
noise: tests/test_oracle_hier_pins.py).
"""
import numpy as np
import pytest

import datagen as dg
import oracle
from parity import (GATE_TOL, LOSS_TOL, announce, check_gating, device_tensor, gpu_inputs,
                    out_tol, rel_err, scalar_rel, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsely_gated_mixture_moe_amd as moe  # noqa: E402

FLOOR = 1e-2


def hier_wl(tokens, a, b, k1, k2, d=512, h=128, dtype=dg.BF16):
    return dg.workload("hier_bf16_16384", tokens=tokens, d_model=d, d_hidden=h, groups=a,
                       group_experts=b, k1=k1, k2=k2, n_experts=a * b, k=k1 * k2,
                       act_dtype=dtype, expert_dtype=dtype, gate_dtype=dtype)


# (tokens, a, b, k1, k2, d, h, dtype): fp32 and bf16; primary and secondary
# gates on the 16x16 kernel (fp32, or n not a multiple of 16) and on the 32x32
# kernel (bf16, n a multiple of 16, d >= 128); ragged batches; every group
# kept (k2 = b); groups that receive no rows; several secondary tiles per group.
CASES = [
    (300, 4, 6, 2, 2, 64, 128, dg.F32),
    (257, 5, 7, 3, 2, 128, 128, dg.F32),
    (1000, 8, 32, 2, 2, 128, 256, dg.BF16),
    (777, 16, 16, 2, 3, 256, 128, dg.BF16),
    (600, 32, 16, 1, 4, 512, 128, dg.BF16),
    (513, 6, 4, 2, 4, 128, 128, dg.BF16),
    (4096, 32, 64, 2, 2, 512, 128, dg.BF16),
    (200, 64, 16, 2, 2, 128, 128, dg.BF16),
]


def _id(c):
    B, a, b, k1, k2, d, h, dt = c
    return f"B{B}-a{a}-b{b}-k{k1}x{k2}-d{d}-{'bf16' if dt == dg.BF16 else 'f32'}"


def run_hier(w, inp, train, **kw):
    g = gpu_inputs(inp)
    out = moe.moe_hier_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w_gate2"],
                               g["w_noise2"], g["eps2"], g["w1"], g["w2"], w.k1, w.k2,
                               b1=g.get("b1"), b2=g.get("b2"), train=train, noise_floor=FLOOR,
                               return_all=True, **kw)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def check_hier(w, inp, out, train, w_imp=0.1, w_load=0.1):
    B, a, b, k1, k2 = w.tokens, w.groups, w.group_experts, w.k1, w.k2
    K, n = k1 * k2, a * b
    # primary gate
    ref = oracle.hier_gate(inp, k1, k2, train=train, noise_floor=FLOOR, want_logits=True)
    s1 = check_gating({"topk_idx": ref["sel1"], "topk_gate": ref["gate1"], "thresh": ref["thr1"]},
                      ref["H1"], out["group_idx"], out["group_gate"], out["group_thresh"])
    # secondary gates on the GPU's groups, in the GPU's rank order
    f1 = out["group_idx"]
    ref2 = oracle.hier_gate(inp, k1, k2, train=train, noise_floor=FLOOR, want_logits=True,
                            force1=f1)
    s2 = check_gating({"topk_idx": ref2["sel2"].reshape(B * k1, k2),
                       "topk_gate": ref2["gate2"].reshape(B * k1, k2),
                       "thresh": ref2["thr2"].reshape(B * k1, 2)},
                      ref2["H2"].reshape(B * k1, b), out["sub_idx"].reshape(B * k1, k2),
                      out["sub_gate"].reshape(B * k1, k2), out["sub_thresh"].reshape(B * k1, 2))
    # everything downstream against the oracle on the GPU's selections
    fo = oracle.hier_forward(inp, k1, k2, train=train, noise_floor=FLOOR, w_importance=w_imp,
                             w_load=w_load, force1=f1, force2=out["sub_idx"])
    assert np.array_equal(out["topk_idx"], fo["leaf_idx"])
    assert rel_err(out["topk_gate"], fo["leaf_gate"]) <= GATE_TOL
    assert np.array_equal(out["counts"], np.bincount(out["topk_idx"].ravel(), minlength=n))
    assert np.array_equal(out["group_rows"], fo["rows1"].astype(np.int32))
    yerr = rel_err(out["y"], fo["y"])
    assert yerr <= out_tol(w.act_dtype == dg.BF16), f"y error {yerr}"
    errs = {"y": yerr}
    for key, rkey in (("importance", "importance"), ("group_importance", "imp1"),
                      ("group_load", "load1"), ("sub_load", "load2"), ("load", "load")):
        e = rel_err(out[key], fo[rkey])
        assert e <= GATE_TOL, f"{key} error {e}"
        errs[key] = e
    for i in range(3):
        assert scalar_rel(out["losses"][i], fo["losses"][i]) <= LOSS_TOL, \
            f"loss {i}: {out['losses'][i]} vs {fo['losses'][i]}"
    errs.update(near_tie1=int(s1["near_tie"]), swapped1=len(s1["swapped"]),
                near_tie2=int(s2["near_tie"]), swapped2=len(s2["swapped"]))
    return errs


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
@pytest.mark.parametrize("train", [True, False])
def test_hier_forward_parity(case, train):
    B, a, b, k1, k2, d, h, dt = case
    w = hier_wl(B, a, b, k1, k2, d, h, dt)
    announce(f"moe_hier_forward {_id(case)} train={train}")
    inp = dg.make_hier_inputs(w, with_bias=(B % 2 == 1))
    out = run_hier(w, inp, train, w_importance=0.2, w_load=0.05)
    print(_id(case), train, check_hier(w, inp, out, train, w_imp=0.2, w_load=0.05))


def test_hier_empty_groups_and_full_groups():
    # k2 = b keeps every expert of a picked group (thresholds -inf at level 2,
    # P = 1) and 64 groups over 40 tokens leave most groups without rows.
    w = hier_wl(40, 64, 4, 2, 4, d=128, h=128)
    announce("moe_hier_forward empty and full groups")
    inp = dg.make_hier_inputs(w)
    out = run_hier(w, inp, True)
    assert np.all(np.isneginf(out["sub_thresh"][:, :, 1]))
    assert (out["group_rows"] == 0).sum() > 0
    res = check_hier(w, inp, out, True)
    print(res)


def test_hier_is_deterministic():
    w = hier_wl(1000, 8, 32, 2, 2, d=256)
    announce("moe_hier_forward determinism")
    inp = dg.make_hier_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeHierForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w_gate2"],
                           g["w_noise2"], g["w1"], g["w2"], 2, 2)
    y1 = f(g["x"], g["eps"], g["eps2"]).clone()
    l1 = (f.importance.clone(), f.load.clone(), f.losses.clone())
    y2 = f(g["x"], g["eps"], g["eps2"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for u, v in zip(l1, (f.importance, f.load, f.losses)):
        assert torch.equal(u, v)


def test_hier_empty_batch():
    w = hier_wl(0, 4, 16, 2, 2, d=128)
    announce("moe_hier_forward empty batch")
    inp = dg.make_hier_inputs(w)
    out = run_hier(w, inp, True)
    assert out["y"].shape == (0, 128)
    assert np.all(out["importance"] == 0) and np.all(out["load"] == 0)
    assert np.all(out["losses"] == 0)


@pytest.mark.timeout(900)
def test_hier_full_size_sampled():
    """The hierarchical workload at its full size in the benchmark's launch
    configuration (MoeHierForward, training mode): 131072 tokens, 128 groups
    x 128 experts 512-1024-512 (16384 leaves, 34.4 GB of bf16 expert weights
    generated on the device), k1 = k2 = 2. Both gate levels are checked on
    every row against the oracle (the secondary gates on the GPU's groups);
    the oracle, forced to the GPU's selections at both levels, then gives the
    leaves (bit-exact), their gates, the leaf counts, both levels' Importance
    and Load, the leaf Load and the losses over the whole batch; y is checked
    on sampled rows, each from its four leaves' weights regenerated on the
    host."""
    w = dg.WORKLOADS["hier_bf16_16384"]
    B, d, h = w.tokens, w.d_model, w.d_hidden
    a, b, k1, k2 = w.groups, w.group_experts, w.k1, w.k2
    n, K = a * b, k1 * k2
    announce("moe_hier_forward full size: gate inputs")
    inp = dg.make_hier_inputs(w, experts=False)
    g = gpu_inputs(inp)
    announce("moe_hier_forward full size: expert weights on the device")
    w1 = device_tensor(w, "w1", (n, h, d))
    w2 = device_tensor(w, "w2", (n, d, h))
    f = moe.MoeHierForward((B, d), g["w_gate"], g["w_noise"], g["w_gate2"], g["w_noise2"], w1, w2,
                           k1, k2, train=True)
    extra = {name: torch.empty(shp, dtype=dt, device=w1.device)
             for name, (shp, dt) in f.output_shapes().items()}
    announce("moe_hier_forward full size: GPU call")
    y = f(g["x"], g["eps"], g["eps2"], **extra)
    torch.cuda.synchronize()
    out = {key: to_host(v) for key, v in extra.items()}
    out.update(y=to_host(y), importance=to_host(f.importance), load=to_host(f.load),
               losses=to_host(f.losses))
    del w1, w2, f, extra
    torch.cuda.empty_cache()
    announce("moe_hier_forward full size: oracle gating, level 1")
    ref = oracle.hier_gate(inp, k1, k2, want_logits=True)
    s1 = check_gating({"topk_idx": ref["sel1"], "topk_gate": ref["gate1"], "thresh": ref["thr1"]},
                      ref["H1"], out["group_idx"], out["group_gate"], out["group_thresh"])
    f1 = out["group_idx"]
    del ref
    announce("moe_hier_forward full size: oracle gating, level 2 on the GPU's groups")
    ref2 = oracle.hier_gate(inp, k1, k2, want_logits=True, force1=f1)
    s2 = check_gating({"topk_idx": ref2["sel2"].reshape(B * k1, k2),
                       "topk_gate": ref2["gate2"].reshape(B * k1, k2),
                       "thresh": ref2["thr2"].reshape(B * k1, 2)},
                      ref2["H2"].reshape(B * k1, b), out["sub_idx"].reshape(B * k1, k2),
                      out["sub_gate"].reshape(B * k1, k2), out["sub_thresh"].reshape(B * k1, 2))
    del ref2
    announce("moe_hier_forward full size: oracle batch sums on the GPU's selections")
    fo = oracle.hier_forward(inp, k1, k2, force1=f1, force2=out["sub_idx"], with_y=False)
    assert np.array_equal(out["topk_idx"], fo["leaf_idx"])
    assert rel_err(out["topk_gate"], fo["leaf_gate"]) <= GATE_TOL
    assert np.array_equal(out["counts"], np.bincount(out["topk_idx"].ravel(), minlength=n))
    assert np.array_equal(out["group_rows"], fo["rows1"].astype(np.int32))
    errs = {}
    for key, rkey in (("importance", "importance"), ("group_importance", "imp1"),
                      ("group_load", "load1"), ("sub_load", "load2"), ("load", "load")):
        e = rel_err(out[key], fo[rkey])
        assert e <= GATE_TOL, f"{key} error {e}"
        errs[key] = e
    for i in range(3):
        assert scalar_rel(out["losses"][i], fo["losses"][i]) <= LOSS_TOL, \
            f"loss {i}: {out['losses'][i]} vs {fo['losses'][i]}"
    # y on sampled rows from the leaves' weights regenerated on the host
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, B // 2, B - 2, B - 1],
                                     rng.choice(B, 150, replace=False)]))
    leaves = np.unique(out["topk_idx"][rows])
    announce(f"moe_hier_forward full size: y on {len(rows)} rows ({len(leaves)} leaves)")
    where = {int(e): i for i, e in enumerate(leaves)}
    sub = {"x": inp["x"],
           "w1": np.stack([dg.gen(w, "w1", int(e) * h * d, h * d) for e in leaves]).reshape(-1, h, d),
           "w2": np.stack([dg.gen(w, "w2", int(e) * d * h, d * h) for e in leaves]).reshape(-1, d, h)}
    tok = np.repeat(rows, K)
    lv = out["topk_idx"][rows].ravel()
    eo = oracle.expert_pairs(sub, tok, [where[int(e)] for e in lv]).reshape(len(rows), K, d)
    order = np.argsort(out["topk_idx"][rows], axis=1, kind="stable")
    gates = np.take_along_axis(fo["leaf_gate"][rows], order, 1)
    eo = np.take_along_axis(eo, order[:, :, None], 1)
    y_ref = (gates[:, :, None] * eo).sum(1)
    yerr = rel_err(out["y"][rows], y_ref)
    assert yerr <= out_tol(True), f"y error {yerr}"
    errs.update(y=yerr, near_tie1=int(s1["near_tie"]), swapped1=len(s1["swapped"]),
                near_tie2=int(s2["near_tie"]), swapped2=len(s2["swapped"]))
    print("hier full size", errs)
