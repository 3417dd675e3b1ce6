"""GPU parity: every entry point of the C ABI against the oracle, on the same
seeded inputs (marked ``gpu``; run on an MI355X after building the library).

Stage tests feed the oracle's own intermediates (selection, routing, expert
outputs) to one kernel at a time, so each kernel is checked on inputs that do
not come from another kernel. The fused ``moe_forward`` is then checked end to
end, at sizes the oracle finishes in seconds (several tiles plus ragged tails)
and at the full 65536-token, 4096-expert size on sampled rows and properties.
"""
import numpy as np
import pytest

import datagen as dg
import oracle
from parity import (GATE_TOL, LOSS_TOL, TOL_BF16, TOL_F32, announce, check_gating, gpu_inputs,
                    near_tie_rows, out_tol, rel_err, scalar_rel, softmax_at, to_device, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsely_gated_mixture_moe_amd as moe  # noqa: E402

FLOOR = 1e-2


def wl(name, **kw):
    return dg.workload(name, **kw)


# Small and ragged shapes: several gate row-blocks and expert chunks plus tails.
GATE_CASES = [
    ("tiny_fp32", {}),
    ("tiny_fp32", {"tokens": 300}),
    ("tiny_fp32", {"tokens": 333, "n_experts": 37, "k": 3, "d_model": 128}),
    ("tiny_fp32", {"tokens": 130, "n_experts": 5, "k": 5}),
    ("tiny_fp32", {"tokens": 257, "n_experts": 9, "k": 1}),
    ("tiny_fp32", {"tokens": 200, "n_experts": 70, "k": 8, "d_model": 256}),
    ("flat_fp32_n32", {}),
    ("zipf_bf16_n256", {"tokens": 1500}),
    ("flat_bf16_n4096", {"tokens": 700}),
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 333, "k": 2, "d_model": 128}),
    ("flat_bf16_n4096", {"tokens": 555, "n_experts": 96, "k": 6, "d_model": 256}),
    ("flat_bf16_n4096", {"tokens": 257, "n_experts": 32, "k": 8}),
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 100, "k": 3}),
]


def _gate_ids(c):
    name, kw = c
    return name + "".join(f"-{k}{v}" for k, v in kw.items())


@pytest.mark.parametrize("case", GATE_CASES, ids=[_gate_ids(c) for c in GATE_CASES])
@pytest.mark.parametrize("train", [True, False])
def test_gate_parity(case, train):
    name, kw = case
    w = wl(name, **kw)
    announce(f"moe_gate {w.name} {kw} train={train}")
    inp = dg.make_inputs(w, experts=False)
    ref = oracle.gate(inp, w.k, train=train, noise_floor=FLOOR, want_logits=True)
    g = gpu_inputs(inp)
    idx, gate, thr = moe.moe_gate(g["x"], g["w_gate"], g["w_noise"], g["eps"] if train else None,
                                  w.k, train=train, noise_floor=FLOOR, gate_bias=g.get("gate_bias"))
    torch.cuda.synchronize()
    stats = check_gating(ref, ref["H"], to_host(idx), to_host(gate), to_host(thr))
    print(w.name, kw, train, {k: v for k, v in stats.items() if k != "swapped"},
          "swapped", len(stats["swapped"]))


# Batches of fewer than 128 row tiles split each tile's sweep over the experts
# when moe_gate has a workspace: one row, a few rows, a ragged tile, and the
# kernels of every dtype (chunks of 16 and 32 experts, tails in the last range).
SPLIT_CASES = [
    ("flat_bf16_n4096", {"tokens": 1}),
    ("flat_bf16_n4096", {"tokens": 7}),
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 512}),
    ("flat_bf16_n4096", {"tokens": 40, "n_experts": 100, "k": 3}),
    ("flat_bf16_n4096", {"tokens": 33, "n_experts": 96, "k": 6, "d_model": 256}),
    ("zipf_bf16_n256", {"tokens": 5}),
    ("tiny_fp32", {"tokens": 3}),
    ("tiny_fp32", {"tokens": 129, "n_experts": 37, "k": 3, "d_model": 128}),
    ("flat_fp32_n32", {"tokens": 64}),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[_gate_ids(c) for c in SPLIT_CASES])
@pytest.mark.parametrize("train", [True, False])
def test_gate_split_sweep(case, train):
    """The split sweep against the oracle, and bit-identical to one workgroup
    per row tile sweeping every expert (moe_gate without a workspace)."""
    name, kw = case
    w = wl(name, **kw)
    announce(f"moe_gate split {w.name} {kw} train={train}")
    inp = dg.make_inputs(w, experts=False, with_bias=(name == "zipf_bf16_n256"))
    ref = oracle.gate(inp, w.k, train=train, noise_floor=FLOOR, want_logits=True)
    g = gpu_inputs(inp)
    act = moe.MOE_F32 if g["x"].dtype == torch.float32 else moe.MOE_BF16
    dims = moe.make_dims(w.tokens, w.d_model, 128, w.n_experts, w.k, act, act,
                         moe.MOE_F32 if g["w_gate"].dtype == torch.float32 else moe.MOE_BF16)
    ws = moe.workspace(dims, moe.make_opts(train, FLOOR), g["x"].device)
    args = (g["x"], g["w_gate"], g["w_noise"], g["eps"] if train else None, w.k)
    kw2 = dict(train=train, noise_floor=FLOOR, gate_bias=g.get("gate_bias"))
    split = moe.moe_gate(*args, ws=ws, **kw2)
    whole = moe.moe_gate(*args, **kw2)
    torch.cuda.synchronize()
    for a_, b_ in zip(split, whole):
        assert np.array_equal(to_host(a_), to_host(b_))
    check_gating(ref, ref["H"], *[to_host(t) for t in split])


SWITCH_CASES = [
    ("flat_bf16_n4096", {"tokens": 700}, True),            # 32x32 kernel (bf16, training)
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 333, "k": 2, "d_model": 128}, False),
    ("zipf_bf16_n256", {"tokens": 1500, "k": 1}, True),    # Switch proper: k = 1
    ("tiny_fp32", {"tokens": 333, "n_experts": 37, "k": 3, "d_model": 128}, True),
    ("flat_bf16_n4096", {"tokens": 5}, True),               # split sweep
    ("flat_bf16_n4096", {"tokens": 3, "n_experts": 512}, False),
]


@pytest.mark.parametrize("case", SWITCH_CASES, ids=[_gate_ids(c[:2]) + f"-train{c[2]}" for c in SWITCH_CASES])
def test_gate_switch_order(case):
    """gate_order 1: the same selection and thresholds as the pages' order,
    the gates from the softmax over all n logits (running max and sum of
    exponentials over the sweep, merged across lanes and expert ranges)."""
    name, kw, train = case
    w = wl(name, **kw)
    announce(f"moe_gate switch order {w.name} {kw} train={train}")
    inp = dg.make_inputs(w, experts=False, with_bias=(name == "zipf_bf16_n256"))
    ref = oracle.gate(inp, w.k, train=train, noise_floor=FLOOR, want_logits=True, gate_order=1)
    g = gpu_inputs(inp)
    act = moe.MOE_F32 if g["x"].dtype == torch.float32 else moe.MOE_BF16
    dims = moe.make_dims(w.tokens, w.d_model, 128, w.n_experts, w.k, act, act,
                         moe.MOE_F32 if g["w_gate"].dtype == torch.float32 else moe.MOE_BF16)
    ws = moe.workspace(dims, moe.make_opts(train, FLOOR, gate_order=1), g["x"].device)
    for w_s in (ws, None):
        idx, gate, thr = moe.moe_gate(g["x"], g["w_gate"], g["w_noise"], g["eps"] if train else None,
                                      w.k, train=train, noise_floor=FLOOR,
                                      gate_bias=g.get("gate_bias"), gate_order=1, ws=w_s)
        torch.cuda.synchronize()
        check_gating(ref, ref["H"], to_host(idx), to_host(gate), to_host(thr), gate_order=1)
        assert np.all(to_host(gate).sum(1) <= 1.0 + 1e-6)


# Inference on the 32x32 kernel (n a multiple of 32: chunks of 32 experts'
# clean rows): bf16 gate weights with the Zipf gate bias, both gate orders,
# whole and split sweeps.
CLEAN32_CASES = [
    ("zipf_bf16_n256", {"tokens": 1500}, 0),
    ("zipf_bf16_n256", {"tokens": 1500}, 1),
    ("zipf_bf16_n256", {"tokens": 3}, 0),
    ("flat_bf16_n4096", {"tokens": 3, "n_experts": 512}, 1),
    ("flat_bf16_n4096", {"tokens": 257, "n_experts": 96, "k": 8, "d_model": 256}, 0),
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 32, "k": 1, "d_model": 128}, 1),
]


@pytest.mark.parametrize("case", CLEAN32_CASES,
                         ids=[_gate_ids(c[:2]) + f"-order{c[2]}" for c in CLEAN32_CASES])
def test_gate_clean32(case):
    name, kw, order = case
    w = wl(name, gate_dtype=dg.BF16, zipf=True, **kw)
    announce(f"moe_gate clean-only 32x32 {w.name} {kw} gate_order={order}")
    inp = dg.make_inputs(w, experts=False)
    assert inp["w_gate"].dtype == np.uint16 and "gate_bias" in inp
    ref = oracle.gate(inp, w.k, train=False, noise_floor=FLOOR, want_logits=True,
                      gate_order=order)
    g = gpu_inputs(inp)
    dims = moe.make_dims(w.tokens, w.d_model, 128, w.n_experts, w.k, moe.MOE_BF16, moe.MOE_BF16,
                         moe.MOE_BF16)
    ws = moe.workspace(dims, moe.make_opts(False, FLOOR, gate_order=order), g["x"].device)
    for w_s in (ws, None):
        idx, gate, thr = moe.moe_gate(g["x"], g["w_gate"], g["w_noise"], None, w.k, train=False,
                                      noise_floor=FLOOR, gate_bias=g.get("gate_bias"),
                                      gate_order=order, ws=w_s)
        torch.cuda.synchronize()
        check_gating(ref, ref["H"], to_host(idx), to_host(gate), to_host(thr), gate_order=order)


def test_forward_switch_order():
    """The whole forward with gate_order 1 and k = 1 (Switch), fp32 so that y
    is held to the fp32 bar: y against the oracle's expert outputs weighted by
    the oracle's all-n softmax gates on the GPU's selection. (The bf16 gate
    kernels' gate_order 1 is covered by test_gate_switch_order.)"""
    w = wl("flat_fp32_n32", tokens=1500, k=1)
    announce("moe_forward switch order")
    inp = dg.make_inputs(w, with_bias=True)
    g = gpu_inputs(inp)
    out = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                          noise_floor=FLOOR, gate_order=1, return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.gate(inp, w.k, noise_floor=FLOOR, want_logits=True, gate_order=1)
    idx = to_host(out["topk_idx"])
    check_gating(ref, ref["H"], idx, to_host(out["topk_gate"]), to_host(out["thresh"]),
                 gate_order=1)
    same = np.all(idx == ref["topk_idx"], axis=1)
    tok = np.repeat(np.arange(w.tokens), w.k)
    eo = oracle.expert_pairs(inp, tok, idx.ravel()).reshape(w.tokens, w.k, w.d_model)
    y_ref = (ref["topk_gate"][:, :, None] * eo).sum(1)
    err = rel_err(to_host(out["y"])[same], y_ref[same])
    print("switch forward y err", err, "rows", int(same.sum()))
    assert err <= out_tol(False)


@pytest.mark.parametrize("case", [("flat_bf16_n4096", {"tokens": 1000, "n_experts": 512}),
                                  ("tiny_fp32", {"tokens": 300, "n_experts": 37, "k": 3})],
                         ids=["bf16-n512", "fp32-n37"])
def test_gate_and_load_with_noise_floor_zero(case):
    """sigma = Softplus(u) with no floor (eq 4 as written): sigma can be tiny, which
    stresses the relative accuracy of Softplus and of the Phi argument."""
    name, kw = case
    w = wl(name, **kw)
    announce(f"moe_gate / moe_aux_losses {w.name} {kw} noise_floor=0")
    inp = dg.make_inputs(w, experts=False)
    ref = oracle.gate(inp, w.k, noise_floor=0.0, want_logits=True)
    g = gpu_inputs(inp)
    idx, gate, thr = moe.moe_gate(g["x"], g["w_gate"], g["w_noise"], g["eps"], w.k,
                                  noise_floor=0.0)
    torch.cuda.synchronize()
    check_gating(ref, ref["H"], to_host(idx), to_host(gate), to_host(thr))
    rt = oracle.route(ref["topk_idx"], ref["topk_gate"], w.n_experts)
    load, losses = moe.moe_aux_losses(
        g["x"], g["w_gate"], g["w_noise"], to_device(ref["thresh"].astype(np.float32)),
        to_device(rt["offsets"]), to_device(rt["perm_token"]),
        to_device(rt["importance"].astype(np.float32)), w.k, noise_floor=0.0)
    torch.cuda.synchronize()
    load_ref = oracle.load(inp, w.k, noise_floor=0.0)
    err = rel_err(to_host(load), load_ref)
    print(w.name, kw, "floor 0 load err", err)
    assert err <= GATE_TOL


def _random_topk(B, n, k, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    if skew == 0.0:
        keys = rng.random((B, n))
    else:
        keys = rng.random((B, n)) * np.arange(1, n + 1) ** (-skew)
    idx = np.argsort(-keys, axis=1)[:, :k].astype(np.int32)
    gate = rng.random((B, k)).astype(np.float32)
    return idx, gate / gate.sum(1, keepdims=True)


ROUTE_CASES = [(256, 16, 2, 0.0), (1000, 37, 3, 0.0), (5000, 256, 4, 1.0), (3, 8, 8, 0.0),
               (4097, 4096, 4, 0.0), (0, 10, 2, 0.0)]


@pytest.mark.parametrize("B,n,k,skew", ROUTE_CASES)
def test_route_parity(B, n, k, skew):
    announce(f"moe_route B={B} n={n} k={k} skew={skew}")
    idx, gate = _random_topk(B, n, k, seed=B + n, skew=skew)
    ref = oracle.route(idx, gate, n)
    out = moe.moe_route(to_device(idx), to_device(gate), n)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm_token", "slot_pos"):
        assert np.array_equal(to_host(out[key]), ref[key]), key
    assert np.array_equal(to_host(out["perm_gate"]), ref["perm_gate"].astype(np.float32))
    assert rel_err(to_host(out["importance"]), ref["importance"]) <= 1e-5


@pytest.mark.parametrize("B,n,k", [(65536, 4096, 4), (131072, 16384, 4)])
def test_route_full_size_against_stable_sort(B, n, k):
    """Full-size routing against numpy's stable argsort (a library routine)."""
    announce(f"moe_route full B={B} n={n}")
    idx, gate = _random_topk(B, n, k, seed=7)
    out = moe.moe_route(to_device(idx), to_device(gate), n)
    torch.cuda.synchronize()
    order = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(to_host(out["perm_token"]), (order // k).astype(np.int32))
    assert np.array_equal(to_host(out["counts"]), np.bincount(idx.ravel(), minlength=n))
    inv = np.empty(B * k, np.int32)
    inv[order] = np.arange(B * k)
    assert np.array_equal(to_host(out["slot_pos"]), inv)
    imp = np.bincount(idx.ravel(), weights=gate.ravel().astype(np.float64), minlength=n)
    assert rel_err(to_host(out["importance"]), imp) <= 1e-5


# capacity < the largest count: dropped pairs in both route paths (one workgroup for
# at most 1024 pairs, five kernels above), skewed so that popular experts overflow
CAPACITY_ROUTE_CASES = [(200, 16, 2, 1.0, 20), (3, 8, 8, 0.0, 1), (3000, 64, 4, 1.0, 150),
                        (65536, 4096, 4, 0.0, 70)]


@pytest.mark.parametrize("B,n,k,skew,cap", CAPACITY_ROUTE_CASES)
def test_route_capacity_parity(B, n, k, skew, cap):
    announce(f"moe_route capacity B={B} n={n} k={k} cap={cap}")
    idx, gate = _random_topk(B, n, k, seed=B + 3 * n, skew=skew)
    ref = oracle.route(idx, gate, n, capacity=cap)
    assert (ref["slot_pos"] < 0).any()  # the case drops pairs
    out = moe.moe_route(to_device(idx), to_device(gate), n, capacity=cap)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm_token", "slot_pos"):
        assert np.array_equal(to_host(out[key]), ref[key]), key
    assert rel_err(to_host(out["importance"]), ref["importance"]) <= 1e-5


@pytest.mark.parametrize("case,cap", [(("zipf_bf16_n256", {"tokens": 2000}), 40),
                                      (("flat_bf16_n4096", {"tokens": 700, "n_experts": 64}), 30),
                                      (("tiny_fp32", {"tokens": 200}), 20)])
def test_forward_capacity_parity(case, cap):
    """The whole forward with a fixed expert capacity: gating against the
    oracle as everywhere; y against the oracle's routing of the GPU's own
    selection with the same capacity (so a near tie elsewhere cannot move the
    ranks), summing only the served slots of each token."""
    name, kw = case
    w = wl(name, **kw)
    announce(f"moe_forward capacity {w.name} {kw} cap={cap}")
    inp = dg.make_inputs(w, with_bias=(name == "zipf_bf16_n256"))
    g = gpu_inputs(inp)
    out = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                          noise_floor=FLOOR, capacity=cap, return_routing=True)
    torch.cuda.synchronize()
    ref_g = oracle.gate(inp, w.k, noise_floor=FLOOR, want_logits=True)
    check_gating(ref_g, ref_g["H"], to_host(out["topk_idx"]), to_host(out["topk_gate"]),
                 to_host(out["thresh"]))
    idx, gate = to_host(out["topk_idx"]), to_host(out["topk_gate"]).astype(np.float64)
    rt = oracle.route(idx, gate, w.n_experts, capacity=cap)
    served = rt["slot_pos"] >= 0
    assert not served.all()
    tok = np.repeat(np.arange(w.tokens), w.k)[served]
    eo = oracle.expert_pairs(inp, tok, idx.ravel()[served])
    y_ref = np.zeros((w.tokens, w.d_model))
    np.add.at(y_ref, tok, gate.ravel()[served][:, None] * eo)
    err = rel_err(to_host(out["y"]), y_ref)
    print(w.name, kw, "cap", cap, "served", served.mean(), "y err", err)
    assert err <= out_tol(w.act_dtype == dg.BF16)
    assert np.array_equal(to_host(out["counts"]), rt["counts"])


def test_route_drops_out_of_range_entries():
    announce("moe_route out-of-range entries")
    idx = np.array([[0, 3], [-1, 2], [3, 9], [2, 0]], np.int32)
    gate = np.full((4, 2), 0.5, np.float32)
    out = moe.moe_route(to_device(idx), to_device(gate), 4)
    torch.cuda.synchronize()
    assert to_host(out["counts"]).tolist() == [2, 0, 2, 2]
    assert to_host(out["offsets"]).tolist() == [0, 2, 2, 4, 6]
    assert to_host(out["perm_token"])[:6].tolist() == [0, 3, 1, 3, 0, 2]
    sp = to_host(out["slot_pos"]).tolist()
    assert sp[2] == -1 and sp[5] == -1
    assert to_host(out["importance"]).tolist() == [1.0, 0.0, 1.0, 1.0]


FFN_CASES = [
    ("tiny_fp32", {}, True),
    ("tiny_fp32", {"tokens": 300, "n_experts": 7, "k": 2, "d_model": 128, "d_hidden": 256}, True),
    ("tiny_fp32", {"tokens": 200, "n_experts": 5, "k": 2, "d_model": 256}, False),
    ("flat_fp32_n32", {"tokens": 700}, True),
    ("zipf_bf16_n256", {"tokens": 1200}, True),
    ("flat_bf16_n4096", {"tokens": 300, "n_experts": 40, "d_model": 64, "d_hidden": 128}, True),
    ("flat_bf16_n4096", {"tokens": 600, "n_experts": 64}, False),
    # batches of few units, split over hidden-chunk ranges (partial sums + reduction)
    ("flat_bf16_n4096", {"tokens": 2, "n_experts": 64}, True),
    ("tiny_fp32", {"tokens": 5}, True),
    ("flat_bf16_n4096", {"tokens": 20, "n_experts": 16, "d_model": 256, "d_hidden": 384}, False),
    # long segments: many 96-row units of one expert, ragged tails, a 768-unit hidden layer
    ("flat_bf16_n4096", {"tokens": 2600, "n_experts": 8, "k": 2}, True),
    ("flat_bf16_n4096", {"tokens": 1500, "n_experts": 4, "k": 1, "d_model": 256,
                         "d_hidden": 256}, False),
    ("zipf_bf16_n256", {"tokens": 4100, "n_experts": 16, "k": 3, "d_hidden": 768}, True),
]


def _routed(w, inp, train=True):
    ref = oracle.gate(inp, w.k, train=train, noise_floor=FLOOR)
    return ref, oracle.route(ref["topk_idx"], ref["topk_gate"], w.n_experts)


@pytest.mark.parametrize("case", FFN_CASES, ids=[_gate_ids(c[:2]) + f"-bias{c[2]}" for c in FFN_CASES])
def test_expert_ffn_parity(case):
    name, kw, bias = case
    w = wl(name, **kw)
    announce(f"moe_expert_ffn {w.name} {kw} bias={bias}")
    inp = dg.make_inputs(w, with_bias=bias)
    _, rt = _routed(w, inp)
    g = gpu_inputs(inp)
    eo = moe.moe_expert_ffn(g["x"], to_device(rt["offsets"]), to_device(rt["perm_token"]), g["w1"],
                            g["w2"], w.k, b1=g.get("b1"), b2=g.get("b2"))
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(w.n_experts, dtype=np.int32), rt["counts"])
    ref = oracle.expert_pairs(inp, rt["perm_token"], experts)
    err = rel_err(to_host(eo), ref)
    print(w.name, kw, "expert_out err", err)
    assert err <= out_tol(w.act_dtype == dg.BF16)


@pytest.mark.parametrize("case", FFN_CASES[:5], ids=[_gate_ids(c[:2]) for c in FFN_CASES[:5]])
def test_combine_parity(case):
    name, kw, bias = case
    w = wl(name, **kw)
    announce(f"moe_combine {w.name} {kw}")
    inp = dg.make_inputs(w, with_bias=bias)
    ref, rt = _routed(w, inp)
    experts = np.repeat(np.arange(w.n_experts, dtype=np.int32), rt["counts"])
    eo = oracle.expert_pairs(inp, rt["perm_token"], experts).astype(np.float32)
    if w.act_dtype == dg.BF16:
        eo = dg.f32_to_bf16(eo)
    y = moe.moe_combine(to_device(eo), to_device(rt["slot_pos"]),
                        to_device(ref["topk_gate"].astype(np.float32)), n_experts=w.n_experts)
    torch.cuda.synchronize()
    y_ref = oracle.y_rows(inp, w.k, noise_floor=FLOOR)
    err = rel_err(to_host(y), y_ref)
    print(w.name, kw, "y err", err)
    assert err <= out_tol(w.act_dtype == dg.BF16)


# plus segments long enough for the Load correction to split them over 8 and
# 16 workgroups per expert (uniform and Zipf-skewed routing)
AUX_CASES = GATE_CASES[:4] + GATE_CASES[6:] + [
    ("flat_bf16_n4096", {"tokens": 16384, "n_experts": 8, "k": 2}),
    ("zipf_bf16_n256", {"tokens": 16384, "n_experts": 64}),
    # every size class of the CV^2 kernel (up to 4096, 16384 and 32768 experts)
    ("flat_bf16_n4096", {"tokens": 96, "n_experts": 4112, "d_model": 128}),
    ("flat_bf16_n4096", {"tokens": 64, "n_experts": 20000, "d_model": 128}),
    ("flat_bf16_n4096", {"tokens": 64, "n_experts": 32768, "k": 2, "d_model": 128}),
]


@pytest.mark.parametrize("case", AUX_CASES, ids=[_gate_ids(c) for c in AUX_CASES])
@pytest.mark.parametrize("train", [True, False])
def test_aux_losses_parity(case, train):
    name, kw = case
    w = wl(name, **kw)
    announce(f"moe_aux_losses {w.name} {kw} train={train}")
    inp = dg.make_inputs(w, experts=False)
    ref, rt = _routed(w, inp, train=train)
    load_ref = oracle.load(inp, w.k, train=train, noise_floor=FLOOR)
    g = gpu_inputs(inp)
    load, losses = moe.moe_aux_losses(
        g["x"], g["w_gate"], g["w_noise"], to_device(ref["thresh"].astype(np.float32)),
        to_device(rt["offsets"]), to_device(rt["perm_token"]),
        to_device(rt["importance"].astype(np.float32)), w.k, train=train, noise_floor=FLOOR,
        w_importance=0.1, w_load=0.3, gate_bias=g.get("gate_bias"))
    torch.cuda.synchronize()
    err = rel_err(to_host(load), load_ref)
    print(w.name, kw, train, "load err", err)
    assert err <= GATE_TOL
    lo = to_host(losses)
    cv_imp = oracle.cv2(rt["importance"].astype(np.float32))
    cv_load = oracle.cv2(load_ref)
    assert scalar_rel(lo[0], cv_imp) <= LOSS_TOL
    assert scalar_rel(lo[1], cv_load) <= LOSS_TOL
    assert scalar_rel(lo[2], 0.1 * cv_imp + 0.3 * cv_load) <= LOSS_TOL


def check_forward(w, inp, out, train, rows=None, full_load=True, w_imp=0.1, w_load=0.1,
                  y_rows=None):
    """End-to-end check of moe_forward's outputs against the oracle: gating on
    ``rows`` (default all), y on ``y_rows`` (default the same rows)."""
    B, n, k = w.tokens, w.n_experts, w.k
    sel_rows = np.arange(B) if rows is None else np.asarray(rows)
    g_idx = to_host(out["topk_idx"])
    g_gate = to_host(out["topk_gate"])
    g_thr = to_host(out["thresh"])
    ref = oracle.gate(inp, k, train=train, noise_floor=FLOOR, rows=sel_rows, want_logits=True)
    stats = check_gating(ref, ref["H"], g_idx, g_gate, g_thr, rows=sel_rows)
    # routing of the GPU's own selection: the stable sort by expert (a property at any size)
    order = np.argsort(g_idx.ravel(), kind="stable")
    counts = to_host(out["counts"])
    assert np.array_equal(counts, np.bincount(g_idx.ravel(), minlength=n))
    assert np.array_equal(to_host(out["perm_token"]), (order // k).astype(np.int32))
    # y on the checked rows; rows whose near-tie selection differs are checked on the GPU's set
    yr = sel_rows if y_rows is None else np.asarray(y_rows)
    y = to_host(out["y"])[yr]
    y_ref = oracle.y_rows(inp, k, rows=yr, train=train, noise_floor=FLOOR)
    at = {int(t): i for i, t in enumerate(yr)}
    for r in stats["swapped"]:
        t = int(sel_rows[r])
        if t not in at:
            continue
        sel = g_idx[t]
        gates = softmax_at(ref["H"][r], sel)
        eo = oracle.expert_pairs(inp, [t] * k, sel)
        y_ref[at[t]] = (gates[:, None] * eo).sum(0)
    yerr = rel_err(y, y_ref)
    assert yerr <= out_tol(w.act_dtype == dg.BF16), f"y error {yerr}"
    # Importance: the gate sums of the GPU's selection; on full-batch checks
    # against the oracle, adjusted for near-tie rows where the GPU chose another valid set.
    imp = to_host(out["importance"])
    assert scalar_rel(imp.sum(), B) <= 1e-5
    res = {"y_err": yerr, "near_tie": stats["near_tie"], "swapped": len(stats["swapped"])}
    if rows is None:
        full = oracle.route(ref["topk_idx"], ref["topk_gate"], n)["importance"]
        for r in stats["swapped"]:
            np.subtract.at(full, ref["topk_idx"][r], ref["topk_gate"][r])
            np.add.at(full, g_idx[r], softmax_at(ref["H"][r], g_idx[r]))
        ierr = rel_err(imp, full)
        assert ierr <= GATE_TOL, f"importance error {ierr}"
        res["imp_err"] = ierr
    else:
        full = np.bincount(g_idx.ravel(), weights=g_gate.ravel().astype(np.float64), minlength=n)
        assert rel_err(imp, full) <= 1e-5
    load = to_host(out["load"])
    lo = to_host(out["losses"])
    if full_load:
        load_ref = oracle.load(inp, k, train=train, noise_floor=FLOOR)
        lerr = rel_err(load, load_ref)
        assert lerr <= GATE_TOL, f"load error {lerr}"
        res["load_err"] = lerr
        cv_imp, cv_load = oracle.cv2(full), oracle.cv2(load_ref)
        assert scalar_rel(lo[0], cv_imp) <= LOSS_TOL
        assert scalar_rel(lo[1], cv_load) <= LOSS_TOL
        assert scalar_rel(lo[2], w_imp * cv_imp + w_load * cv_load) <= LOSS_TOL
    return res


FWD_CASES = [
    ("flat_bf16_n4096", {"tokens": 3, "n_experts": 512, "d_hidden": 256}, False),
    ("flat_bf16_n4096", {"tokens": 200, "n_experts": 1024, "d_hidden": 128}, True),
    ("tiny_fp32", {}, True),
    ("tiny_fp32", {"tokens": 333, "n_experts": 37, "k": 3, "d_model": 128}, False),
    ("tiny_fp32", {"tokens": 100, "n_experts": 4, "k": 4}, False),
    ("flat_fp32_n32", {}, False),
    ("zipf_bf16_n256", {"tokens": 4096}, False),
    ("flat_bf16_n4096", {"tokens": 2048, "n_experts": 512}, False),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[_gate_ids(c[:2]) for c in FWD_CASES])
@pytest.mark.parametrize("train", [True, False])
def test_forward_parity(case, train):
    name, kw, bias = case
    w = wl(name, **kw)
    announce(f"moe_forward {w.name} {kw} train={train} bias={bias}")
    inp = dg.make_inputs(w, with_bias=bias)
    g = gpu_inputs(inp)
    out = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                          train=train, noise_floor=FLOOR, return_routing=True)
    torch.cuda.synchronize()
    res = check_forward(w, inp, out, train)
    print(w.name, kw, train, res)


def test_forward_full_size_sampled():
    """The benchmark's workload in the benchmark's launch configuration
    (MoeForward, training mode, default options): 65536 tokens, 4096 experts
    512-1024-512, k 4, bf16. Gating and y are checked on sampled rows (both
    ends, tile edges and random rows), routing and Importance on the whole
    batch through properties, and Load and the losses against the oracle's
    full-batch Load."""
    w = wl("flat_bf16_n4096")
    B, d, n, k = w.tokens, w.d_model, w.n_experts, w.k
    announce(f"moe_forward full size {w.name}: generating inputs")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], k,
                       gate_bias=g.get("gate_bias"), train=True)
    dev = g["x"].device
    out = {"topk_idx": torch.empty((B, k), dtype=torch.int32, device=dev),
           "topk_gate": torch.empty((B, k), dtype=torch.float32, device=dev),
           "thresh": torch.empty((B, 2), dtype=torch.float32, device=dev),
           "counts": torch.empty(n, dtype=torch.int32, device=dev),
           "perm_token": torch.empty(B * k, dtype=torch.int32, device=dev)}
    announce("moe_forward full size: GPU call")
    y = f(g["x"], g["eps"], **out)
    torch.cuda.synchronize()
    out.update(y=y, importance=f.importance, load=f.load, losses=f.losses)
    rng = np.random.default_rng(7)
    edges = [0, 1, 127, 128, 255, 256, 257, B // 2, B - 257, B - 256, B - 2, B - 1]
    rows = np.unique(np.concatenate([edges, rng.choice(B, 400, replace=False)]))
    announce("moe_forward full size: oracle on sampled rows and full-batch Load")
    res = check_forward(w, inp, out, True, rows=rows, full_load=True)
    print(w.name, "full size", len(rows), "rows", res)


def test_forward_zipf_full_size_sampled():
    """The Zipf-skewed workload at its full size in the benchmark's launch
    configuration (MoeForward, training mode): 32768 tokens, 256 experts
    512-1024-512, k 4, bf16 activations and experts, fp32 gate weights with
    the calibrated Zipf gate bias (about 21K rows on expert 0, over 200 FFN
    work units of that one expert). Gating, routing, Importance, Load and the
    losses are checked on the whole batch against the oracle; y on sampled
    rows: both ends, every FFN unit edge of the most popular expert's first
    and last units and a few in between, the whole segment of the least
    popular expert, and random rows."""
    w = wl("zipf_bf16_n256")
    B, d, n, k = w.tokens, w.d_model, w.n_experts, w.k
    announce(f"moe_forward full size {w.name}: generating inputs")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeForward((B, d), g["w_gate"], g["w_noise"], g["w1"], g["w2"], k,
                       gate_bias=g["gate_bias"], train=True)
    dev = g["x"].device
    out = {"topk_idx": torch.empty((B, k), dtype=torch.int32, device=dev),
           "topk_gate": torch.empty((B, k), dtype=torch.float32, device=dev),
           "thresh": torch.empty((B, 2), dtype=torch.float32, device=dev),
           "counts": torch.empty(n, dtype=torch.int32, device=dev),
           "perm_token": torch.empty(B * k, dtype=torch.int32, device=dev)}
    announce("moe_forward zipf full size: GPU call")
    y = f(g["x"], g["eps"], **out)
    torch.cuda.synchronize()
    out.update(y=y, importance=f.importance, load=f.load, losses=f.losses)
    counts = to_host(out["counts"])
    perm = to_host(out["perm_token"])
    off = np.concatenate([[0], np.cumsum(counts)])
    top, last = int(np.argmax(counts)), int(np.argmin(counts))
    assert counts[top] > 10000, f"the skew is gone: top expert has {counts[top]} rows"
    unit = 96  # rows per FFN work unit of the bf16 kernel at d = 512
    seg = perm[off[top]:off[top + 1]]
    pos = []
    for u in list(range(3)) + list(range(len(seg) // unit - 2, (len(seg) + unit - 1) // unit)) + \
            [len(seg) // (2 * unit)]:
        for p in (u * unit, u * unit + 1, u * unit + unit - 1):
            if 0 <= p < len(seg):
                pos.append(p)
    rng = np.random.default_rng(3)
    edges = [0, 1, 255, 256, 257, B // 2, B - 257, B - 256, B - 2, B - 1]
    y_rows = np.unique(np.concatenate([edges, seg[pos], perm[off[last]:off[last + 1]],
                                       rng.choice(B, 200, replace=False)]))
    announce(f"moe_forward zipf full size: oracle, gating on all rows, y on {len(y_rows)} rows")
    res = check_forward(w, inp, out, True, rows=None, full_load=True, y_rows=y_rows)
    print(w.name, "full size: top expert", top, counts[top], "rows; least", last, counts[last],
          "; y rows", len(y_rows), res)


def test_forward_is_deterministic():
    w = wl("zipf_bf16_n256", tokens=2048)
    announce("moe_forward determinism")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w1"], g["w2"], w.k,
                       gate_bias=g["gate_bias"])
    y1 = f(g["x"], g["eps"]).clone()
    l1 = (f.importance.clone(), f.load.clone(), f.losses.clone())
    y2 = f(g["x"], g["eps"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for a, b in zip(l1, (f.importance, f.load, f.losses)):
        assert torch.equal(a, b)


def test_ffn_timing_counts_forward_calls():
    w = wl("flat_bf16_n4096", tokens=4096, n_experts=256)
    announce("moe_ffn_timing")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w1"], g["w2"], w.k)
    f(g["x"], g["eps"])
    moe.moe_ffn_timing(True)
    try:
        for _ in range(3):
            f(g["x"], g["eps"])
    finally:
        moe.moe_ffn_timing(False)
    f(g["x"], g["eps"])  # not timed
    n, ms = moe.moe_ffn_timing_read()
    assert n == 3 and ms > 0


@pytest.mark.parametrize("tokens,train", [(3, False), (5, True), (3000, True)])
def test_forward_graph_replays(tokens, train):
    """moe_forward captured in a HIP graph (it allocates nothing, makes no
    copies or fills and never synchronizes): every replay, with eager calls
    of the same MoeForward on other inputs and synchronizations in between,
    gives exactly the eager outputs. Small batches take the split gate and
    FFN and the one-workgroup route."""
    w = wl("flat_bf16_n4096", tokens=tokens, n_experts=256, d_hidden=256)
    announce(f"moe_forward graph replay tokens={tokens} train={train}")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w1"], g["w2"], w.k,
                       train=train)
    x, eps = g["x"].clone(), g["eps"].clone()
    y = torch.empty_like(x)
    idx = torch.empty((w.tokens, w.k), dtype=torch.int32, device=x.device)
    f(x, eps, y, topk_idx=idx)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, idx, f.importance, f.load, f.losses)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(x, eps, y, topk_idx=idx)
    other_x, other_eps = torch.flip(x, [0]).contiguous(), torch.flip(eps, [0]).contiguous()
    for _ in range(3):
        f(other_x, other_eps)  # eager work on the same workspace and loss buffers
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(ref, (y, idx, f.importance, f.load, f.losses)):
            assert torch.equal(a_, b_)


def test_empty_batch():
    w = wl("tiny_fp32", tokens=0)
    announce("moe_forward empty batch")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    out = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], w.k,
                          return_routing=True)
    torch.cuda.synchronize()
    assert to_host(out["y"]).shape == (0, w.d_model)
    assert np.all(to_host(out["importance"]) == 0) and np.all(to_host(out["load"]) == 0)
    assert np.all(to_host(out["losses"]) == 0)
