"""GPU parity of batchwise gating (moe_batchwise_forward) against the oracle.

Each expert's choice is compared with the oracle's column-wise choice on the
fp32 scores. Both sides decide in fp32, but the GPU's scores come from a
different accumulation order than the oracle's fp64 sums, so a column whose
m-th and (m+1)-th oracle scores (or a score and the threshold) are within the
near-tie margin may take another valid set; such a set is checked for
validity, and y, the gates and Importance are then checked against the oracle
evaluated on the GPU's choice.
"""
import numpy as np
import pytest

import datagen as dg
import oracle
from parity import (GATE_TOL, LOSS_TOL, NEAR_TIE_ABS, NEAR_TIE_REL, announce, gpu_inputs,
                    out_tol, rel_err, scalar_rel, to_device, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsely_gated_mixture_moe_amd as moe  # noqa: E402

FLOOR = 1e-2


def margin(v):
    return NEAR_TIE_REL * np.abs(v) + NEAR_TIE_ABS


def gpu_keep(out, B, n, m):
    """The GPU's choice as a [B, n] mask, after checking each list's form."""
    counts = to_host(out["counts"])
    tok = to_host(out["sel_token"]).reshape(n, m)
    keep = np.zeros((B, n), bool)
    for e in range(n):
        c = int(counts[e])
        assert 0 <= c <= m
        lst = tok[e, :c]
        assert np.all((lst >= 0) & (lst < B)), f"expert {e}: row out of range"
        assert np.all(np.diff(lst) > 0), f"expert {e}: rows not ascending"
        keep[lst, e] = True
    return counts, keep


def check_column_choice(S32, keep_gpu, keep_ref, m, thr):
    """Columns where the GPU's choice differs from the oracle's must be near
    ties: every row the GPU took scores (within the margin) at least as high
    as every passing row it left, its rows pass the threshold (within the
    margin), and it took min(m, passing rows) rows up to rows at the
    threshold's margin."""
    diff = np.flatnonzero((keep_gpu != keep_ref).any(axis=0))
    for e in diff:
        col = S32[:, e]
        t = -np.inf if thr is None else float(thr[e])
        took, left = keep_gpu[:, e], ~keep_gpu[:, e]
        if took.any():
            lo = col[took].min()
            assert lo > t - margin(t if np.isfinite(t) else lo), f"expert {e}: row below threshold"
            passing_left = left & (col > t + (margin(t) if np.isfinite(t) else 0.0))
            if passing_left.any():
                hi = col[passing_left].max()
                assert hi <= lo + margin(max(abs(hi), abs(lo))), \
                    f"expert {e}: left {hi} above taken {lo}"
        n_pass_lo = int((col > t + (margin(t) if np.isfinite(t) else 0.0)).sum())
        n_pass_hi = int((col > t - (margin(t) if np.isfinite(t) else 0.0)).sum())
        assert min(m, n_pass_lo) <= took.sum() <= min(m, n_pass_hi)
    return len(diff)


def check_batchwise(w, inp, out, m, train, thr=None):
    B, n = w.tokens, w.n_experts
    counts, keep = gpu_keep(out, B, n, m)
    ref = oracle.batchwise_forward(inp, m, train=train, noise_floor=FLOOR, threshold=thr)
    S32 = ref["H"].astype(np.float32).astype(np.float64)
    ndiff = check_column_choice(S32, keep, ref["keep"], m, thr)
    # scores and gates of the GPU's own choice
    on = oracle.batchwise_forward(inp, m, train=train, noise_floor=FLOOR, keep=keep)
    tok = to_host(out["sel_token"]).reshape(n, m)
    sc = to_host(out["sel_score"]).reshape(n, m)
    gt = to_host(out["sel_gate"]).reshape(n, m)
    got_s, ref_s, got_g, ref_g = [], [], [], []
    for e in range(n):
        lst = tok[e, :counts[e]]
        got_s.append(sc[e, :counts[e]])
        ref_s.append(on["H"][lst, e])
        got_g.append(gt[e, :counts[e]])
        ref_g.append(on["G"][lst, e])
    if counts.sum():
        serr = rel_err(np.concatenate(got_s), np.concatenate(ref_s))
        gerr = rel_err(np.concatenate(got_g), np.concatenate(ref_g))
        assert serr <= GATE_TOL, f"score error {serr}"
        assert gerr <= GATE_TOL, f"gate error {gerr}"
    y = to_host(out["y"])
    yerr = rel_err(y, on["y"])
    assert yerr <= out_tol(w.act_dtype == dg.BF16), f"y error {yerr}"
    assert np.all(y[~keep.any(axis=1)] == 0.0)
    ierr = rel_err(to_host(out["importance"]), on["importance"])
    assert ierr <= GATE_TOL, f"importance error {ierr}"
    assert np.array_equal(to_host(out["load"]), counts.astype(np.float32))
    lo = to_host(out["losses"])
    assert scalar_rel(lo[0], on["losses"][0]) <= LOSS_TOL
    assert scalar_rel(lo[1], on["losses"][1]) <= LOSS_TOL
    assert scalar_rel(lo[2], 0.1 * on["losses"][0] + 0.1 * on["losses"][1]) <= LOSS_TOL
    return {"y_err": yerr, "imp_err": ierr, "near_tie_columns": ndiff,
            "same_as_oracle": bool(np.array_equal(keep, ref["keep"]))}


def run(w, inp, m, train, thr=None):
    g = gpu_inputs(inp)
    t = None if thr is None else to_device(np.asarray(thr, np.float32))
    out = moe.moe_batchwise_forward(g["x"], g["w_gate"], g["w_noise"], g.get("eps"), g["w1"],
                                    g["w2"], m, b1=g.get("b1"), b2=g.get("b2"),
                                    gate_bias=g.get("gate_bias"), expert_threshold=t,
                                    train=train, noise_floor=FLOOR)
    torch.cuda.synchronize()
    return out


# (workload, overrides, rows per expert (None: k B / n), train, bias)
CASES = [
    ("tiny_fp32", {}, None, True, False),
    ("tiny_fp32", {"tokens": 333, "n_experts": 37, "k": 3}, None, False, True),
    ("flat_bf16_n4096", {"tokens": 1000, "n_experts": 64, "d_hidden": 256}, None, True, True),
    ("flat_bf16_n4096", {"tokens": 3000, "n_experts": 48, "d_hidden": 128}, None, False, False),
    ("flat_fp32_n32", {"tokens": 2048, "d_hidden": 128}, None, True, False),
    ("tiny_fp32", {"tokens": 5000, "n_experts": 4}, None, True, False),    # m = 2500 > 1024
    ("tiny_fp32", {"tokens": 20000}, 1000, True, False),                    # too many candidates
    ("tiny_fp32", {"tokens": 1, "n_experts": 8}, 1, False, False),         # every expert, one row
    ("flat_bf16_n4096", {"tokens": 700, "n_experts": 32, "d_hidden": 128}, 700, True, False),
    ("zipf_bf16_n256", {"tokens": 2048, "d_hidden": 128}, None, False, False),  # gate bias, 16x16
    ("zipf_bf16_n256", {"tokens": 2048, "d_hidden": 128, "gate_dtype": dg.BF16}, None, False,
     False),                                                                # gate bias, 32x32
]


def _ids(c):
    name, kw, m, train, _ = c
    return name + "".join(f"-{k}{v}" for k, v in kw.items()) + f"-m{m}-train{int(train)}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_batchwise_parity(case):
    name, kw, m, train, bias = case
    w = dg.workload(name, **kw)
    m = m or max(1, w.k * w.tokens // w.n_experts)
    announce(f"moe_batchwise_forward {w.name} {kw} m={m} train={train}")
    inp = dg.make_inputs(w, with_bias=bias)
    out = run(w, inp, m, train)
    res = check_batchwise(w, inp, out, m, train)
    if m <= w.tokens:
        assert np.all(to_host(out["counts"]) == m)  # no threshold: every expert fills up
    print(w.name, kw, m, train, res)


@pytest.mark.parametrize("quantile,m_frac", [(0.9, 1.0), (0.5, 0.1), (0.99, 0.02)])
def test_batchwise_thresholds(quantile, m_frac):
    """Inference rule: per-expert thresholds (a quantile of each column's
    scores), with no cap (m = B) or a cap below the passing count."""
    w = dg.workload("flat_fp32_n32", tokens=3000, d_hidden=128)
    m = max(1, int(m_frac * w.tokens))
    announce(f"moe_batchwise_forward thresholds q={quantile} m={m}")
    inp = dg.make_inputs(w, with_bias=True)
    H = oracle.gate(inp, 1, train=False, want_logits=True)["H"]
    thr = np.quantile(H, quantile, axis=0).astype(np.float32)
    thr[3] = np.inf   # an expert that takes nothing
    thr[5] = -np.inf  # an expert without a threshold
    out = run(w, inp, m, False, thr)
    res = check_batchwise(w, inp, out, m, False, thr)
    assert to_host(out["counts"])[3] == 0
    print(quantile, m, res)


def test_batchwise_ties_go_to_the_lower_row():
    """Repeated rows of x give exactly equal scores (train = 0); the choice
    among them must be the lower rows, as in the oracle, with no margin."""
    w = dg.workload("tiny_fp32", tokens=600, n_experts=16, k=2)
    inp = dg.make_inputs(w)
    inp["x"] = np.ascontiguousarray(np.repeat(inp["x"][:200], 3, axis=0))
    m = w.k * w.tokens // w.n_experts
    announce(f"moe_batchwise_forward ties m={m}")
    out = run(w, inp, m, False)
    counts, keep = gpu_keep(out, w.tokens, w.n_experts, m)
    ref = oracle.batchwise_forward(inp, m, train=False)
    S32 = ref["H"].astype(np.float32).astype(np.float64)
    ndiff = check_column_choice(S32, keep, ref["keep"], m, None)
    # every cut falls inside a group of three equal rows or between groups; a
    # column's choice then matches the oracle's except where the fp32 scores of
    # different groups are near ties
    for e in range(w.n_experts):
        lst = np.flatnonzero(keep[:, e])
        for r in lst:  # a taken row's lower equal twins are taken too
            g0 = r - r % 3
            assert keep[g0:r, e].all(), f"expert {e}: row {r} taken before a lower twin"
    check_batchwise(w, inp, out, m, False)
    print("ties: columns differing from the oracle", ndiff)


def test_batchwise_empty_batch():
    w = dg.workload("tiny_fp32", tokens=0)
    g = gpu_inputs(dg.make_inputs(dg.workload("tiny_fp32", tokens=4)))
    x = torch.empty((0, w.d_model), dtype=torch.float32, device="cuda")
    eps = torch.empty((0, w.n_experts), dtype=torch.float32, device="cuda")
    announce("moe_batchwise_forward empty batch")
    out = moe.moe_batchwise_forward(x, g["w_gate"], g["w_noise"], eps, g["w1"], g["w2"], 4)
    torch.cuda.synchronize()
    assert np.all(to_host(out["counts"]) == 0)
    assert np.all(to_host(out["importance"]) == 0.0)
    assert np.all(to_host(out["losses"]) == 0.0)


def test_batchwise_full_size_sampled():
    """The 65536-token, 4096-expert bf16 workload in training mode with
    m = k B / n = 64: every expert takes 64 rows; eight experts' whole
    columns are checked against the oracle's choice, and sampled rows against
    the GPU's per-expert cut (its lowest taken score) and the oracle's y."""
    w = dg.workload("flat_bf16_n4096")
    B, n = w.tokens, w.n_experts
    m = w.k * B // n
    announce(f"moe_batchwise_forward full size {w.name}: generating inputs")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    f = moe.MoeBatchwiseForward((B, w.d_model), g["w_gate"], g["w_noise"], g["w1"], g["w2"], m,
                                gate_bias=g.get("gate_bias"))
    announce("moe_batchwise_forward full size: GPU call")
    y = f(g["x"], g["eps"])
    torch.cuda.synchronize()
    counts = to_host(f.counts)
    assert np.all(counts == m)
    tok = to_host(f.sel_token).reshape(n, m)
    sc = to_host(f.sel_score).reshape(n, m)
    gate = to_host(f.sel_gate).reshape(n, m)
    assert np.all(np.diff(tok, axis=1) > 0) and tok.min() >= 0 and tok.max() < B
    rng = np.random.default_rng(9)
    experts = np.unique(np.concatenate([[0, 1, n - 1], rng.choice(n, 5, replace=False)]))
    announce("moe_batchwise_forward full size: oracle columns")
    cols = oracle.score_columns(inp, experts, train=True, noise_floor=FLOOR)
    for j, e in enumerate(experts):
        col32 = cols[:, j].astype(np.float32).astype(np.float64)
        _, kref = oracle.batchwise_select(col32[:, None], m)
        kg = np.zeros((B, 1), bool)
        kg[tok[e], 0] = True
        check_column_choice(col32[:, None], kg, kref, m, None)
        assert rel_err(sc[e], cols[tok[e], j]) <= GATE_TOL
    # sampled rows: the GPU's choice against its cut, then y and the gates
    cut = sc.min(axis=1)
    rows = np.unique(np.concatenate([[0, 1, B // 2, B - 1], rng.choice(B, 300, replace=False)]))
    announce("moe_batchwise_forward full size: oracle rows")
    H = oracle.gate(inp, 1, rows=rows, want_logits=True, noise_floor=FLOOR)["H"]
    member = {}
    for e in range(n):
        for q, t in enumerate(tok[e]):
            member.setdefault(int(t), []).append((e, q))
    yg = to_host(y)
    yerr = 0.0
    for i, t in enumerate(rows):
        taken = sorted(member.get(int(t), []))
        es = np.array([e for e, _ in taken], dtype=np.int64)
        h32 = H[i].astype(np.float32).astype(np.float64)
        clear_in = h32 > cut + margin(cut)
        clear_out = h32 < cut - margin(cut)
        mask = np.zeros(n, bool)
        mask[es] = True
        assert not (clear_in & ~mask).any(), f"row {t}: left above an expert's cut"
        assert not (clear_out & mask).any(), f"row {t}: taken below an expert's cut"
        if es.size == 0:
            assert np.all(yg[t] == 0.0)
            continue
        v = H[i, es]
        gr = np.exp(v - v.max())
        gr /= gr.sum()
        assert rel_err(np.array([gate[e, q] for e, q in taken]), gr) <= GATE_TOL
        eo = oracle.expert_pairs(inp, [int(t)] * es.size, es.astype(np.int32))
        yerr = max(yerr, rel_err(yg[t], (gr[:, None] * eo).sum(0)))
    assert yerr <= out_tol(True), f"y error {yerr}"
    print("batchwise full size", len(rows), "rows, y err", yerr)


def test_batchwise_is_deterministic():
    """Every sum over a token's experts or an expert's rows runs in a fixed
    order, so two calls give bitwise-equal outputs (the token lists are filled
    with atomics and then sorted)."""
    w = dg.workload("flat_bf16_n4096", tokens=4096, n_experts=256, d_hidden=256)
    announce("moe_batchwise_forward determinism")
    inp = dg.make_inputs(w, with_bias=True)
    g = gpu_inputs(inp)
    m = w.k * w.tokens // w.n_experts
    f = moe.MoeBatchwiseForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w1"], g["w2"],
                                m, b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"))
    y1 = f(g["x"], g["eps"]).clone()
    first = [t.clone() for t in (f.counts, f.sel_token, f.sel_score, f.sel_gate, f.importance,
                                 f.losses)]
    y2 = f(g["x"], g["eps"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for a_, b_ in zip(first, (f.counts, f.sel_token, f.sel_score, f.sel_gate, f.importance,
                              f.losses)):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("tokens,train", [(5, True), (3000, False)])
def test_batchwise_graph_replays(tokens, train):
    """moe_batchwise_forward captured in a HIP graph (no allocations, copies,
    fills or synchronizations inside): each replay, with eager calls on other
    inputs and synchronizations in between, gives exactly the eager outputs."""
    w = dg.workload("flat_bf16_n4096", tokens=tokens, n_experts=256, d_hidden=256)
    announce(f"moe_batchwise_forward graph replay tokens={tokens} train={train}")
    inp = dg.make_inputs(w)
    g = gpu_inputs(inp)
    m = max(1, w.k * w.tokens // w.n_experts)
    f = moe.MoeBatchwiseForward(tuple(g["x"].shape), g["w_gate"], g["w_noise"], g["w1"], g["w2"],
                                m, train=train)
    x, eps = g["x"].clone(), g["eps"].clone()
    y = torch.empty_like(x)
    f(x, eps, y)
    torch.cuda.synchronize()
    outs = lambda: (y, f.counts, f.sel_token, f.sel_gate, f.importance, f.losses)  # noqa: E731
    ref = [t.clone() for t in outs()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(x, eps, y)
    other_x, other_eps = torch.flip(x, [0]).contiguous(), torch.flip(eps, [0]).contiguous()
    for _ in range(3):
        f(other_x, other_eps)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(ref, outs()):
            assert torch.equal(a_, b_)
