"""Pins of the oracle against what the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: a
worked example printed on the pages (fixtures in tests/golden/, each with its
citation), a closed form, an invariant the pages state, a special case that
reduces to a textbook or library routine, brute force on a tiny input, or a
Monte Carlo estimate of the probability eq 8 defines. The constructions are
chosen so that a plausible slip (a transposed weight, a dropped bias, a wrong
sign, a wrong threshold, sample instead of population variance) fails one of
them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import norm

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def inputs(x, wg, wn, eps=None, bg=None, w1=None, w2=None, b1=None, b2=None):
    inp = {"x": f32(x), "w_gate": f32(wg), "w_noise": f32(wn)}
    if eps is not None:
        inp["eps"] = f32(eps)
    if bg is not None:
        inp["gate_bias"] = f32(bg)
    for key, v in (("w1", w1), ("w2", w2), ("b1", b1), ("b2", b2)):
        if v is not None:
            inp[key] = f32(v)
    return inp


def identity_gate(H):
    """x = H, W_g = I, W_noise = 0: the clean logits are the given values."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float32))
    n = H.shape[1]
    return inputs(H, np.eye(n), np.zeros((n, n)))


def const_experts(n, d, h=3, scale=1.0, seed=0):
    """Experts with E_i(x) = b2_i for every x (W1 = W2 = 0)."""
    rng = np.random.default_rng(seed)
    return {"w1": np.zeros((n, h, d), np.float32), "w2": np.zeros((n, d, h), np.float32),
            "b1": f32(rng.normal(size=(n, h))), "b2": f32(scale * rng.normal(size=(n, d)))}


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def test_gating_worked_example():
    g = golden("gating_example.json")
    out = oracle.gate(identity_gate(g["logits"]), g["k"], train=False)
    assert out["topk_idx"][0].tolist() == g["expected_topk"]
    gates = out["topk_gate"][0]
    for got, printed in zip(gates, g["printed_gates"]):
        assert abs(got - printed) <= g["printed_precision"]
    # the first expert left out is expert 1 of the page, which missed by 0.1
    vk, vk1 = out["thresh"][0]
    assert vk1 == pytest.approx(g["logits"][g["expected_next"]], abs=1e-6)
    assert vk - vk1 == pytest.approx(g["printed_margin"], abs=1e-6)
    # survivors' softmax: the gate ratio is e^(1.7 - 1.5)
    l = np.float32(g["logits"]).astype(np.float64)
    assert gates[0] / gates[1] == pytest.approx(math.exp(l[3] - l[4]), rel=1e-12)


def test_importance_worked_example():
    """k = n = 4, no noise: every token's gate row is the dense softmax; rows
    chosen so each one is (0.45, 0.3, 0.15, 0.1) and the batch of 8 sums to the
    page's importances."""
    g = golden("importance_example.json")
    n, B = g["n"], g["batch"]
    row = np.array(g["importance"]) / B
    logits = np.log(row) + 0.25
    inp = identity_gate(np.tile(logits, (B, 1)))
    inp.update(const_experts(n, n))
    out = oracle.forward(inp, n, train=False, w_importance=g["w_importance"], w_load=0.0)
    assert np.allclose(out["importance"], g["importance"], atol=1e-6)
    assert out["importance"].mean() == pytest.approx(g["printed_mean"], abs=1e-6)
    assert out["losses"][0] == pytest.approx(g["printed_cv2"], abs=g["printed_precision"])
    assert out["losses"][0] == pytest.approx(g["printed_mean_sq_dev"] / g["printed_mean"] ** 2, rel=1e-5)
    assert out["losses"][2] == pytest.approx(g["printed_loss"], abs=g["printed_precision"])
    assert oracle.cv2(g["importance"]) == pytest.approx(0.30, rel=1e-12)


def _load_case(clean, u, eps, k, floor=0.0):
    """x = [clean | u], W_g = [I 0], W_noise = [0 I]: clean logits and noise
    pre-activations are given directly."""
    clean, u, eps = (np.asarray(v, dtype=np.float64) for v in (clean, u, eps))
    n = clean.size
    x = np.concatenate([clean, u])[None, :]
    wg = np.hstack([np.eye(n), np.zeros((n, n))])
    wn = np.hstack([np.zeros((n, n)), np.eye(n)])
    return inputs(x, wg, wn, eps=eps[None, :]), floor


def test_load_worked_example():
    g = golden("load_example.json")
    sigma = g["noise_std"]
    u = math.log(math.expm1(sigma))  # Softplus(u) = sigma
    # expert 0: clean 1.0, sigma 0.5, not selected; expert 1 holds the top-1 logit 1.3
    inp, floor = _load_case([g["clean_logit"], g["threshold"], 0.2], [u, 0.0, 0.0], [0.0, 0.0, 0.0], 1)
    gate = oracle.gate(inp, 1, noise_floor=floor, want_logits=True)
    assert gate["topk_idx"][0, 0] == 1
    assert gate["sigma"][0, 0] == pytest.approx(sigma, rel=1e-6)
    load = oracle.load(inp, 1, noise_floor=floor)
    assert load[0] == pytest.approx(g["printed_P"], abs=g["printed_precision"])
    assert load[0] == pytest.approx(norm.cdf(g["printed_z"]), abs=1e-6)


def test_initial_noise_std():
    g = golden("initial_noise_std.json")
    assert oracle.softplus(0.0) == pytest.approx(g["softplus_at_zero_printed"], abs=g["printed_precision"])
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)


def test_layer_size_arithmetic():
    """Shape sanity of the pages' 512-1024-512 experts (weights only, no biases)."""
    g = golden("layer_size.json")
    per_expert = g["d_hidden"] * (g["d_model"] + g["d_model"])
    assert round(per_expert / 1e6) == 1
    assert round(per_expert * g["experts"] / 1e9, 1) == 4.3
    assert round(per_expert * g["k"] / 1e6, 1) == 4.2
    # the oracle's expert touches exactly those weights: with d = 512, h = 1024
    # a single nonzero input feeds every hidden unit once
    d, h = 8, 16
    rng = np.random.default_rng(0)
    w1 = rng.uniform(0.5, 1.0, (1, h, d))
    w2 = rng.uniform(0.5, 1.0, (1, d, h))
    x = np.zeros((1, d)); x[0, 3] = 1.0
    out = oracle.expert_pairs({"x": f32(x), "w1": f32(w1), "w2": f32(w2)}, [0], [0])
    assert np.allclose(out[0], f32(w2)[0].astype(np.float64) @ f32(w1)[0, :, 3].astype(np.float64))


# --------------------------------------------------------------------------
# Logits: closed forms that catch transposed weights, bias and noise slips
# --------------------------------------------------------------------------

def test_logits_closed_form_selection_matrices():
    rng = np.random.default_rng(1)
    B, d, n = 5, 7, 5
    x = rng.normal(size=(B, d)).astype(np.float32)
    pc = [(3 * i + 1) % d for i in range(n)]
    pu = [(2 * i + 5) % d for i in range(n)]
    wg = np.zeros((n, d)); wn = np.zeros((n, d))
    for i in range(n):
        wg[i, pc[i]] = 1.0
        wn[i, pu[i]] = 1.0
    bg = rng.normal(size=n)
    eps = rng.normal(size=(B, n))
    floor = 0.01
    out = oracle.gate(inputs(x, wg, wn, eps=eps, bg=bg), 2, noise_floor=floor, want_logits=True)
    xd = x.astype(np.float64)
    clean = xd[:, pc] + f32(bg).astype(np.float64)
    u = xd[:, pu]
    sigma = np.log1p(np.exp(u)) + floor
    assert np.allclose(out["clean"], clean, rtol=0, atol=1e-12)
    assert np.allclose(out["sigma"], sigma, rtol=1e-12, atol=0)
    assert np.allclose(out["H"], clean + f32(eps).astype(np.float64) * sigma, rtol=0, atol=1e-12)


def test_softplus_closed_forms():
    assert oracle.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=1e-14)
    assert oracle.softplus(40.0) == pytest.approx(40.0 + math.exp(-40.0), rel=1e-15)
    assert oracle.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert oracle.softplus(800.0) == 800.0  # no overflow


def test_inference_mode_has_no_noise():
    rng = np.random.default_rng(2)
    B, d, n = 6, 9, 6
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)),
                 eps=rng.normal(size=(B, n)) * 50.0)
    out = oracle.gate(inp, 3, train=False, want_logits=True)
    assert np.array_equal(out["H"], out["clean"])
    # the selection is then the top 3 clean logits
    assert np.array_equal(out["topk_idx"], np.argsort(-out["clean"], axis=1, kind="stable")[:, :3])


def test_zero_init_routes_by_noise_alone():
    """W_g = W_noise = 0: every clean logit is 0, the noise std is ln 2 + floor,
    and the top k are the k largest noise draws."""
    rng = np.random.default_rng(3)
    B, d, n, k, floor = 64, 5, 12, 3, 0.01
    eps = rng.normal(size=(B, n)).astype(np.float32)
    inp = inputs(rng.normal(size=(B, d)), np.zeros((n, d)), np.zeros((n, d)), eps=eps)
    out = oracle.gate(inp, k, noise_floor=floor, want_logits=True)
    assert np.all(out["clean"] == 0.0)
    assert np.allclose(out["sigma"], math.log(2.0) + floor, rtol=1e-15)
    assert np.array_equal(out["topk_idx"], np.argsort(-eps, axis=1, kind="stable")[:, :k])


def test_zero_init_load_closed_form():
    """Zero init, floor 0: P_in = Phi(-eps_(k+1)), P_out = Phi(-eps_(k)) where
    eps_(j) is the row's j-th largest draw."""
    rng = np.random.default_rng(4)
    B, d, n, k = 40, 3, 7, 2
    eps = rng.normal(size=(B, n)).astype(np.float64)
    inp = inputs(rng.normal(size=(B, d)), np.zeros((n, d)), np.zeros((n, d)), eps=eps)
    load = oracle.load(inp, k, noise_floor=0.0)
    e = f32(eps).astype(np.float64)
    srt = -np.sort(-e, axis=1)
    rank = np.argsort(np.argsort(-e, axis=1, kind="stable"), axis=1)
    P = np.where(rank < k, norm.cdf(-srt[:, [k]]), norm.cdf(-srt[:, [k - 1]]))
    assert np.allclose(load, P.sum(0), rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Top-k: brute force over all k-subsets, ties, k = 1
# --------------------------------------------------------------------------

def brute_force_topk(h, k):
    best = None
    for s in itertools.combinations(range(len(h)), k):
        key = (sum(h[i] for i in s), tuple(-i for i in s))
        if best is None or key > best[0]:
            best = (key, s)
    return set(best[1])


@pytest.mark.parametrize("n,k", [(2, 1), (5, 2), (8, 3), (10, 4), (7, 7), (9, 8)])
def test_topk_brute_force(n, k):
    rng = np.random.default_rng(10 * n + k)
    H = rng.normal(size=(30, n)).astype(np.float32)
    out = oracle.gate(identity_gate(H), k, train=False)
    for t in range(H.shape[0]):
        row = [float(v) for v in H[t]]
        sel = out["topk_idx"][t].tolist()
        assert set(sel) == brute_force_topk(row, k)
        assert all(row[sel[j]] >= row[sel[j + 1]] for j in range(k - 1))
        others = [row[i] for i in range(n) if i not in sel]
        assert out["thresh"][t, 0] == pytest.approx(row[sel[-1]])
        if k < n:
            assert out["thresh"][t, 1] == pytest.approx(max(others))
        else:
            assert out["thresh"][t, 1] == -math.inf


def test_topk_ties_go_to_lower_index():
    out = oracle.gate(identity_gate([[1.0, 2.0, 2.0, 2.0, 0.0], [3.0, 3.0, 3.0, 3.0, 3.0]]), 2,
                      train=False)
    assert out["topk_idx"].tolist() == [[1, 2], [0, 1]]
    assert out["topk_gate"][0].tolist() == [0.5, 0.5]
    assert out["thresh"][0].tolist() == [2.0, 2.0]


def test_k1_gate_is_exactly_one():
    rng = np.random.default_rng(5)
    out = oracle.gate(identity_gate(rng.normal(size=(50, 6))), 1, train=False)
    assert np.all(out["topk_gate"] == 1.0)


def test_gate_rows_are_sparse_and_normalised():
    rng = np.random.default_rng(6)
    B, d, n, k = 200, 10, 16, 4
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)) / 3, rng.normal(size=(n, d)) / 3,
                 eps=rng.normal(size=(B, n)))
    out = oracle.gate(inp, k)
    g = out["topk_gate"]
    assert np.all(g > 0) and np.all(g <= 1)
    assert np.allclose(g.sum(1), 1.0, atol=1e-12)
    assert all(len(set(r)) == k for r in out["topk_idx"].tolist())
    assert np.all(np.diff(g, axis=1) <= 0)  # rank order = descending gate


# --------------------------------------------------------------------------
# Experts and the weighted sum (eq 1)
# --------------------------------------------------------------------------

def test_expert_closed_form_selection_matrices():
    """d = 6, h = 4 (not square): W1 picks inputs, W2 picks hidden units, so
    E(x)_c = ReLU(x[pi[s[c]]] + b1[s[c]]) + b2[c]."""
    rng = np.random.default_rng(7)
    d, h, T = 6, 4, 9
    pi = [4, 0, 5, 2]          # hidden j reads input pi[j]
    s = [3, 1, 0, 2, 1, 3]     # output c reads hidden s[c]
    w1 = np.zeros((1, h, d)); w2 = np.zeros((1, d, h))
    for j in range(h):
        w1[0, j, pi[j]] = 1.0
    for c in range(d):
        w2[0, c, s[c]] = 1.0
    b1 = rng.normal(size=(1, h)); b2 = rng.normal(size=(1, d))
    x = rng.normal(size=(T, d))
    inp = {"x": f32(x), "w1": f32(w1), "w2": f32(w2), "b1": f32(b1), "b2": f32(b2)}
    out = oracle.expert_pairs(inp, list(range(T)), [0] * T)
    xd, b1d, b2d = (f32(v).astype(np.float64) for v in (x, b1, b2))
    hid = np.maximum(xd[:, pi] + b1d[0], 0.0)
    assert np.allclose(out, hid[:, s] + b2d[0], rtol=0, atol=1e-14)
    assert np.any(xd[:, pi] + b1d[0] < 0)  # the ReLU was exercised


def test_expert_linear_regime_matches_matmul():
    """Non-negative inputs and W1, b1: the ReLU never clips and the expert is the
    affine map W2 (W1 x + b1) + b2, compared with numpy's matmul."""
    rng = np.random.default_rng(8)
    n, d, h, T = 3, 5, 7, 6
    w1 = f32(rng.uniform(0, 1, (n, h, d))); b1 = f32(rng.uniform(0, 1, (n, h)))
    w2 = f32(rng.normal(size=(n, d, h))); b2 = f32(rng.normal(size=(n, d)))
    x = f32(rng.uniform(0, 1, (T, d)))
    inp = {"x": x, "w1": w1, "w2": w2, "b1": b1, "b2": b2}
    toks = np.repeat(np.arange(T), n)
    exps = np.tile(np.arange(n), T)
    out = oracle.expert_pairs(inp, toks, exps)
    D = lambda a: a.astype(np.float64)
    for q, (t, e) in enumerate(zip(toks, exps)):
        ref = D(w2[e]) @ (D(w1[e]) @ D(x[t]) + D(b1[e])) + D(b2[e])
        assert np.allclose(out[q], ref, rtol=1e-13, atol=1e-13)


def test_combine_with_constant_experts():
    """E_i(x) = b2_i: y_t = sum_j g_tj b2[S_tj], the gate-weighted sum of eq 1."""
    rng = np.random.default_rng(9)
    B, d, n, k = 50, 6, 9, 3
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)) / 4,
                 eps=rng.normal(size=(B, n)))
    inp.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.forward(inp, k)
    Gd = np.zeros((B, n))
    np.put_along_axis(Gd, out["topk_idx"], out["topk_gate"], axis=1)
    assert np.allclose(out["y"], Gd @ inp["b2"].astype(np.float64), rtol=0, atol=1e-13)
    assert np.allclose(oracle.y_rows(inp, k, rows=[3, 17, 49]), out["y"][[3, 17, 49]], atol=0)


def test_single_expert_is_the_mlp():
    """n = k = 1: the layer is its one expert (gate exactly 1)."""
    rng = np.random.default_rng(10)
    B, d, h = 12, 5, 4
    w1 = f32(rng.normal(size=(1, h, d))); w2 = f32(rng.normal(size=(1, d, h)))
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(1, d)), rng.normal(size=(1, d)),
                 eps=rng.normal(size=(B, 1)), w1=w1, w2=w2)
    out = oracle.forward(inp, 1)
    ref = oracle.expert_pairs(inp, np.arange(B), np.zeros(B, np.int32))
    assert np.array_equal(out["y"], ref)
    assert np.all(out["topk_gate"] == 1.0)


def test_dense_softmax_moe_when_k_equals_n():
    """k = n without noise reduces to the dense softmax gate of eq 2: with
    constant experts, y = softmax(x W_g) B2 (scipy's softmax, numpy's matmul)."""
    rng = np.random.default_rng(11)
    B, d, n = 40, 6, 5
    x = f32(rng.normal(size=(B, d))); wg = f32(rng.normal(size=(n, d)))
    inp = inputs(x, wg, np.zeros((n, d)))
    inp.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.forward(inp, n, train=False)
    dense = sp_softmax(x.astype(np.float64) @ wg.astype(np.float64).T, axis=1)
    assert np.allclose(out["y"], dense @ inp["b2"].astype(np.float64), rtol=1e-10, atol=1e-12)
    assert np.allclose(out["importance"], dense.sum(0), rtol=1e-10)
    assert np.allclose(out["load"], B)  # every expert is always kept


# --------------------------------------------------------------------------
# Load: Monte Carlo of eq 8, k = n, inference mode
# --------------------------------------------------------------------------

def test_load_probability_matches_monte_carlo():
    """Eq 8 defines P(x, i) as the probability that expert i stays in the top k
    when only its own noise draw is redrawn. Estimate it by redrawing and
    ranking with numpy, and compare with the oracle's eq 9 for every expert."""
    rng = np.random.default_rng(12)
    d, n, k = 6, 10, 3
    x = rng.normal(size=(1, d)); wg = rng.normal(size=(n, d)) / 2; wn = rng.normal(size=(n, d)) / 2
    eps = rng.normal(size=(1, n))
    inp = inputs(x, wg, wn, eps=eps)
    g = oracle.gate(inp, k, want_logits=True)
    clean, sigma, H = g["clean"][0], g["sigma"][0], g["H"][0]
    N = 200_000
    for i in range(n):
        trials = np.tile(H, (N, 1))
        trials[:, i] = clean[i] + rng.standard_normal(N) * sigma[i]
        # expert i stays in the top k iff fewer than k others beat it
        beats = (np.delete(trials, i, axis=1) > trials[:, [i]]).sum(1)
        p_mc = np.mean(beats < k)
        single = dict(inp)
        p = oracle.load(single, k)[i]
        tol = 5 * math.sqrt(max(p * (1 - p), 1e-6) / N) + 1e-9
        assert abs(p - p_mc) <= tol, (i, p, p_mc)


def test_load_in_and_out_thresholds():
    """The selected expert is measured against the (k+1)-th logit, the others
    against the k-th (eq 8: the k-th largest of the other logits)."""
    u = math.log(math.expm1(0.5))
    inp, floor = _load_case([2.0, 1.3, 0.2], [u, u, u], [0.0, 0.0, 0.0], 1)
    load = oracle.load(inp, 1, noise_floor=floor)
    assert load[0] == pytest.approx(norm.cdf((2.0 - 1.3) / 0.5), abs=1e-6)  # in: vs (k+1)-th = 1.3
    assert load[1] == pytest.approx(norm.cdf((1.3 - 2.0) / 0.5), abs=1e-6)  # out: vs k-th = 2.0
    assert load[2] == pytest.approx(norm.cdf((0.2 - 2.0) / 0.5), abs=1e-6)


def test_load_k_equals_n_is_batch_size():
    rng = np.random.default_rng(13)
    B, d, n = 33, 4, 5
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)),
                 eps=rng.normal(size=(B, n)))
    assert np.array_equal(oracle.load(inp, n), np.full(n, float(B)))


def test_inference_load_is_the_hard_count():
    rng = np.random.default_rng(14)
    B, d, n, k = 100, 5, 8, 2
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)))
    load = oracle.load(inp, k, train=False)
    g = oracle.gate(inp, k, train=False)
    assert np.array_equal(load, np.bincount(g["topk_idx"].ravel(), minlength=n).astype(float))


# --------------------------------------------------------------------------
# Importance, CV^2 and the losses
# --------------------------------------------------------------------------

def test_cv2_closed_forms():
    v = np.array([3.0, 1.0])
    assert oracle.cv2(v) == pytest.approx(((3 - 1) / (3 + 1)) ** 2, rel=1e-15)
    rng = np.random.default_rng(15)
    w = rng.uniform(0.1, 5, 37)
    assert oracle.cv2(2 * w) == pytest.approx(oracle.cv2(w), rel=1e-13)
    assert oracle.cv2(np.full(9, 4.2)) == pytest.approx(0.0, abs=1e-28)
    assert oracle.cv2([5.0]) == 0.0
    assert oracle.cv2([0.0, 0.0]) == 0.0
    assert oracle.cv2(w) == pytest.approx(np.var(w) / np.mean(w) ** 2, rel=1e-12)


def test_importance_sums_to_batch_and_k1_is_counts():
    rng = np.random.default_rng(16)
    B, d, n = 120, 6, 7
    base = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)),
                  eps=rng.normal(size=(B, n)))
    base.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.forward(base, 3)
    assert out["importance"].sum() == pytest.approx(B, rel=1e-12)
    out1 = oracle.forward(base, 1)
    assert np.array_equal(out1["importance"], np.bincount(out1["topk_idx"][:, 0], minlength=n).astype(float))


def test_losses_combine_both_cv2():
    rng = np.random.default_rng(17)
    B, d, n, k = 64, 5, 6, 2
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)))
    inp.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.forward(inp, k, train=False, w_importance=0.3, w_load=0.7)
    counts = np.bincount(out["topk_idx"].ravel(), minlength=n).astype(float)
    assert np.array_equal(out["load"], counts)
    assert out["losses"][1] == pytest.approx(np.var(counts) / counts.mean() ** 2, rel=1e-12)
    assert out["losses"][2] == pytest.approx(0.3 * out["losses"][0] + 0.7 * out["losses"][1], rel=1e-14)


# --------------------------------------------------------------------------
# Routing: the per-expert row sets, made stable
# --------------------------------------------------------------------------

def test_route_is_the_stable_sort_by_expert():
    rng = np.random.default_rng(18)
    B, n, k = 300, 11, 3
    idx = np.stack([rng.permutation(n)[:k] for _ in range(B)]).astype(np.int32)
    gates = rng.uniform(size=(B, k))
    r = oracle.route(idx, gates, n)
    order = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(r["perm_token"], order // k)
    assert np.array_equal(r["perm_gate"], gates.ravel()[order])
    assert np.array_equal(r["counts"], np.bincount(idx.ravel(), minlength=n))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    inv = np.empty(B * k, np.int64); inv[order] = np.arange(B * k)
    assert np.array_equal(r["slot_pos"], inv)
    assert np.allclose(r["importance"], np.bincount(idx.ravel(), weights=gates.ravel(), minlength=n),
                       rtol=1e-13)


def test_route_handles_empty_experts():
    idx = np.array([[0, 3], [3, 0], [0, 3]], np.int32)
    r = oracle.route(idx, np.full((3, 2), 0.5), 6)
    assert r["counts"].tolist() == [3, 0, 0, 3, 0, 0]
    assert r["offsets"].tolist() == [0, 3, 3, 3, 6, 6, 6]
    assert r["perm_token"].tolist() == [0, 1, 2, 0, 1, 2]


def _exact_logits_input(h, d=64):
    """x = e_0 and W_g row i = h_i e_0, so that clean_i = h_i exactly (fp32)."""
    n = len(h)
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 1.0
    wg = np.zeros((n, d), np.float32)
    wg[:, 0] = h
    return {"x": x, "w_gate": wg, "w_noise": np.zeros((n, d), np.float32),
            "eps": np.zeros((1, n), np.float32)}


def test_switch_order_hand_example():
    """Logits 0, ln 2, ln 3: the softmax over all three is 1/6, 2/6, 3/6. The
    Switch order keeps the largest with gate 1/2 (k = 1) or 1/2, 1/3 (k = 2);
    the pages' order renormalises the kept: 1 (k = 1), 3/5, 2/5 (k = 2)."""
    h = np.array([0.0, np.log(2.0), np.log(3.0)], np.float32)
    inp = _exact_logits_input(h)
    for k, switch, kept in ((1, [0.5], [1.0]), (2, [1 / 2, 1 / 3], [3 / 5, 2 / 5])):
        s = oracle.gate(inp, k, train=False, gate_order=1)
        p = oracle.gate(inp, k, train=False, gate_order=0)
        assert s["topk_idx"].tolist() == p["topk_idx"].tolist() == [[2, 1][:k]]
        assert np.allclose(s["topk_gate"][0], switch, rtol=1e-6)
        assert np.allclose(p["topk_gate"][0], kept, rtol=1e-6)


def test_switch_order_k_equals_n_is_the_dense_softmax():
    rng = np.random.default_rng(21)
    inp = {"x": rng.normal(size=(40, 64)).astype(np.float32),
           "w_gate": (rng.normal(size=(6, 64)) / 8).astype(np.float32),
           "w_noise": (rng.normal(size=(6, 64)) / 8).astype(np.float32),
           "eps": rng.normal(size=(40, 6)).astype(np.float32)}
    a = oracle.gate(inp, 6, train=True, gate_order=1)
    b = oracle.gate(inp, 6, train=True, gate_order=0)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert np.allclose(a["topk_gate"], b["topk_gate"], rtol=1e-12)
    c = oracle.gate(inp, 2, train=True, gate_order=1)
    assert np.all(c["topk_gate"].sum(1) < 1.0) and np.all(c["topk_gate"] > 0)


def test_route_capacity_hand_example():
    """Fixed expert capacity (the GShard variant named beside the layer): each
    expert serves its first C pairs in (token, slot) order. Worked by hand for
    B = 5, k = 2, n = 3, C = 2: expert 0 is picked by (0,0) (1,0) (2,1) (3,0)
    (4,1) at positions 0-4 and serves the first two; expert 1 by (0,1) (2,0)
    (3,1) at 5-7, serving two; expert 2 by (1,1) (4,0) at 8-9, serving both."""
    idx = np.array([[0, 1], [0, 2], [1, 0], [0, 1], [2, 0]], np.int32)
    gates = np.full((5, 2), 0.5)
    full = oracle.route(idx, gates, 3)
    assert full["slot_pos"].tolist() == [0, 5, 1, 8, 6, 2, 3, 7, 9, 4]
    capped = oracle.route(idx, gates, 3, capacity=2)
    assert capped["slot_pos"].tolist() == [0, 5, 1, 8, 6, -1, -1, -1, 9, -1]
    # the demand is unchanged: segments, counts and Importance list every pair
    for key in ("counts", "offsets", "perm_token", "perm_gate", "importance"):
        assert np.array_equal(full[key], capped[key])


def test_route_capacity_properties():
    rng = np.random.default_rng(19)
    B, n, k = 400, 13, 3
    idx = np.stack([rng.permutation(n)[:k] for _ in range(B)]).astype(np.int32)
    gates = rng.uniform(size=(B, k))
    full = oracle.route(idx, gates, n)
    for cap in (1, 5, 50, int(full["counts"].max())):
        r = oracle.route(idx, gates, n, capacity=cap)
        kept = r["slot_pos"] >= 0
        served = np.bincount(idx.ravel()[kept], minlength=n)
        assert np.array_equal(served, np.minimum(full["counts"], cap))
        # a served pair keeps its position; it precedes every dropped pair of its expert
        assert np.array_equal(r["slot_pos"][kept], full["slot_pos"][kept])
        for e in range(n):
            pe = np.flatnonzero(idx.ravel() == e)
            assert kept[pe].tolist() == sorted(kept[pe].tolist(), reverse=True)
    r = oracle.route(idx, gates, n, capacity=int(full["counts"].max()))
    assert np.array_equal(r["slot_pos"], full["slot_pos"])


# --------------------------------------------------------------------------
# bf16 inputs are read by exact widening
# --------------------------------------------------------------------------

def test_bf16_inputs_widen_exactly():
    import datagen as dg
    rng = np.random.default_rng(19)
    B, d, n = 10, 8, 6
    x = f32(rng.normal(size=(B, d)))
    xb = dg.f32_to_bf16(x)
    wg = f32(rng.normal(size=(n, d)))
    a = oracle.gate({"x": xb, "w_gate": dg.f32_to_bf16(wg), "w_noise": dg.f32_to_bf16(wg)}, 2,
                    train=False, want_logits=True)
    b = oracle.gate({"x": dg.bf16_to_f32(xb), "w_gate": dg.bf16_to_f32(dg.f32_to_bf16(wg)),
                     "w_noise": dg.bf16_to_f32(dg.f32_to_bf16(wg))}, 2, train=False, want_logits=True)
    assert np.array_equal(a["clean"], b["clean"])
