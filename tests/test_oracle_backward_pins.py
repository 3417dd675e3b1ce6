"""Pins of the oracle's backward pass against what the pages and the
mathematics fix (no GPU).

Reading (the pages' paragraph on which parameters receive gradients, in the
explainer's "Implementation notes"): the experts get gradient only from their
routed rows, scaled by their gates; W_g through the softmax over the kept
logits (task and Importance losses) and through the numerator of eq 9 (Load
loss, also for experts that were not kept); W_noise through the noise term of
the kept logits and through the denominator of eq 9; the selection and eq 9's
thresholds pass none.

* worked numbers of [MoE-explainer]: a kept gate's derivative by its own
  logit G(1 - G) = 0.55 x 0.45 = 0.25 ("Noisy top-k gating", k >= 2); the
  CV^2 gradient +0.2 / -0.15 for the importances (3.6, 2.4, 1.2, 0.8) with
  the mean fixed ("Why experts collapse..."); dP/dc = phi(-0.6) / 0.5 = 0.67
  ("A differentiable count of examples");
* the whole backward against central differences of the oracle's forward
  objective with the selection and the thresholds held fixed (every input
  and parameter element, training and inference, with biases);
* k = 1: the task loss sends nothing to W_g (the softmax of one kept logit is
  exactly 1);
* one expert, k = 1, no noise, no losses: the textbook two-layer ReLU network
  backward written with NumPy matrix products.
"""
import math

import numpy as np
import pytest
from scipy.stats import norm

import datagen as dg
import oracle

FLOOR = 1e-2


def test_kept_gate_derivative_worked_example():
    """Kept logits 1.7 and 1.5 give gates 0.55 / 0.45; the derivative of a gate
    by its own logit is G(1 - G), printed as 0.25."""
    H = np.array([1.7, 1.5])
    g = np.exp(H - H.max())
    g /= g.sum()
    dH = oracle.kept_softmax_grad(g, [1.0, 0.0])  # d gate_1 / d H
    assert dH[0] == pytest.approx(g[0] * (1 - g[0]), rel=1e-14)
    assert round(dH[0], 2) == 0.25
    assert dH[1] == pytest.approx(-g[0] * g[1], rel=1e-14)
    # the gates sum to 1 whatever the logits: a common gradient on every gate
    # reaches no logit
    np.testing.assert_allclose(oracle.kept_softmax_grad(g, [3.0, 3.0]), 0.0, atol=1e-15)


def test_cv2_gradient_worked_example():
    """Importances (3.6, 2.4, 1.2, 0.8): with the mean fixed the gradient of
    CV^2 is 2 (v_i - mean) / (n mean^2) = +0.2 for the first, -0.15 for the
    last; the unconstrained gradient adds the common -V / (n/2 mean^3) term."""
    v = np.array([3.6, 2.4, 1.2, 0.8])
    g = oracle.cv2_grad(v)
    np.testing.assert_allclose(g, [0.125, -0.025, -0.175, -0.225], rtol=1e-13)
    fixed_mean = g - g.mean()
    assert fixed_mean[0] == pytest.approx(0.2, rel=1e-12)
    assert fixed_mean[-1] == pytest.approx(-0.15, rel=1e-12)
    # against central differences of CV^2 itself (pinned by its worked value 0.30)
    h = 1e-6
    for i in range(4):
        e = np.zeros(4)
        e[i] = h
        fd = (oracle.cv2(v + e) - oracle.cv2(v - e)) / (2 * h)
        assert g[i] == pytest.approx(fd, rel=1e-7, abs=1e-10)
    assert np.all(oracle.cv2_grad([5.0]) == 0.0) and np.all(oracle.cv2_grad([0.0, 0.0]) == 0.0)


def test_load_probability_derivative_worked_example():
    """Clean logit 1.0, threshold 1.3, noise scale 0.5: dP/dc = phi(-0.6) / 0.5
    = 0.67; dP/dsigma against a library normal CDF's central differences."""
    dc, ds = oracle.p_eq9_grad(1.0, 1.3, 0.5)
    assert dc == pytest.approx(norm.pdf(-0.6) / 0.5, rel=1e-13)
    assert round(dc, 2) == 0.67
    h = 1e-6
    fd = (norm.cdf((1.0 - 1.3) / (0.5 + h)) - norm.cdf((1.0 - 1.3) / (0.5 - h))) / (2 * h)
    assert ds == pytest.approx(fd, rel=1e-7)
    assert oracle.p_eq9_grad(1.0, -math.inf, 0.5) == (0.0, 0.0)  # k == n: P = 1


def small_case(seed, n=6, k=2, B=7, d=8, h=16, bias=True):
    w = dg.workload("tiny_fp32", seed=seed, tokens=B, d_model=d, d_hidden=h, n_experts=n, k=k,
                    noise_scale=1.0)
    inp = dg.make_inputs(w, with_bias=bias)
    if bias:
        inp["gate_bias"] = (0.3 * dg.normal(seed, 99, 0, n)).astype(np.float32)
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((B, d))
    return w, inp, dy


PARAMS = ["x", "w_gate", "w_noise", "gate_bias", "w1", "b1", "w2", "b2"]
GRAD = {"x": "dx", "w_gate": "dw_gate", "w_noise": "dw_noise", "gate_bias": "dgate_bias",
        "w1": "dw1", "b1": "db1", "w2": "dw2", "b2": "db2"}


@pytest.mark.parametrize("train", [True, False])
@pytest.mark.parametrize("seed,n,k", [(101, 6, 2), (102, 5, 3), (103, 4, 4)])
def test_backward_matches_central_differences(train, seed, n, k):
    """Every gradient element against (J(p + s) - J(p - s)) / 2s of the
    forward objective, selection and thresholds fixed to the oracle's own.
    The step s = 2^-12 is exact on the fp32 inputs; the chosen data keeps
    every hidden pre-activation away from ReLU's kink."""
    w, inp, dy = small_case(seed, n=n, k=k)
    aux, wi, wl = 0.7, 0.3, 0.2
    ref = oracle.gate(inp, k, train=train, noise_floor=FLOOR)
    sel, thr = ref["topk_idx"], ref["thresh"]
    # the kink: |pre-activation| of every hidden unit of every kept pair
    x64 = inp["x"].astype(np.float64)
    pre = np.einsum("td,ehd->teh", x64, inp["w1"].astype(np.float64)) + inp["b1"][None]
    kept_pre = np.take_along_axis(pre, sel[:, :, None].astype(np.int64), 1)
    # a step moves a pre-activation by at most ~1e-3 (|x|, |W1| < 4; s = 2.4e-4)
    assert np.abs(kept_pre).min() > 0.005, "data too close to a ReLU kink"
    grads = oracle.backward(inp, k, dy, aux_scale=aux, train=train, noise_floor=FLOOR,
                            w_importance=wi, w_load=wl, force_idx=sel)

    def J(p):
        return oracle.objective(p, k, dy, sel, thr, aux_scale=aux, train=train, noise_floor=FLOOR,
                                w_importance=wi, w_load=wl)

    s = 2.0 ** -12
    worst = 0.0
    for name in PARAMS:
        if name == "w_noise" and not train:
            assert np.all(grads["dw_noise"] == 0.0)
            continue
        a = inp[name]
        g = grads[GRAD[name]]
        fd = np.empty(a.size)
        for i in range(a.size):
            p = dict(inp)
            ap = a.copy().ravel()
            ap[i] += s
            p[name] = ap.reshape(a.shape).astype(np.float32)
            jp = J(p)
            ap[i] -= 2 * s
            p[name] = ap.reshape(a.shape).astype(np.float32)
            fd[i] = (jp - J(p)) / (2 * s)
        scale = max(np.abs(fd).max(), 1e-3)
        err = np.abs(g.ravel() - fd).max() / scale
        worst = max(worst, err)
        assert err <= 2e-5, f"{name}: max |analytic - FD| / max|FD| = {err}"
    print("worst", worst)


def test_k1_task_loss_sends_nothing_to_the_gate():
    """k = 1 without noise and without the losses: the single kept gate is
    exactly 1 whatever its logit, so W_g and the gate bias get exactly 0."""
    w, inp, dy = small_case(21, n=5, k=1)
    gr = oracle.backward(inp, 1, dy, aux_scale=1.0, train=False, w_importance=0.0, w_load=0.0)
    assert np.all(gr["dw_gate"] == 0.0) and np.all(gr["dgate_bias"] == 0.0)
    # with the Importance loss on, k = 1 still gives 0 through the same softmax
    gr = oracle.backward(inp, 1, dy, aux_scale=1.0, train=False, w_importance=0.5, w_load=0.0)
    assert np.all(gr["dw_gate"] == 0.0)


def test_single_expert_is_the_mlp_backward():
    """n = 1, k = 1, no noise, no losses: y = E(x) = ReLU(x W1^T + b1) W2^T + b2,
    whose backward is written here with NumPy products."""
    w, inp, dy = small_case(31, n=1, k=1, B=9, d=8, h=16)
    gr = oracle.backward(inp, 1, dy, train=False, w_importance=0.0, w_load=0.0)
    x = inp["x"].astype(np.float64)
    W1, b1 = inp["w1"][0].astype(np.float64), inp["b1"][0].astype(np.float64)
    W2 = inp["w2"][0].astype(np.float64)
    A = x @ W1.T + b1
    Hh = np.maximum(A, 0.0)
    dH = dy @ W2
    dA = dH * (A > 0)
    np.testing.assert_allclose(gr["dw2"][0], dy.T @ Hh, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["db2"][0], dy.sum(0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dw1"][0], dA.T @ x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["db1"][0], dA.sum(0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dx"], dA @ W1, rtol=1e-12, atol=1e-12)
    assert np.all(gr["dw_gate"] == 0.0)


def test_unselected_experts_get_gate_gradient_only_from_the_load_loss():
    """An expert no token kept receives no Importance or task gradient (its
    gate is exactly 0), but the Load loss still moves its clean logit through
    eq 9's numerator; its expert parameters get nothing."""
    w, inp, dy = small_case(41, n=6, k=2, B=3)
    ref = oracle.gate(inp, 2, noise_floor=FLOOR)
    unused = np.setdiff1d(np.arange(6), ref["topk_idx"].ravel())
    assert unused.size > 0
    no_load = oracle.backward(inp, 2, dy, w_importance=0.5, w_load=0.0, noise_floor=FLOOR)
    with_load = oracle.backward(inp, 2, dy, w_importance=0.5, w_load=0.5, noise_floor=FLOOR)
    for e in unused:
        assert np.all(no_load["dw_gate"][e] == 0.0) and no_load["dgate_bias"][e] == 0.0
        assert np.abs(with_load["dw_gate"][e]).max() > 0.0
        assert np.all(with_load["dw1"][e] == 0.0) and np.all(with_load["db2"][e] == 0.0)


@pytest.mark.parametrize("train", [True, False])
def test_sampled_backward_is_the_backward(train):
    """The sampled backward (one gate pass over the batch, then only the listed
    experts and tokens) gives the whole backward's values: every expert and
    token listed, and a subset listed out of order, with a forced selection."""
    w, inp, dy = small_case(51, n=7, k=3, B=40)
    ref = oracle.gate(inp, 3, train=train, noise_floor=FLOOR)
    sel = ref["topk_idx"][:, ::-1].copy()  # the same sets, another slot order
    kw = dict(aux_scale=0.8, train=train, noise_floor=FLOOR, w_importance=0.3, w_load=0.4,
              force_idx=sel)
    full = oracle.backward(inp, 3, dy, **kw)
    allE, allT = np.arange(7), np.arange(40)
    sm = oracle.backward_sampled(inp, 3, dy, gate_experts=allE, experts=allE, tokens=allT, **kw)
    for key in ("dw_gate", "dw_noise", "dgate_bias", "dw1", "db1", "dw2", "db2", "dx"):
        np.testing.assert_allclose(sm[key], full[key], rtol=1e-12, atol=1e-14, err_msg=key)
    E, T = np.array([5, 0, 3]), np.array([39, 2, 17, 0])
    sub = oracle.backward_sampled(inp, 3, dy, gate_experts=E, experts=E[::-1], tokens=T, **kw)
    np.testing.assert_allclose(sub["dw_gate"], full["dw_gate"][E], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["dw1"], full["dw1"][E[::-1]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["dx"], full["dx"][T], rtol=1e-12, atol=1e-14)
