"""Pins of the hierarchical oracle (section "Hierarchical MoE" of the explainer
"Mixture of Experts: Outrageously Large Neural Networks"; eq 12 is missing from
the page and is read from its prose).

Each check ties the hierarchical oracle to something other than itself:
  * a = 1, k1 = 1 reduces to the flat layer over the group's b experts, and
    b = 1, k2 = 1 to the flat layer over the a groups (the flat oracle is
    pinned on its own in test_oracle_pins.py);
  * with every expert kept and no noise the layer is a dense two-level softmax
    mixture, computed here independently with numpy matrix products;
  * structural invariants: k1*k2 distinct leaves per token inside the chosen
    groups, leaf gates that are products of the two levels and sum to 1,
    Importance summing to B.
The hierarchy's balancing losses appear on none of the pages; the oracle's
reading (leaf Importance = the leaf gate sums, leaf Load = Load1_i Load2_ij /
|X_i|) is pinned at its limits:
  * the two reductions above;
  * with every expert kept and no noise, leaf Importance against the dense
    mixture's gate products;
  * with train = 0 both levels' Loads are hard counts, so the leaf Load is the
    number of tokens at each leaf, counted here from the selection alone, and
    the losses are the CV^2 of those counts and of the leaf gate sums;
  * in training with the noise scale driven to zero every eq 9 term is
    exactly 0 or 1, and the training formula gives the same hard counts.
Between those limits the product form is a reading: no page defines it.
"""
import numpy as np
import pytest

import datagen as dg
import oracle

FLOOR = 1e-2


def hier_wl(tokens=200, a=4, b=6, k1=2, k2=2, d=64, h=128, dtype=dg.F32):
    return dg.workload("hier_bf16_16384", tokens=tokens, d_model=d, d_hidden=h, groups=a,
                       group_experts=b, k1=k1, k2=k2, n_experts=a * b, k=k1 * k2,
                       act_dtype=dtype, expert_dtype=dtype, gate_dtype=dtype)


def as64(a):
    return dg.as_f32(a).astype(np.float64)


@pytest.mark.parametrize("train", [True, False])
def test_one_group_is_the_flat_layer(train):
    w = hier_wl(tokens=300, a=1, b=12, k1=1, k2=3)
    inp = dg.make_hier_inputs(w, with_bias=True)
    hier = oracle.hier_forward(inp, 1, 3, train=train, noise_floor=FLOOR)
    flat_inp = {"x": inp["x"], "w_gate": inp["w_gate2"][0], "w_noise": inp["w_noise2"][0],
                "eps": np.ascontiguousarray(inp["eps2"][:, 0, :]), "w1": inp["w1"],
                "w2": inp["w2"], "b1": inp["b1"], "b2": inp["b2"]}
    flat = oracle.forward(flat_inp, 3, train=train, noise_floor=FLOOR)
    np.testing.assert_array_equal(hier["leaf_idx"], flat["topk_idx"])
    np.testing.assert_allclose(hier["leaf_gate"], flat["topk_gate"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(hier["y"], flat["y"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hier["importance"], flat["importance"], rtol=1e-12)
    np.testing.assert_allclose(hier["load"], flat["load"], rtol=1e-12)
    np.testing.assert_allclose(hier["losses"], flat["losses"], rtol=1e-10, atol=1e-15)
    # the single group takes every token, with gate and Load exactly B
    assert hier["rows1"][0] == w.tokens and hier["imp1"][0] == pytest.approx(w.tokens)
    assert hier["load1"][0] == pytest.approx(w.tokens)


@pytest.mark.parametrize("train", [True, False])
def test_one_expert_per_group_is_the_flat_layer(train):
    w = hier_wl(tokens=300, a=10, b=1, k1=3, k2=1)
    inp = dg.make_hier_inputs(w)
    hier = oracle.hier_forward(inp, 3, 1, train=train, noise_floor=FLOOR)
    flat_inp = {"x": inp["x"], "w_gate": inp["w_gate"], "w_noise": inp["w_noise"],
                "eps": inp["eps"], "w1": inp["w1"], "w2": inp["w2"]}
    flat = oracle.forward(flat_inp, 3, train=train, noise_floor=FLOOR)
    np.testing.assert_array_equal(hier["leaf_idx"], flat["topk_idx"])
    np.testing.assert_allclose(hier["leaf_gate"], flat["topk_gate"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(hier["y"], flat["y"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hier["importance"], flat["importance"], rtol=1e-12)
    np.testing.assert_allclose(hier["load"], flat["load"], rtol=1e-12)
    np.testing.assert_allclose(hier["imp1"], flat["importance"], rtol=1e-12)
    np.testing.assert_allclose(hier["losses"], flat["losses"], rtol=1e-10, atol=1e-15)


def test_all_kept_without_noise_is_a_dense_two_level_mixture():
    a, b, B, d, h = 3, 4, 40, 64, 128
    w = hier_wl(tokens=B, a=a, b=b, k1=a, k2=b, d=d, h=h)
    inp = dg.make_hier_inputs(w)
    out = oracle.hier_forward(inp, a, b, train=False)
    x = as64(inp["x"])

    def softmax(z):
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=-1, keepdims=True)

    g1 = softmax(x @ as64(inp["w_gate"]).T)                               # [B, a]
    g2 = softmax(np.einsum("td,ijd->tij", x, as64(inp["w_gate2"])))       # [B, a, b]
    w1, w2 = as64(inp["w1"]), as64(inp["w2"])
    y = np.zeros((B, d))
    for i in range(a):
        for j in range(b):
            e = i * b + j
            E = np.maximum(x @ w1[e].T, 0.0) @ w2[e].T
            y += (g1[:, i] * g2[:, i, j])[:, None] * E
    np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["importance"], (g1[:, :, None] * g2).sum(0).ravel(),
                               rtol=1e-10)
    # every leaf holds every token: hard Load B everywhere, CV^2 0
    np.testing.assert_allclose(out["load"], B)
    assert out["losses"][1] == 0.0


def test_structure_of_the_selection():
    w = hier_wl(tokens=257, a=8, b=16, k1=2, k2=3, dtype=dg.BF16)
    inp = dg.make_hier_inputs(w)
    g = oracle.hier_gate(inp, 2, 3, noise_floor=FLOOR, want_logits=True)
    f = oracle.hier_forward(inp, 2, 3, noise_floor=FLOOR)
    K = 6
    np.testing.assert_array_equal(g["leaf_idx"], f["leaf_idx"])
    np.testing.assert_allclose(g["leaf_gate"], f["leaf_gate"], rtol=1e-15)
    for t in range(w.tokens):
        leaves = g["leaf_idx"][t]
        assert len(set(leaves.tolist())) == K
        # slot (r, j) is leaf sel1[r] * b + sel2[r, j]
        np.testing.assert_array_equal(leaves.reshape(2, 3) // 16, np.repeat(g["sel1"][t][:, None], 3, 1))
        np.testing.assert_array_equal(leaves.reshape(2, 3) % 16, g["sel2"][t])
    np.testing.assert_allclose(g["leaf_gate"].reshape(-1, 2, 3),
                               g["gate1"][:, :, None] * g["gate2"], rtol=1e-15)
    np.testing.assert_allclose(g["leaf_gate"].sum(1), 1.0, rtol=1e-12)
    # each level selects its top k by logit, ranked
    H1, H2 = g["H1"], g["H2"]
    for t in range(w.tokens):
        o1 = np.argsort(-H1[t].astype(np.float32), kind="stable")
        np.testing.assert_array_equal(g["sel1"][t], o1[:2])
        assert g["thr1"][t, 0] == H1[t, o1[1]] and g["thr1"][t, 1] == H1[t, o1[2]]
        for r in range(2):
            o2 = np.argsort(-H2[t, r].astype(np.float32), kind="stable")
            np.testing.assert_array_equal(g["sel2"][t, r], o2[:3])
    assert f["importance"].sum() == pytest.approx(w.tokens, rel=1e-12)
    assert f["rows1"].sum() == w.tokens * 2
    np.testing.assert_allclose(f["imp1"].sum(), w.tokens, rtol=1e-12)
    # leaf Load from the level vectors
    l1, l2, r1 = f["load1"], f["load2"].reshape(8, 16), f["rows1"]
    np.testing.assert_allclose(f["load"].reshape(8, 16),
                               np.where(r1[:, None] > 0, l1[:, None] * l2 / np.maximum(r1, 1)[:, None], 0),
                               rtol=1e-12)


def test_secondary_noise_is_indexed_by_primary_rank():
    # eps2[t, r, :] belongs to the r-th picked group: swapping the two rank
    # rows of eps2 and forcing the primary picks in swapped order gives the
    # same secondary choices per group.
    w = hier_wl(tokens=64, a=5, b=8, k1=2, k2=2)
    inp = dg.make_hier_inputs(w)
    g = oracle.hier_gate(inp, 2, 2, noise_floor=FLOOR)
    sw = dict(inp)
    sw["eps2"] = np.ascontiguousarray(inp["eps2"][:, ::-1, :])
    g2 = oracle.hier_gate(sw, 2, 2, noise_floor=FLOOR, force1=g["sel1"][:, ::-1])
    np.testing.assert_array_equal(g2["sel2"], g["sel2"][:, ::-1])
    np.testing.assert_allclose(g2["gate2"], g["gate2"][:, ::-1], rtol=1e-15)


def test_forced_selection():
    w = hier_wl(tokens=50, a=6, b=5, k1=2, k2=2)
    inp = dg.make_hier_inputs(w)
    own = oracle.hier_forward(inp, 2, 2, noise_floor=FLOOR)
    g = oracle.hier_gate(inp, 2, 2, noise_floor=FLOOR, want_logits=True)
    same = oracle.hier_forward(inp, 2, 2, noise_floor=FLOOR, force1=g["sel1"], force2=g["sel2"])
    for key in own:
        np.testing.assert_array_equal(own[key], same[key])
    # another primary set on row 0: the secondary gates then run on those groups
    f1 = g["sel1"].copy()
    other = [i for i in range(6) if i not in f1[0]]
    f1[0] = [other[0], other[1]]
    alt = oracle.hier_gate(inp, 2, 2, noise_floor=FLOOR, force1=f1, want_logits=True)
    np.testing.assert_array_equal(alt["sel1"][0], f1[0])
    np.testing.assert_array_equal(alt["leaf_idx"][0].reshape(2, 2) // 5,
                                  np.repeat(f1[0][:, None], 2, 1))
    H = alt["H1"][0]
    e = np.exp(H[f1[0]] - H[f1[0]].max())
    np.testing.assert_allclose(alt["gate1"][0], e / e.sum(), rtol=1e-14)
    np.testing.assert_array_equal(alt["thr1"][0], g["thr1"][0])
    np.testing.assert_array_equal(alt["leaf_idx"][1:], g["leaf_idx"][1:])
    with pytest.raises(ValueError):
        bad = g["sel1"].copy()
        bad[0] = [1, 1]
        oracle.hier_gate(inp, 2, 2, force1=bad)


def test_batch_sums_without_the_experts():
    """hier_forward(with_y=False) skips only the experts: every batch sum and
    the selection equal the full call's, bit for bit."""
    w = hier_wl(tokens=300, a=5, b=7, k1=2, k2=2)
    inp = dg.make_hier_inputs(w)
    full = oracle.hier_forward(inp, 2, 2, noise_floor=FLOOR)
    gates_only = {k: v for k, v in inp.items() if k not in ("w1", "w2")}
    part = oracle.hier_forward(gates_only, 2, 2, noise_floor=FLOOR, with_y=False)
    assert "y" not in part
    for key, v in part.items():
        np.testing.assert_array_equal(v, full[key], err_msg=key)


def _cv2(v):
    """Population variance over the squared mean (0 for one entry or mean 0)."""
    v = np.asarray(v, np.float64)
    m = v.mean()
    return 0.0 if v.size <= 1 or m == 0 else float(((v - m) ** 2).mean() / m ** 2)


@pytest.mark.parametrize("a,b,k1,k2", [(4, 6, 2, 2), (8, 5, 3, 2), (3, 16, 1, 4)])
def test_hard_leaf_load_is_the_leaf_count(a, b, k1, k2):
    """train = 0: Load1_i = |X_i| and Load2_ij counts the rows of X_i that
    picked j, so Load1_i Load2_ij / |X_i| is the number of tokens at leaf
    (i, j); leaf Importance is each leaf's sum of leaf gates; the losses are
    their CV^2 with weights 0.1."""
    w = hier_wl(tokens=500, a=a, b=b, k1=k1, k2=k2)
    inp = dg.make_hier_inputs(w, experts=False)
    out = oracle.hier_forward(inp, k1, k2, train=False, with_y=False)
    n = a * b
    idx = out["leaf_idx"].ravel()
    counts = np.bincount(idx, minlength=n).astype(np.float64)
    np.testing.assert_allclose(out["load"], counts, rtol=1e-12, atol=0)
    imp = np.bincount(idx, weights=out["leaf_gate"].ravel(), minlength=n)
    np.testing.assert_allclose(out["importance"], imp, rtol=1e-12, atol=1e-12)
    cvi, cvl = _cv2(imp), _cv2(counts)
    np.testing.assert_allclose(out["losses"], [cvi, cvl, 0.1 * cvi + 0.1 * cvl],
                               rtol=1e-10, atol=1e-15)
    # the primary level's hard Load is its routed row count
    np.testing.assert_allclose(out["load1"], out["rows1"], rtol=0, atol=0)
    np.testing.assert_allclose(out["rows1"], np.bincount(idx // b, minlength=a) / k2)


def test_vanishing_noise_leaf_load_is_the_leaf_count():
    """train = 1 with the noise scale driven to zero: a constant feature
    x[:, 0] = 1 and noise weights of -40 on it (all others 0) make every noise
    pre-activation -40, so sigma = Softplus(-40) ~ 4e-18 with the floor at 0.
    Each eq 9 term Phi((clean - thr) / sigma) is then exactly 0 or 1, the
    selection is the noise-free one, and the training Loads of both levels and
    of the leaves equal the hard counts."""
    a, b, k1, k2 = 6, 8, 2, 3
    w = hier_wl(tokens=400, a=a, b=b, k1=k1, k2=k2)
    inp = dg.make_hier_inputs(w, experts=False)
    x = inp["x"].copy()
    x[:, 0] = 1.0
    inp["x"] = x
    wn = np.zeros_like(inp["w_noise"])
    wn[:, 0] = -40.0
    inp["w_noise"] = wn
    wn2 = np.zeros_like(inp["w_noise2"])
    wn2[:, :, 0] = -40.0
    inp["w_noise2"] = wn2
    tr = oracle.hier_forward(inp, k1, k2, train=True, noise_floor=0.0, with_y=False)
    hard = oracle.hier_forward(inp, k1, k2, train=False, with_y=False)
    np.testing.assert_array_equal(tr["leaf_idx"], hard["leaf_idx"])
    counts = np.bincount(hard["leaf_idx"].ravel(), minlength=a * b).astype(np.float64)
    np.testing.assert_allclose(tr["load"], counts, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(tr["load1"], tr["rows1"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(tr["losses"][1], _cv2(counts), rtol=1e-10)
