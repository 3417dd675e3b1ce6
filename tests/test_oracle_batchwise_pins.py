"""Pins of the oracle's batchwise gating ([MoE-explainer] "What the paper
measured": each expert takes the top m = k|X|/n rows of the batch in
training, a learned per-expert threshold at inference).

The pages give no worked example for this gate, so the pins are a hand-worked
case, a brute-force count of ranks (a second formulation of the column-wise
choice), and the special cases that reduce to the dense softmax or to one
expert.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle

from test_oracle_pins import const_experts, f32, inputs


# Hand-worked case: B = 4 rows, n = 2 experts, k = 1, so m = k B / n = 2.
#   column 0: 3, 2, 2, 0 -> rows 0 (3) and 1 (2; row 2 ties at 2 and loses to the lower row)
#   column 1: 1, 5, 4, 6 -> rows 3 (6) and 1 (5)
# Gates: row 0 keeps only expert 0 -> (1, 0); row 1 keeps both -> softmax(2, 5) =
# (1 / (1 + e^3), e^3 / (1 + e^3)) = (0.04742587..., 0.95257412...); row 2 keeps
# nothing -> (0, 0); row 3 keeps only expert 1 -> (0, 1).
HAND_S = np.array([[3.0, 1.0], [2.0, 5.0], [2.0, 4.0], [0.0, 6.0]])


def test_hand_worked_selection_and_gates():
    counts, keep = oracle.batchwise_select(HAND_S, 2)
    assert counts.tolist() == [2, 2]
    assert keep.tolist() == [[True, False], [True, True], [False, False], [False, True]]
    G = oracle.batchwise_gates(HAND_S, keep)
    g1 = 1.0 / (1.0 + math.e ** 3)
    assert G[0].tolist() == [1.0, 0.0]
    assert G[1] == pytest.approx([g1, 1.0 - g1], abs=1e-15)
    assert abs(G[1, 0] - 0.0474258731775668) < 1e-15
    assert G[2].tolist() == [0.0, 0.0]
    assert G[3].tolist() == [0.0, 1.0]


def test_hand_worked_thresholds():
    """Inference rule: thresholds (1.5, 4.5) and no cap (m = B) keep column 0's
    rows 0-2 (3, 2, 2 > 1.5) and column 1's rows 1, 3 (5, 6 > 4.5); a cap of
    m = 2 then drops row 2 from column 0 (the tie at 2 goes to row 1)."""
    counts, keep = oracle.batchwise_select(HAND_S, 4, np.array([1.5, 4.5]))
    assert counts.tolist() == [3, 2]
    assert keep.tolist() == [[True, False], [True, True], [True, False], [False, True]]
    G = oracle.batchwise_gates(HAND_S, keep)
    assert G[2].tolist() == [1.0, 0.0]
    counts, keep = oracle.batchwise_select(HAND_S, 2, np.array([1.5, 4.5]))
    assert counts.tolist() == [2, 2]
    assert keep[:, 0].tolist() == [True, True, False, False]
    # a threshold equal to a score excludes it (strictly greater)
    counts, _ = oracle.batchwise_select(HAND_S, 4, np.array([2.0, 6.0]))
    assert counts.tolist() == [1, 0]


def brute_force_keep(S, m, thr):
    """Row t is kept by expert i when it passes the threshold and fewer than m
    passing rows of the column rank above it (a larger score, or an equal
    score on a lower row)."""
    B, n = S.shape
    keep = np.zeros((B, n), bool)
    for i in range(n):
        for t in range(B):
            if not S[t, i] > thr[i]:
                continue
            above = sum(1 for u in range(B)
                        if S[u, i] > thr[i] and (S[u, i] > S[t, i] or (S[u, i] == S[t, i] and u < t)))
            keep[t, i] = above < m
    return keep


@pytest.mark.parametrize("seed", range(4))
def test_selection_matches_brute_force_ranks(seed):
    rng = np.random.default_rng(100 + seed)
    B, n = 23, 5
    S = rng.integers(-3, 4, size=(B, n)).astype(np.float64)  # many ties
    m = int(rng.integers(1, B + 1))
    thr = np.where(rng.random(n) < 0.5, -np.inf, rng.integers(-3, 3, size=n).astype(np.float64))
    counts, keep = oracle.batchwise_select(S, m, thr)
    ref = brute_force_keep(S, m, thr)
    assert np.array_equal(keep, ref)
    assert np.array_equal(counts, ref.sum(0))


def test_training_rule_gives_every_expert_m_rows():
    rng = np.random.default_rng(7)
    B, n, k = 64, 8, 2
    m = k * B // n
    S = rng.normal(size=(B, n))
    counts, keep = oracle.batchwise_select(S, m)
    assert np.all(counts == m)
    # every kept score is at least every dropped score of its column
    for i in range(n):
        assert S[keep[:, i], i].min() >= S[~keep[:, i], i].max()
    G = oracle.batchwise_gates(S, keep)
    rows = keep.any(axis=1)
    assert np.allclose(G[rows].sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(G[~rows] == 0.0)
    assert np.all((G > 0) == keep)


def test_every_row_kept_is_the_dense_softmax():
    """m = B without thresholds: every expert takes every row, so the gates are
    the dense softmax of eq 2 (scipy's) and, with constant experts, y is that
    softmax times the experts' outputs (numpy's matmul)."""
    rng = np.random.default_rng(11)
    B, d, n = 30, 6, 5
    x = f32(rng.normal(size=(B, d)))
    wg = f32(rng.normal(size=(n, d)))
    inp = inputs(x, wg, np.zeros((n, d)))
    inp.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.batchwise_forward(inp, B, train=False)
    dense = sp_softmax(x.astype(np.float64) @ wg.astype(np.float64).T, axis=1)
    assert np.all(out["counts"] == B)
    assert np.allclose(out["G"], dense, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["y"], dense @ inp["b2"].astype(np.float64), rtol=1e-10, atol=1e-12)
    assert np.allclose(out["importance"], dense.sum(0), rtol=1e-10)
    assert out["losses"][1] == 0.0


def test_one_expert_is_the_mlp_on_its_rows():
    """n = 1: the expert takes its m best rows with gate exactly 1, and y of
    those rows is the expert's output; the other rows get 0."""
    rng = np.random.default_rng(12)
    B, d, h, m = 10, 5, 4, 6
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(1, d)), rng.normal(size=(1, d)),
                 eps=rng.normal(size=(B, 1)), w1=rng.normal(size=(1, h, d)),
                 w2=rng.normal(size=(1, d, h)))
    out = oracle.batchwise_forward(inp, m)
    kept = np.flatnonzero(out["keep"][:, 0])
    assert kept.size == m
    H = out["H"][:, 0].astype(np.float32)
    assert H[kept].min() >= np.delete(H, kept).max()
    ref = oracle.expert_pairs(inp, kept, np.zeros(m, np.int32))
    assert np.array_equal(out["y"][kept], ref)
    assert np.all(out["y"][np.setdiff1d(np.arange(B), kept)] == 0.0)
    assert np.all(out["G"][kept, 0] == 1.0)


def test_infinite_thresholds():
    rng = np.random.default_rng(13)
    B, d, n = 9, 4, 3
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), np.zeros((n, d)))
    inp.update({key: f32(v) for key, v in const_experts(n, d).items()})
    out = oracle.batchwise_forward(inp, B, train=False, threshold=np.full(n, np.inf))
    assert np.all(out["counts"] == 0) and np.all(out["y"] == 0.0)
    a = oracle.batchwise_forward(inp, B, train=False, threshold=np.full(n, -np.inf))
    b = oracle.batchwise_forward(inp, B, train=False)
    assert np.array_equal(a["y"], b["y"])


def test_score_columns_match_the_gate_logits():
    """The column helper and the row-wise gate give the same H (two code
    paths: numpy over columns, the C oracle over rows)."""
    rng = np.random.default_rng(14)
    B, d, n = 20, 8, 6
    inp = inputs(rng.normal(size=(B, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)),
                 eps=rng.normal(size=(B, n)), bg=rng.normal(size=n))
    H = oracle.gate(inp, 1, want_logits=True)["H"]
    cols = [4, 0, 5]
    assert np.allclose(oracle.score_columns(inp, cols), H[:, cols], rtol=1e-12, atol=1e-12)
    Hc = oracle.gate(inp, 1, train=False, want_logits=True)["H"]
    assert np.allclose(oracle.score_columns(inp, cols, train=False), Hc[:, cols], rtol=1e-12,
                       atol=1e-12)
