"""Helpers for comparing the HIP path with the oracle.

Tolerances (max relative error, judged against max(|ref|, RMS(ref)) so that
near-zero elements are measured on the tensor's own scale):
  * fp32 workloads: 1e-4;  bf16 workloads: 2e-2 (outputs y and expert outputs);
  * gate outputs (gates, thresholds), Importance, Load and the losses are fp32
    arithmetic in every workload and are held to 1e-4, the fp32 bar (the
    losses as scalars: |g - r| / |r| <= ``LOSS_TOL``).

Near ties. The selection is decided on fp32 logits whose rounding differs
between the GPU's accumulation order and the oracle's fp64 sums. A row is a
near tie when its k-th and (k+1)-th oracle logits are within
``1e-4 * max(|v_k|, |v_k+1|) + 1e-6``. On all other rows the selected expert
sets must match exactly; on near-tie rows the GPU's set must be a valid top k
of the oracle's logits within that margin, and everything downstream is
checked against the oracle evaluated on the GPU's (valid) set.
"""
from __future__ import annotations

import os
import sys
from typing import Dict

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
GATE_TOL = 1e-4
LOSS_TOL = 1e-4
NEAR_TIE_REL = 1e-4
NEAR_TIE_ABS = 1e-6


def announce(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so a crash still shows
    it), also appended to gpu_cases.log in the output folder at the repository
    root, whose growth shows that a long case is still making progress."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)
    with open(os.path.join(output_dir(), "gpu_cases.log"), "a") as f:
        f.write(msg + "\n")


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    denom = np.maximum(np.abs(ref), rms)
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(got - ref) / denom))


def scalar_rel(got, ref) -> float:
    got, ref = float(got), float(ref)
    if ref == 0.0:
        return abs(got)
    return abs(got - ref) / abs(ref)


def near_tie_rows(thresh: np.ndarray) -> np.ndarray:
    vk, vk1 = thresh[:, 0], thresh[:, 1]
    finite = np.isfinite(vk1)
    margin = np.where(finite, vk - vk1, np.inf)
    scale = np.maximum(np.abs(vk), np.where(finite, np.abs(vk1), 0.0))
    return margin <= NEAR_TIE_REL * scale + NEAR_TIE_ABS


def softmax_at(H_row: np.ndarray, idx: np.ndarray) -> np.ndarray:
    v = H_row[idx].astype(np.float64)
    e = np.exp(v - v.max())
    return e / e.sum()


def check_gating(ref: Dict[str, np.ndarray], H: np.ndarray, g_idx: np.ndarray,
                 g_gate: np.ndarray, g_thr: np.ndarray, rows=None,
                 gate_order: int = 0) -> Dict[str, object]:
    """Compare GPU gating on rows `rows` (default all) with the oracle's.

    ``ref`` holds the oracle's topk_idx/topk_gate/thresh for those rows and
    ``H`` the oracle's noisy logits for them. Returns the near-tie rows whose
    GPU set differs (``swapped``) for downstream adjustment.
    """
    k = g_idx.shape[1]
    if rows is not None:
        g_idx, g_gate, g_thr = g_idx[rows], g_gate[rows], g_thr[rows]
    r_idx, r_gate, r_thr = ref["topk_idx"], ref["topk_gate"], ref["thresh"]
    tie = near_tie_rows(r_thr)
    same_set = np.array([set(a) == set(b) for a, b in zip(g_idx.tolist(), r_idx.tolist())])
    bad = ~same_set & ~tie
    assert not bad.any(), f"selection differs on {bad.sum()} non-near-tie rows, e.g. row " \
                          f"{np.nonzero(bad)[0][:5]}: gpu {g_idx[bad][:3]} oracle {r_idx[bad][:3]}"
    swapped = np.nonzero(~same_set)[0]
    # near-tie rows with another set: it must still be a top k within the margin
    for r in swapped:
        sel = g_idx[r]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < H.shape[1]
        rest = np.setdiff1d(np.arange(H.shape[1]), sel)
        lo = H[r, sel].min()
        hi = H[r, rest].max() if rest.size else -np.inf
        scale = max(abs(lo), abs(hi) if np.isfinite(hi) else 0.0)
        assert lo >= hi - (NEAR_TIE_REL * scale + NEAR_TIE_ABS), f"row {r}: not a valid top-k"
    # gates per expert (order-free), against the oracle on the GPU's set
    ref_gate_by_set = np.empty_like(g_gate, dtype=np.float64)
    for r in range(g_idx.shape[0]):
        if same_set[r]:
            m = {int(e): gv for e, gv in zip(r_idx[r], r_gate[r])}
            ref_gate_by_set[r] = [m[int(e)] for e in g_idx[r]]
        elif gate_order == 1:  # the softmax over all n at the GPU's set
            e = np.exp(H[r] - H[r].max())
            ref_gate_by_set[r] = e[g_idx[r]] / e.sum()
        else:
            ref_gate_by_set[r] = softmax_at(H[r], g_idx[r])
    gerr = rel_err(g_gate, ref_gate_by_set)
    assert gerr <= GATE_TOL, f"gate error {gerr}"
    # rank order: the GPU's slots must be in descending oracle logit, up to the margin
    Hs = np.take_along_axis(H, g_idx.astype(np.int64), axis=1)
    scale = np.abs(Hs).max(axis=1, keepdims=True)
    assert np.all(np.diff(Hs, axis=1) <= NEAR_TIE_REL * scale + NEAR_TIE_ABS)
    # thresholds: k-th and (k+1)-th largest logits
    terr = rel_err(np.where(np.isfinite(g_thr), g_thr, 0), np.where(np.isfinite(r_thr), r_thr, 0))
    assert np.array_equal(np.isfinite(g_thr), np.isfinite(r_thr))
    assert terr <= GATE_TOL, f"threshold error {terr}"
    return {"near_tie": int(tie.sum()), "swapped": swapped, "gate_err": gerr, "thr_err": terr}


def to_device(a: np.ndarray, device="cuda"):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return (t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
                << 16).view(np.float32)
    return t.detach().cpu().numpy()


def gpu_inputs(inp: Dict[str, np.ndarray], device="cuda") -> Dict[str, object]:
    return {k: to_device(v, device) for k, v in inp.items()}


def device_tensor(w, name: str, shape, device="cuda", chunk: int = 1 << 27):
    """Input tensor ``name`` of workload ``w`` generated chunk by chunk straight
    into device memory (so tens of GB of expert weights never sit in host
    memory); progress goes to the case log."""
    import torch
    import datagen as dg
    total = int(np.prod(shape))
    bf16 = dg.gen(w, name, 0, 1).dtype == np.uint16
    t = torch.empty(total, dtype=torch.bfloat16 if bf16 else torch.float32, device=device)
    for i, off in enumerate(range(0, total, chunk)):
        cnt = min(chunk, total - off)
        a = dg.gen(w, name, off, cnt)
        src = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        t[off:off + cnt].copy_(src)
        if i % 16 == 15:
            announce(f"  {name}: {(off + cnt) / total:.0%}")
    return t.view(*shape)


def out_tol(act_is_bf16: bool) -> float:
    return TOL_BF16 if act_is_bf16 else TOL_F32


def output_dir() -> str:
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    os.makedirs(d, exist_ok=True)
    return d
