"""Oracle for the sparsely-gated MoE forward pass (test infrastructure only).

A thin ctypes wrapper over ``moe_oracle.cpp``: a plain CPU implementation of
the pages' equations in fp64, shared with nothing on the GPU path. Only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package.

Inputs are numpy arrays in the storage layouts of ``datagen`` (fp32 arrays as
float32, bf16 arrays as uint16 bit patterns); outputs are float64/int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_D = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile the oracle with g++/OpenMP (plain -O2, no fast-math)."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_threads.restype = _I
        lib.oracle_set_threads.argtypes = [_I]
        lib.oracle_set_threads.restype = None
        lib.oracle_softplus.argtypes = [_D]
        lib.oracle_softplus.restype = _D
        lib.oracle_phi.argtypes = [_D]
        lib.oracle_phi.restype = _D
        lib.oracle_cv2.argtypes = [_I, _P]
        lib.oracle_cv2.restype = _D
        lib.oracle_gate.argtypes = [_I64, _P, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D, _I,
                                    _P, _P, _P, _P, _P, _P]
        lib.oracle_load.argtypes = [_I64, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D, _I, _P]
        lib.oracle_y_rows.argtypes = [_I64, _P, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D,
                                      _I, _P, _P, _P, _P, _I, _P]
        lib.oracle_expert_pairs.argtypes = [_I64, _P, _P, _I, _I, _P, _I, _P, _P, _P, _P, _I, _P]
        lib.oracle_route.argtypes = [_I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_forward.argtypes = [_I64, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D,
                                       _I, _P, _P, _P, _P, _I, _D, _D, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_hier_gate.argtypes = [_I64, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P,
                                         _I, _P, _P, _I, _D, _I, _P, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_hier_forward.argtypes = [_I64, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P,
                                            _I, _P, _P, _I, _D, _I, _P, _P, _P, _P, _P, _P, _I,
                                            _D, _D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_objective.argtypes = [_I64, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D,
                                         _P, _P, _P, _P, _I, _D, _D, _P, _D, _P, _P, _P]
        lib.oracle_backward.argtypes = [_I64, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D,
                                        _I, _P, _P, _P, _P, _I, _D, _D, _P, _D, _P] + [_P] * 8
        lib.oracle_backward_sampled.argtypes = (
            [_I64, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _D, _I, _P, _P, _P, _P, _I,
             _D, _D, _P, _D, _P] + [_I, _P, _P, _P, _P] + [_I, _P, _P, _P, _P, _P] + [_I, _P, _P])
        lib.oracle_backward_sampled.restype = _I
        lib.oracle_cv2_grad.argtypes = [_I, _P, _P]
        lib.oracle_cv2_grad.restype = None
        lib.oracle_kept_softmax_grad.argtypes = [_I, _P, _P, _P]
        lib.oracle_kept_softmax_grad.restype = None
        lib.oracle_p_eq9_grad.argtypes = [_D, _D, _D, _P, _P]
        lib.oracle_p_eq9_grad.restype = None
        for f in ("oracle_objective", "oracle_backward"):
            getattr(lib, f).restype = _I
        for f in ("oracle_gate", "oracle_load", "oracle_y_rows", "oracle_expert_pairs",
                  "oracle_route", "oracle_forward", "oracle_hier_gate", "oracle_hier_forward"):
            getattr(lib, f).restype = _I
        _lib = lib
    return _lib


def _arr(a, dtype=None):
    if a is None:
        return None, 0
    a = np.ascontiguousarray(a) if dtype is None else np.ascontiguousarray(a, dtype=dtype)
    if a.dtype == np.uint16:
        return a, 1
    if a.dtype != np.float32:
        a = np.ascontiguousarray(a, dtype=np.float32)
    return a, 0


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (code {rc})")


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's later calls from this thread."""
    _load().oracle_set_threads(int(n))


def softplus(u: float) -> float:
    return _load().oracle_softplus(float(u))


def phi(z: float) -> float:
    return _load().oracle_phi(float(z))


def cv2(v) -> float:
    """CV^2 of a vector with the population variance (eqs 7 and 11)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    return _load().oracle_cv2(v.size, v.ctypes.data)


class _Gate:
    """Common gate arguments, kept alive for the duration of a call."""

    def __init__(self, inp: Dict[str, np.ndarray], train: bool):
        self.x, self.x_dt = _arr(inp["x"])
        self.wg, self.w_dt = _arr(inp["w_gate"])
        self.wn, wn_dt = _arr(inp["w_noise"])
        if wn_dt != self.w_dt:
            raise ValueError("w_gate and w_noise must share a dtype")
        bg = inp.get("gate_bias")
        self.bg = None if bg is None else np.ascontiguousarray(bg, dtype=np.float32)
        eps = inp.get("eps") if train else None
        self.eps = None if eps is None else np.ascontiguousarray(eps, dtype=np.float32)
        self.B, self.d = self.x.shape
        self.n = self.wg.shape[0]
        if self.wg.shape != (self.n, self.d) or self.wn.shape != (self.n, self.d):
            raise ValueError("w_gate/w_noise must be [n, d]")
        if self.eps is not None and self.eps.shape != (self.B, self.n):
            raise ValueError("eps must be [B, n]")

    def args(self):
        return (_ptr(self.x), self.x_dt, _ptr(self.wg), _ptr(self.wn), self.w_dt, _ptr(self.bg),
                _ptr(self.eps))


def gate(inp: Dict[str, np.ndarray], k: int, train: bool = True, noise_floor: float = 1e-2,
         rows: Optional[Sequence[int]] = None, decide_fp32: bool = True,
         want_logits: bool = False, gate_order: int = 0) -> Dict[str, np.ndarray]:
    """Noisy top-k gating for all rows or a list of rows.

    gate_order 1 keeps the same selection but takes the gates from the softmax
    over all n logits, the order of operations [MoE-explainer] "From LSTMs to
    Switch and Mixtral" attributes to Switch: G_i = exp(H_i) / sum_j exp(H_j)
    for the kept i (so a row's gates sum to at most 1)."""
    g = _Gate(inp, train)
    n = g.n
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = g.B if rws is None else rws.size
    out = {"topk_idx": np.empty((nr, k), np.int32), "topk_gate": np.empty((nr, k), np.float64),
           "thresh": np.empty((nr, 2), np.float64)}
    want_logits = want_logits or gate_order == 1
    if want_logits:
        for key in ("clean", "sigma", "H"):
            out[key] = np.empty((nr, n), np.float64)
    rc = _load().oracle_gate(nr, _ptr(rws), g.d, n, k, *g.args(), int(train), float(noise_floor),
                             int(decide_fp32), _ptr(out.get("clean")), _ptr(out.get("sigma")),
                             _ptr(out.get("H")), _ptr(out["topk_idx"]), _ptr(out["topk_gate"]),
                             _ptr(out["thresh"]))
    _check(rc, "gate")
    if gate_order == 1 and nr > 0:
        H = out["H"]
        top = H.max(axis=1, keepdims=True)
        z = np.exp(H - top).sum(axis=1, keepdims=True)
        out["topk_gate"] = np.exp(np.take_along_axis(H, out["topk_idx"].astype(np.int64), 1) - top) / z
    return out


def load(inp: Dict[str, np.ndarray], k: int, train: bool = True, noise_floor: float = 1e-2,
         decide_fp32: bool = True) -> np.ndarray:
    """Load vector (eq 10) over the whole batch."""
    g = _Gate(inp, train)
    out = np.empty(g.n, np.float64)
    rc = _load().oracle_load(g.B, g.d, g.n, k, *g.args(), int(train), float(noise_floor),
                             int(decide_fp32), out.ctypes.data)
    _check(rc, "load")
    return out


def _experts(inp):
    w1, e_dt = _arr(inp["w1"])
    w2, e2 = _arr(inp["w2"])
    b1, _ = _arr(inp.get("b1"))
    b2, _ = _arr(inp.get("b2"))
    if e2 != e_dt:
        raise ValueError("w1 and w2 must share a dtype")
    for b in (b1, b2):
        if b is not None and (b.dtype == np.uint16) != (e_dt == 1):
            raise ValueError("biases must share the expert dtype")
    h = w1.shape[1]
    return w1, b1, w2, b2, e_dt, h


def y_rows(inp: Dict[str, np.ndarray], k: int, rows: Optional[Sequence[int]] = None,
           train: bool = True, noise_floor: float = 1e-2, decide_fp32: bool = True) -> np.ndarray:
    """MoE output (eq 1) for all rows or a list of rows."""
    g = _Gate(inp, train)
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = g.B if rws is None else rws.size
    y = np.empty((nr, g.d), np.float64)
    rc = _load().oracle_y_rows(nr, _ptr(rws), g.d, h, g.n, k, *g.args(), int(train),
                               float(noise_floor), int(decide_fp32), _ptr(w1), _ptr(b1), _ptr(w2),
                               _ptr(b2), e_dt, y.ctypes.data)
    _check(rc, "y_rows")
    return y


def expert_pairs(inp: Dict[str, np.ndarray], tokens: Sequence[int], experts: Sequence[int]) -> np.ndarray:
    """E_e(x_t) for each listed (token, expert) pair."""
    x, x_dt = _arr(inp["x"])
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    e = np.ascontiguousarray(experts, dtype=np.int32)
    if t.shape != e.shape:
        raise ValueError("tokens and experts must have the same length")
    d = x.shape[1]
    out = np.empty((t.size, d), np.float64)
    rc = _load().oracle_expert_pairs(t.size, t.ctypes.data, e.ctypes.data, d, h, _ptr(x), x_dt,
                                     _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), e_dt, out.ctypes.data)
    _check(rc, "expert_pairs")
    return out


def route(topk_idx: np.ndarray, topk_gate: np.ndarray, n: int,
          capacity: int = 0) -> Dict[str, np.ndarray]:
    """Stable expert-major routing of the (token, slot) pairs, plus Importance.

    capacity > 0 is the fixed per-expert capacity of the GShard variant that
    [MoE-explainer] "From LSTMs to Switch and Mixtral" contrasts with this
    layer: an expert serves only its first `capacity` routed rows (in (token,
    slot) order, i.e. the first positions of its segment); the other pairs keep
    their place in the segments, counts and Importance but get slot_pos -1, so
    they add nothing to y."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    gates = np.ascontiguousarray(topk_gate, dtype=np.float64)
    B, k = idx.shape
    out = {"counts": np.empty(n, np.int32), "offsets": np.empty(n + 1, np.int32),
           "perm_token": np.empty(B * k, np.int32), "perm_gate": np.empty(B * k, np.float64),
           "slot_pos": np.empty(B * k, np.int32), "importance": np.empty(n, np.float64)}
    rc = _load().oracle_route(B, n, k, idx.ctypes.data, gates.ctypes.data,
                              *[out[key].ctypes.data for key in ("counts", "offsets", "perm_token",
                                                                 "perm_gate", "slot_pos",
                                                                 "importance")])
    _check(rc, "route")
    if capacity > 0:
        sp = out["slot_pos"]
        for p in range(B * k):
            if sp[p] >= 0 and sp[p] - out["offsets"][idx.flat[p]] >= capacity:
                sp[p] = -1
    return out


def forward(inp: Dict[str, np.ndarray], k: int, train: bool = True, noise_floor: float = 1e-2,
            w_importance: float = 0.1, w_load: float = 0.1,
            decide_fp32: bool = True) -> Dict[str, np.ndarray]:
    """The layer's forward pass on the batch: eqs 1 and 3-11."""
    g = _Gate(inp, train)
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    B, d, n = g.B, g.d, g.n
    out = {"y": np.empty((B, d), np.float64), "topk_idx": np.empty((B, k), np.int32),
           "topk_gate": np.empty((B, k), np.float64), "thresh": np.empty((B, 2), np.float64),
           "importance": np.empty(n, np.float64), "load": np.empty(n, np.float64),
           "losses": np.empty(3, np.float64)}
    rc = _load().oracle_forward(B, d, h, n, k, *g.args(), int(train), float(noise_floor),
                                int(decide_fp32), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), e_dt,
                                float(w_importance), float(w_load),
                                *[out[key].ctypes.data for key in ("y", "topk_idx", "topk_gate",
                                                                   "thresh", "importance", "load",
                                                                   "losses")])
    _check(rc, "forward")
    return out


# ---------------------------------------------------------------------------
# Backward pass ("Implementation notes": which parameters receive gradients;
# the selection and eq 9's thresholds pass none)
# ---------------------------------------------------------------------------

def cv2_grad(v) -> np.ndarray:
    """d CV^2(v) / d v_i (population variance)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.empty_like(v)
    _load().oracle_cv2_grad(v.size, v.ctypes.data, g.ctypes.data)
    return g


def kept_softmax_grad(gates, dgates) -> np.ndarray:
    """Gradient on the kept logits from the gradient on their softmax gates."""
    g = np.ascontiguousarray(gates, dtype=np.float64)
    dg = np.ascontiguousarray(dgates, dtype=np.float64)
    dH = np.empty_like(g)
    _load().oracle_kept_softmax_grad(g.size, g.ctypes.data, dg.ctypes.data, dH.ctypes.data)
    return dH


def p_eq9_grad(c: float, thr: float, sigma: float):
    """(dP/dc, dP/dsigma) of eq 9's P = Phi((c - thr) / sigma), thr fixed."""
    dc, ds = ctypes.c_double(), ctypes.c_double()
    _load().oracle_p_eq9_grad(float(c), float(thr), float(sigma), ctypes.byref(dc),
                              ctypes.byref(ds))
    return dc.value, ds.value


def _dy(dy, B, d):
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    if dy.shape != (B, d):
        raise ValueError("dy must be [B, d]")
    return dy


def objective(inp: Dict[str, np.ndarray], k: int, dy, force_idx, thresh, aux_scale: float = 1.0,
              train: bool = True, noise_floor: float = 1e-2, w_importance: float = 0.1,
              w_load: float = 0.1) -> float:
    """J = sum dy . y + aux_scale (w_imp CV^2(Imp) + w_load CV^2(Load)) with the
    selection fixed to force_idx [B, k] and eq 9's thresholds to thresh [B, 2]."""
    g = _Gate(inp, train)
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    dy = _dy(dy, g.B, g.d)
    f = _forced(force_idx, (g.B, k))
    th = np.ascontiguousarray(thresh, dtype=np.float64)
    J = ctypes.c_double()
    rc = _load().oracle_objective(g.B, g.d, h, g.n, k, *g.args(), int(train), float(noise_floor),
                                  _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), e_dt,
                                  float(w_importance), float(w_load), dy.ctypes.data,
                                  float(aux_scale), _ptr(f), th.ctypes.data, ctypes.byref(J))
    _check(rc, "objective")
    return J.value


def backward(inp: Dict[str, np.ndarray], k: int, dy, aux_scale: float = 1.0, train: bool = True,
             noise_floor: float = 1e-2, w_importance: float = 0.1, w_load: float = 0.1,
             force_idx=None, decide_fp32: bool = True) -> Dict[str, np.ndarray]:
    """Gradients of sum dy . y + aux_scale * (weighted losses) with respect to
    x, the gate parameters and the expert parameters (fp64), the selection
    (the oracle's own, or force_idx [B, k]) and eq 9's thresholds held fixed.
    Returns dx [B, d], dw_gate / dw_noise [n, d], dgate_bias [n], dw1 [n, h, d],
    db1 [n, h], dw2 [n, d, h], db2 [n, d]."""
    g = _Gate(inp, train)
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    B, d, n = g.B, g.d, g.n
    dy = _dy(dy, B, d)
    f = _forced(force_idx, (B, k))
    out = {"dx": np.empty((B, d)), "dw_gate": np.empty((n, d)), "dw_noise": np.empty((n, d)),
           "dgate_bias": np.empty(n), "dw1": np.empty((n, h, d)), "db1": np.empty((n, h)),
           "dw2": np.empty((n, d, h)), "db2": np.empty((n, d))}
    rc = _load().oracle_backward(B, d, h, n, k, *g.args(), int(train), float(noise_floor),
                                 int(decide_fp32), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), e_dt,
                                 float(w_importance), float(w_load), dy.ctypes.data,
                                 float(aux_scale), _ptr(f),
                                 *[out[key].ctypes.data for key in (
                                     "dx", "dw_gate", "dw_noise", "dgate_bias", "dw1", "db1",
                                     "dw2", "db2")])
    _check(rc, "backward")
    return out


def backward_sampled(inp: Dict[str, np.ndarray], k: int, dy, gate_experts=(), experts=(),
                     tokens=(), aux_scale: float = 1.0, train: bool = True,
                     noise_floor: float = 1e-2, w_importance: float = 0.1, w_load: float = 0.1,
                     force_idx=None, decide_fp32: bool = True) -> Dict[str, np.ndarray]:
    """The gradients of ``backward`` for a few experts and tokens (fp64), for
    batches too large for the whole backward: dw_gate / dw_noise [len(gate_experts), d]
    and dgate_bias [len(gate_experts)] for the listed gate experts; dw1 [ne, h, d],
    db1 [ne, h], dw2 [ne, d, h], db2 [ne, d] for the listed experts; dx [nt, d] for
    the listed tokens. Importance and Load are still taken over the whole batch."""
    g = _Gate(inp, train)
    w1, b1, w2, b2, e_dt, h = _experts(inp)
    B, d, n = g.B, g.d, g.n
    dy = _dy(dy, B, d)
    f = _forced(force_idx, (B, k))
    ge = np.ascontiguousarray(gate_experts, dtype=np.int32)
    ee = np.ascontiguousarray(experts, dtype=np.int32)
    tt = np.ascontiguousarray(tokens, dtype=np.int64)
    ng, ne, nt = ge.size, ee.size, tt.size
    out = {"dw_gate": np.empty((ng, d)), "dw_noise": np.empty((ng, d)),
           "dgate_bias": np.empty(ng), "dw1": np.empty((ne, h, d)), "db1": np.empty((ne, h)),
           "dw2": np.empty((ne, d, h)), "db2": np.empty((ne, d)), "dx": np.empty((nt, d))}
    rc = _load().oracle_backward_sampled(
        B, d, h, n, k, *g.args(), int(train), float(noise_floor), int(decide_fp32), _ptr(w1),
        _ptr(b1), _ptr(w2), _ptr(b2), e_dt, float(w_importance), float(w_load), dy.ctypes.data,
        float(aux_scale), _ptr(f),
        ng, ge.ctypes.data, out["dw_gate"].ctypes.data, out["dw_noise"].ctypes.data,
        out["dgate_bias"].ctypes.data,
        ne, ee.ctypes.data, out["dw1"].ctypes.data, out["db1"].ctypes.data,
        out["dw2"].ctypes.data, out["db2"].ctypes.data,
        nt, tt.ctypes.data, out["dx"].ctypes.data)
    _check(rc, "backward_sampled")
    return out


# ---------------------------------------------------------------------------
# Hierarchical MoE (section "Hierarchical MoE"; eq 12 read from its prose)
# ---------------------------------------------------------------------------

class _HierGate:
    """Arguments of both gate levels: ``w_gate``/``w_noise`` [a, d], ``eps`` [B, a],
    ``w_gate2``/``w_noise2`` [a, b, d], ``eps2`` [B, k1, b]."""

    def __init__(self, inp: Dict[str, np.ndarray], k1: int, k2: int, train: bool):
        self.x, self.x_dt = _arr(inp["x"])
        self.wg1, self.w_dt = _arr(inp["w_gate"])
        self.wn1, _ = _arr(inp["w_noise"])
        self.wg2, w2_dt = _arr(inp["w_gate2"])
        self.wn2, _ = _arr(inp["w_noise2"])
        if w2_dt != self.w_dt:
            raise ValueError("both gate levels must share a dtype")
        self.B, self.d = self.x.shape
        self.a, self.b = self.wg2.shape[0], self.wg2.shape[1]
        if self.wg1.shape != (self.a, self.d) or self.wg2.shape != (self.a, self.b, self.d):
            raise ValueError("gate weights must be [a, d] and [a, b, d]")
        self.k1, self.k2 = k1, k2
        self.eps1 = np.ascontiguousarray(inp["eps"], dtype=np.float32) if train else None
        self.eps2 = np.ascontiguousarray(inp["eps2"], dtype=np.float32) if train else None
        if train and (self.eps1.shape != (self.B, self.a) or
                      self.eps2.shape != (self.B, k1, self.b)):
            raise ValueError("eps must be [B, a] and eps2 [B, k1, b]")

    def args(self):
        return (_ptr(self.x), self.x_dt, _ptr(self.wg1), _ptr(self.wn1), _ptr(self.wg2),
                _ptr(self.wn2), self.w_dt, _ptr(self.eps1), _ptr(self.eps2))


def _forced(f, shape):
    if f is None:
        return None
    f = np.ascontiguousarray(f, dtype=np.int32)
    if f.shape != shape:
        raise ValueError(f"forced selection must have shape {shape}")
    return f


def hier_gate(inp: Dict[str, np.ndarray], k1: int, k2: int, rows: Optional[Sequence[int]] = None,
              train: bool = True, noise_floor: float = 1e-2, decide_fp32: bool = True,
              force1=None, force2=None, want_logits: bool = False) -> Dict[str, np.ndarray]:
    """Both gate levels on token rows ``rows`` (default all).

    Returns sel1/gate1 [R, k1], thr1 [R, 2]; sel2/gate2 [R, k1, k2] (expert index within
    the group), thr2 [R, k1, 2]; leaf_idx/leaf_gate [R, k1*k2] in slot order (r, j);
    with ``want_logits`` also H1 [R, a] and H2 [R, k1, b]. ``force1`` [R, k1] and
    ``force2`` [R, k1, k2] replace the selections (e.g. another valid choice on a near-tie row).
    """
    g = _HierGate(inp, k1, k2, train)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = g.B if rows_a is None else rows_a.size
    K = k1 * k2
    f1 = _forced(force1, (R, k1))
    f2 = _forced(force2, (R, k1, k2))
    out = {"sel1": np.empty((R, k1), np.int32), "gate1": np.empty((R, k1)),
           "thr1": np.empty((R, 2)), "sel2": np.empty((R, k1, k2), np.int32),
           "gate2": np.empty((R, k1, k2)), "thr2": np.empty((R, k1, 2)),
           "leaf_idx": np.empty((R, K), np.int32), "leaf_gate": np.empty((R, K))}
    if want_logits:
        out["H1"] = np.empty((R, g.a))
        out["H2"] = np.empty((R, k1, g.b))
    rc = _load().oracle_hier_gate(
        R, _ptr(rows_a), g.d, g.a, g.b, k1, k2, *g.args(), int(train), float(noise_floor),
        int(decide_fp32), _ptr(f1), _ptr(f2), *[_ptr(out.get(key)) for key in (
            "sel1", "gate1", "thr1", "H1", "sel2", "gate2", "thr2", "H2", "leaf_idx",
            "leaf_gate")])
    _check(rc, "hier_gate")
    return out


def hier_forward(inp: Dict[str, np.ndarray], k1: int, k2: int, train: bool = True,
                 noise_floor: float = 1e-2, w_importance: float = 0.1, w_load: float = 0.1,
                 decide_fp32: bool = True, force1=None, force2=None,
                 with_y: bool = True) -> Dict[str, np.ndarray]:
    """The hierarchical layer's forward pass on the whole batch.

    Returns y [B, d], leaf_idx/leaf_gate [B, k1*k2], imp1/load1/rows1 [a], load2 [a*b],
    importance/load [a*b] (leaf) and losses [3]. ``with_y=False`` skips the
    experts (no y; ``inp`` then needs no expert weights).
    """
    g = _HierGate(inp, k1, k2, train)
    if with_y:
        w1, b1, w2, b2, e_dt, h = _experts(inp)
    else:
        w1 = b1 = w2 = b2 = None
        e_dt, h = 0, 0
    n = g.a * g.b
    K = k1 * k2
    f1 = _forced(force1, (g.B, k1))
    f2 = _forced(force2, (g.B, k1, k2))
    out = {"y": np.empty((g.B, g.d)) if with_y else None,
           "leaf_idx": np.empty((g.B, K), np.int32),
           "leaf_gate": np.empty((g.B, K)), "imp1": np.empty(g.a), "load1": np.empty(g.a),
           "rows1": np.empty(g.a), "load2": np.empty(n), "importance": np.empty(n),
           "load": np.empty(n), "losses": np.empty(3)}
    rc = _load().oracle_hier_forward(
        g.B, g.d, h, g.a, g.b, k1, k2, *g.args(), int(train), float(noise_floor),
        int(decide_fp32), _ptr(f1), _ptr(f2), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), e_dt,
        float(w_importance), float(w_load),
        *[_ptr(out[key]) for key in ("y", "leaf_idx", "leaf_gate", "imp1", "load1",
                                     "rows1", "load2", "importance", "load", "losses")])
    _check(rc, "hier_forward")
    if not with_y:
        del out["y"]
    return out


# ---------------------------------------------------------------------------
# Batchwise gating ([MoE-explainer] "What the paper measured": the gate of the
# single-pair translation models, the paper's Appendix F)
# ---------------------------------------------------------------------------

def batchwise_select(S, m: int, threshold=None):
    """Column-wise choice of batchwise gating on a score matrix S [B, n].

    Expert i takes the rows t with S[t, i] > threshold[i] (every row when
    ``threshold`` is None), at most m of them: the m largest scores, ties to
    the lower row. The pages' training rule is threshold None with
    m = k B / n (each expert gets the same batch size); their inference rule
    is a learned per-expert threshold, here with m as a cap (m = B: none).
    Returns (counts [n] int32, keep [B, n] bool)."""
    S = np.asarray(S, dtype=np.float64)
    B, n = S.shape
    thr = np.full(n, -np.inf) if threshold is None else np.asarray(threshold, np.float64)
    keep = np.zeros((B, n), bool)
    for i in range(n):
        col = S[:, i]
        cand = np.flatnonzero(col > thr[i])
        if cand.size > m:
            # descending score; the stable sort keeps equal scores in row order
            order = np.argsort(-col[cand], kind="stable")
            cand = cand[order[:m]]
        keep[cand, i] = True
    return keep.sum(axis=0).astype(np.int32), keep


def batchwise_gates(S, keep) -> np.ndarray:
    """Gates of batchwise gating: each row's softmax over its kept scores (the
    softmax eq 3 applies to the kept logits), 0 elsewhere; a row that no
    expert took has no gates."""
    S = np.asarray(S, dtype=np.float64)
    G = np.zeros(S.shape)
    for t in range(S.shape[0]):
        idx = np.flatnonzero(keep[t])
        if idx.size:
            v = S[t, idx]
            e = np.exp(v - v.max())
            G[t, idx] = e / e.sum()
    return G


def batchwise_forward(inp: Dict[str, np.ndarray], m: int, train: bool = True,
                      noise_floor: float = 1e-2, threshold=None, decide_fp32: bool = True,
                      keep=None) -> Dict[str, np.ndarray]:
    """Forward pass with batchwise gating on the whole batch.

    The scores are H of eq 4 (noise included when ``train``), computed by
    ``gate``; the choice is ``batchwise_select`` on the scores rounded to fp32
    when ``decide_fp32`` (the precision the kernels decide in); the gates use
    the fp64 scores. y[t] = sum_i G[t, i] E_i(x[t]) (eq 1). ``keep`` [B, n]
    replaces the choice (e.g. another valid one on a near-tie column).
    Returns y, H, keep, counts, G, importance (= G.sum(0)), load (= counts)
    and losses [CV^2(importance), CV^2(load)]."""
    g = gate(inp, 1, train=train, noise_floor=noise_floor, want_logits=True)
    H = g["H"]
    if keep is None:
        Sd = H.astype(np.float32).astype(np.float64) if decide_fp32 else H
        thr = None if threshold is None else np.asarray(threshold, np.float32).astype(np.float64)
        counts, keep = batchwise_select(Sd, m, thr)
    else:
        keep = np.asarray(keep, bool)
        counts = keep.sum(axis=0).astype(np.int32)
    G = batchwise_gates(H, keep)
    B = H.shape[0]
    d = np.asarray(inp["x"]).shape[1]
    y = np.zeros((B, d))
    tok, exp_ = np.nonzero(keep)
    if tok.size:
        E = expert_pairs(inp, tok, exp_.astype(np.int32))
        for r in range(tok.size):
            y[tok[r]] += G[tok[r], exp_[r]] * E[r]
    imp = G.sum(axis=0)
    load = counts.astype(np.float64)
    return {"y": y, "H": H, "keep": keep, "counts": counts, "G": G, "importance": imp,
            "load": load, "losses": np.array([cv2(imp), cv2(load)])}


def _widen(a) -> np.ndarray:
    """Storage arrays (float32, or bf16 as uint16 bit patterns) as float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def score_columns(inp: Dict[str, np.ndarray], experts: Sequence[int], train: bool = True,
                  noise_floor: float = 1e-2) -> np.ndarray:
    """H of eq 4 for every row of the batch and the listed experts only
    ([B, len(experts)], fp64): clean = x . W_g[e] + b_e, sigma =
    Softplus(x . W_noise[e]) + floor, H = clean + eps[:, e] * sigma (train)."""
    e = np.asarray(experts, dtype=np.int64)
    x = _widen(inp["x"])
    clean = x @ _widen(inp["w_gate"])[e].T
    if inp.get("gate_bias") is not None:
        clean = clean + np.asarray(inp["gate_bias"], np.float64)[e]
    if not train:
        return clean
    u = x @ _widen(inp["w_noise"])[e].T
    sigma = np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u))) + noise_floor
    return clean + np.asarray(inp["eps"], np.float64)[:, e] * sigma
