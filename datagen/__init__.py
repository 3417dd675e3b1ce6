"""Seeded synthetic workloads for the sparsely-gated MoE forward pass.

This module is the only code shared by the oracle side and the GPU side: it
turns (workload, seed, tensor id, element range) into the input arrays, and
holds none of the method's arithmetic.  Draws come from Philox4x32-10 with a
Box-Muller transform (``philox_normal.c``), so any slice of any tensor can be
regenerated on its own (the hierarchical workload's 34 GB of expert weights is
regenerated per expert instead of being held).

Storage layouts (row-major, contiguous):

* ``x``      [B, d]        tokens (all positions of all sequences, flattened)
* ``w_gate`` [n, d]        row i holds expert i's clean-logit weights (the
                           pages' W_g is d x n; this is its transpose)
* ``w_noise``[n, d]        same for the noise-scale weights W_noise
* ``gate_bias`` [n]        optional additive bias on the clean logits
* ``eps``    [B, n]        the standard-normal noise draws, passed in
* ``w1``     [n, h, d]     expert input layer, row j = hidden unit j
* ``b1``     [n, h]
* ``w2``     [n, d, h]     expert output layer, row c = output unit c
* ``b2``     [n, d]

bf16 arrays are returned as ``numpy.uint16`` holding round-to-nearest-even
bf16 bit patterns; fp32 arrays as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_normal.c")
_LIB_PATH = os.path.join(_HERE, "libmoedatagen.so")
_lib = None

F32 = 0
BF16 = 1

# Tensor ids: the third Philox counter word.
TID = {
    "x": 1, "w_gate": 2, "w_noise": 3, "eps": 4, "w1": 5, "b1": 6, "w2": 7, "b2": 8,
    "w_gate2": 9, "w_noise2": 10, "eps2": 11,
}


def build(force: bool = True) -> str:
    """Compile the generator with gcc/OpenMP into ``libmoedatagen.so``."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.dg_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.dg_philox4x32_10.restype = None
        lib.dg_normal.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                  ctypes.c_uint64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.dg_normal.restype = ctypes.c_int
        lib.dg_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
        lib.dg_f32_to_bf16.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib.dg_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def normal(seed: int, tid: int, offset: int, count: int, scale: float = 1.0,
           dtype: int = F32) -> np.ndarray:
    """Draws ``scale * z[e]`` for e in [offset, offset + count) of tensor ``tid``."""
    lib = _load()
    out = np.empty(count, dtype=np.float32 if dtype == F32 else np.uint16)
    if count:
        rc = lib.dg_normal(seed, tid, offset, count, float(scale), dtype, out.ctypes.data)
        if rc != 0:
            raise ValueError("bad dtype")
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        _load().dg_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact bf16 (uint16 bit patterns) -> fp32 widening."""
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """fp32 view of an array that is either fp32 or bf16 bit patterns."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """Shape, storage types and input recipe of one synthetic workload."""
    name: str
    seed: int
    tokens: int
    d_model: int
    d_hidden: int
    n_experts: int
    k: int
    act_dtype: int = F32      # x, expert outputs, y
    expert_dtype: int = F32   # w1, b1, w2, b2
    gate_dtype: int = F32     # w_gate, w_noise
    noise_scale: float = 1.0  # multiplier on w_noise's N(0, 1/d) draws
    zipf: bool = False        # add the calibrated Zipf gate bias
    # hierarchical workloads only: groups a (= n_experts of level 1), experts b per group
    groups: int = 0
    group_experts: int = 0
    k1: int = 0
    k2: int = 0
    description: str = ""

    @property
    def hierarchical(self) -> bool:
        return self.groups > 0


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32", 1, 256, 64, 128, 16, 2,
        description="256 tokens, d 64, 16 experts 64-128-64, k 2, fp32"),
    "flat_fp32_n32": Workload(
        "flat_fp32_n32", 2, 8192, 512, 1024, 32, 4, noise_scale=0.1,
        description="8192 tokens, d 512, 32 experts 512-1024-512, k 4, fp32, W_noise x0.1"),
    "zipf_bf16_n256": Workload(
        "zipf_bf16_n256", 3, 32768, 512, 1024, 256, 4, act_dtype=BF16, expert_dtype=BF16,
        gate_dtype=F32, zipf=True,
        description="32768 tokens, d 512, 256 experts 512-1024-512, k 4, bf16 act/experts, "
                    "fp32 gate weights, Zipf(1.0) expert popularity via gate bias"),
    "flat_bf16_n4096": Workload(
        "flat_bf16_n4096", 4, 65536, 512, 1024, 4096, 4, act_dtype=BF16, expert_dtype=BF16,
        gate_dtype=BF16,
        description="65536 tokens, d 512, 4096 experts 512-1024-512 (4.3B expert params), "
                    "k 4, bf16"),
    "hier_bf16_16384": Workload(
        "hier_bf16_16384", 5, 131072, 512, 1024, 16384, 4, act_dtype=BF16, expert_dtype=BF16,
        gate_dtype=BF16, groups=128, group_experts=128, k1=2, k2=2,
        description="131072 tokens, d 512, 128 groups x 128 experts (16384 leaves), "
                    "k1 = k2 = 2, bf16"),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields overridden (e.g. tokens=...)."""
    return replace(WORKLOADS[name], **overrides)


_ZIPF_JSON = os.path.join(_HERE, "zipf_tau.json")


def zipf_tau() -> float:
    """Calibrated Zipf scale of the gate bias (written by tests/golden/calibrate_zipf_tau.py)."""
    with open(_ZIPF_JSON) as f:
        return float(json.load(f)["tau"])


def gate_bias(w: Workload, tau: Optional[float] = None) -> Optional[np.ndarray]:
    """Gate bias b[e] = -tau * ln(e + 1): expert e's prior popularity falls with its rank."""
    if not w.zipf:
        return None
    t = zipf_tau() if tau is None else tau
    return (-t * np.log(np.arange(1, w.n_experts + 1, dtype=np.float64))).astype(np.float32)


def gen(w: Workload, name: str, offset: int = 0, count: Optional[int] = None) -> np.ndarray:
    """Flat slice [offset, offset + count) of input tensor ``name`` of workload ``w``."""
    d, h, n = w.d_model, w.d_hidden, w.n_experts
    if w.hierarchical:
        a, b = w.groups, w.group_experts
        sizes = {"x": w.tokens * d, "w_gate": a * d, "w_noise": a * d, "eps": w.tokens * a,
                 "w_gate2": a * b * d, "w_noise2": a * b * d, "eps2": w.tokens * w.k1 * b,
                 "w1": n * h * d, "b1": n * h, "w2": n * d * h, "b2": n * d}
    else:
        sizes = {"x": w.tokens * d, "w_gate": n * d, "w_noise": n * d, "eps": w.tokens * n,
                 "w1": n * h * d, "b1": n * h, "w2": n * d * h, "b2": n * d}
    total = sizes[name]
    if count is None:
        count = total - offset
    if offset < 0 or offset + count > total:
        raise ValueError(f"{name}: slice [{offset}, {offset + count}) outside [0, {total})")
    scale = {
        "x": 1.0, "eps": 1.0, "eps2": 1.0,
        "w_gate": 1.0 / math.sqrt(d), "w_noise": w.noise_scale / math.sqrt(d),
        "w_gate2": 1.0 / math.sqrt(d), "w_noise2": w.noise_scale / math.sqrt(d),
        "w1": 1.0 / math.sqrt(d), "b1": 1.0 / math.sqrt(d),
        "w2": 1.0 / math.sqrt(h), "b2": 1.0 / math.sqrt(h),
    }[name]
    dtype = {
        "x": w.act_dtype, "eps": F32, "eps2": F32,
        "w_gate": w.gate_dtype, "w_noise": w.gate_dtype,
        "w_gate2": w.gate_dtype, "w_noise2": w.gate_dtype,
        "w1": w.expert_dtype, "b1": w.expert_dtype, "w2": w.expert_dtype, "b2": w.expert_dtype,
    }[name]
    return normal(w.seed, TID[name], offset, count, scale, dtype)


def make_inputs(w: Workload, with_bias: bool = False, experts: bool = True,
                gate_bias_tau: Optional[float] = None) -> Dict[str, np.ndarray]:
    """All inputs of a flat workload as shaped numpy arrays.

    ``with_bias`` adds the expert biases b1/b2 (otherwise they are absent).
    ``experts=False`` skips the expert weights (for gating-only uses).
    ``gate_bias_tau`` overrides the stored Zipf scale (used when calibrating it).
    """
    if w.hierarchical:
        raise ValueError("use make_hier_inputs for hierarchical workloads")
    B, d, h, n = w.tokens, w.d_model, w.d_hidden, w.n_experts
    out = {
        "x": gen(w, "x").reshape(B, d),
        "w_gate": gen(w, "w_gate").reshape(n, d),
        "w_noise": gen(w, "w_noise").reshape(n, d),
        "eps": gen(w, "eps").reshape(B, n),
    }
    bg = gate_bias(w, gate_bias_tau)
    if bg is not None:
        out["gate_bias"] = bg
    if experts:
        out["w1"] = gen(w, "w1").reshape(n, h, d)
        out["w2"] = gen(w, "w2").reshape(n, d, h)
        if with_bias:
            out["b1"] = gen(w, "b1").reshape(n, h)
            out["b2"] = gen(w, "b2").reshape(n, d)
    return out


def make_hier_inputs(w: Workload, with_bias: bool = False, experts: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of a hierarchical workload.

    Level 1: ``w_gate``/``w_noise`` [a, d], ``eps`` [B, a].
    Level 2: ``w_gate2``/``w_noise2`` [a, b, d], ``eps2`` [B, k1, b] indexed by the
    token's level-1 rank r (the r-th selected group draws eps2[t, r, :]).
    Experts: leaf i*b + j, ``w1`` [a*b, h, d], ``w2`` [a*b, d, h].
    """
    if not w.hierarchical:
        raise ValueError("not a hierarchical workload")
    B, d, h = w.tokens, w.d_model, w.d_hidden
    a, b = w.groups, w.group_experts
    out = {
        "x": gen(w, "x").reshape(B, d),
        "w_gate": gen(w, "w_gate").reshape(a, d),
        "w_noise": gen(w, "w_noise").reshape(a, d),
        "eps": gen(w, "eps").reshape(B, a),
        "w_gate2": gen(w, "w_gate2").reshape(a, b, d),
        "w_noise2": gen(w, "w_noise2").reshape(a, b, d),
        "eps2": gen(w, "eps2").reshape(B, w.k1, b),
    }
    if experts:
        n = a * b
        out["w1"] = gen(w, "w1").reshape(n, h, d)
        out["w2"] = gen(w, "w2").reshape(n, d, h)
        if with_bias:
            out["b1"] = gen(w, "b1").reshape(n, h)
            out["b2"] = gen(w, "b2").reshape(n, d)
    return out
