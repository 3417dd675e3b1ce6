"""ctypes binding of ``libmoe_mi355x.so`` (the C ABI of include/moe.h).

Argument marshalling only: every entry point checks tensor dtypes, shapes,
devices and contiguity, passes raw device pointers and torch's current HIP
stream to the library, and raises ``MoeError`` with the library's message on a
nonzero status. All computation happens in the library's HIP kernels; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_F32 = 0
MOE_BF16 = 1


class MoeError(RuntimeError):
    pass


class MoeDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("d_hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("k", ctypes.c_int32),
                ("act_dtype", ctypes.c_int), ("expert_dtype", ctypes.c_int),
                ("gate_dtype", ctypes.c_int), ("capacity", ctypes.c_int32),
                ("expert_layout", ctypes.c_int32)]


class MoeGateOpts(ctypes.Structure):
    _fields_ = [("train", ctypes.c_int32), ("noise_floor", ctypes.c_float),
                ("w_importance", ctypes.c_float), ("w_load", ctypes.c_float),
                ("gate_order", ctypes.c_int32)]


class MoeHierDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("d_hidden", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("group_experts", ctypes.c_int32), ("k1", ctypes.c_int32), ("k2", ctypes.c_int32),
                ("act_dtype", ctypes.c_int), ("expert_dtype", ctypes.c_int),
                ("gate_dtype", ctypes.c_int), ("expert_layout", ctypes.c_int32)]


_HIER_OUT_FIELDS = ("topk_idx", "topk_gate", "counts", "group_idx", "group_gate", "group_thresh",
                    "group_rows", "group_importance", "group_load", "sub_idx", "sub_gate",
                    "sub_thresh", "sub_load")


class MoeHierOutputs(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in _HIER_OUT_FIELDS]


_P = ctypes.c_void_p
_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparsely_gated_mixture_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDims), ctypes.POINTER(MoeGateOpts)]
        L.moe_workspace_size.restype = ctypes.c_size_t
        D, O = ctypes.POINTER(MoeDims), ctypes.POINTER(MoeGateOpts)
        S = ctypes.c_size_t
        L.moe_gate.argtypes = [D, O, _P, _P, _P, _P, _P, _P, _P, _P, _P, S, _P]
        L.moe_route.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, S, _P]
        L.moe_expert_ffn.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, S, _P]
        L.moe_pack_expert_weights.argtypes = [D, _P, _P, _P, _P, _P]
        L.moe_combine.argtypes = [D, _P, _P, _P, _P, _P]
        L.moe_aux_losses.argtypes = [D, O, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, S, _P]
        L.moe_forward.argtypes = [D, O] + [_P] * 19 + [S, _P]
        L.moe_forward_noalloc.argtypes = [D, O] + [_P] * 18 + [_P]
        L.moe_backward_workspace_size.argtypes = [D, O]
        L.moe_backward_workspace_size.restype = ctypes.c_size_t
        L.moe_backward.argtypes = [D, O] + [_P] * 15 + [ctypes.c_float] + [_P] * 9 + [S, _P]
        HD = ctypes.POINTER(MoeHierDims)
        L.moe_hier_workspace_size.argtypes = [HD, O]
        L.moe_hier_workspace_size.restype = ctypes.c_size_t
        L.moe_hier_forward.argtypes = ([HD, O] + [_P] * 15 + [ctypes.POINTER(MoeHierOutputs), _P, S,
                                                              _P])
        L.moe_batchwise_workspace_size.argtypes = [D, O, ctypes.c_int32]
        L.moe_batchwise_workspace_size.restype = ctypes.c_size_t
        L.moe_batchwise_forward.argtypes = [D, O, ctypes.c_int32] + [_P] * 19 + [S, _P]
        L.moe_ffn_timing.argtypes = [ctypes.c_int]
        L.moe_ffn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double)]
        for f in ("moe_gate", "moe_route", "moe_expert_ffn", "moe_combine", "moe_aux_losses",
                  "moe_forward", "moe_forward_noalloc", "moe_backward", "moe_hier_forward",
                  "moe_batchwise_forward", "moe_ffn_timing",
                  "moe_ffn_timing_read"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise MoeError(f"{what}: {L.moe_status_string(status).decode()}: "
                       f"{L.moe_last_error().decode()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoeError(f"unsupported dtype {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise MoeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise MoeError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_ffn_timing(enable: bool) -> None:
    """Start (clearing the record) or stop timing the expert-FFN kernel of
    forward calls on the current device."""
    _check(lib().moe_ffn_timing(1 if enable else 0), "moe_ffn_timing")


def moe_ffn_timing_read() -> Tuple[int, float]:
    """(timed expert-FFN kernels, their summed duration in ms); waits for them."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().moe_ffn_timing_read(ctypes.byref(n), ctypes.byref(ms)), "moe_ffn_timing_read")
    return int(n.value), float(ms.value)


def make_dims(tokens: int, d_model: int, d_hidden: int, n_experts: int, k: int,
              act_dtype: int, expert_dtype: int, gate_dtype: int, capacity: int = 0,
              expert_layout: int = 0) -> MoeDims:
    return MoeDims(tokens, d_model, d_hidden, n_experts, k, act_dtype, expert_dtype, gate_dtype,
                   capacity, expert_layout)


def moe_pack_expert_weights(w1, w2, stream=None):
    """(w1_packed, w2_packed): w1 [n, h, d] and w2 [n, d, h] in the packed operand layout
    (expert_layout=1 of moe_expert_ffn / moe_forward); same shapes, dtypes and bytes, the
    elements reordered."""
    _dev(w1, "w1")
    n, h, d = w1.shape
    _dev(w2, "w2", w1.dtype, (n, d, h))
    dims = make_dims(0, d, h, n, 1, _dt(w1), _dt(w1), _dt(w1))
    w1p = torch.empty_like(w1)
    w2p = torch.empty_like(w2)
    st = lib().moe_pack_expert_weights(ctypes.byref(dims), _ptr(w1), _ptr(w2), _ptr(w1p),
                                       _ptr(w2p), _stream(stream))
    _check(st, "moe_pack_expert_weights")
    return w1p, w2p


def make_opts(train: bool = True, noise_floor: float = 1e-2, w_importance: float = 0.1,
              w_load: float = 0.1, gate_order: int = 0) -> MoeGateOpts:
    return MoeGateOpts(int(bool(train)), noise_floor, w_importance, w_load, int(gate_order))


def moe_workspace_size(dims: MoeDims, opts: Optional[MoeGateOpts] = None) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(dims),
                                        ctypes.byref(opts) if opts is not None else None))


def workspace(dims: MoeDims, opts: Optional[MoeGateOpts], device) -> torch.Tensor:
    """A device byte buffer of moe_workspace_size() bytes (torch's allocator
    returns 512-byte aligned blocks)."""
    nbytes = moe_workspace_size(dims, opts)
    if nbytes == 0 and dims.tokens > 0:
        _check(1, "moe_workspace_size")
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _gate_dims(x, w_gate, k, d_hidden=128, w1=None) -> MoeDims:
    B, d = x.shape
    n = w_gate.shape[0]
    e_dt = _dt(w1) if w1 is not None else _dt(x)
    return make_dims(B, d, d_hidden if w1 is None else w1.shape[1], n, k, _dt(x), e_dt, _dt(w_gate))


def moe_gate(x, w_gate, w_noise, eps, k: int, *, train: bool = True, noise_floor: float = 1e-2,
             gate_bias=None, ws: Optional[torch.Tensor] = None, gate_order: int = 0,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Noisy top-k gating -> (topk_idx [B,k] int32, topk_gate [B,k] fp32, thresh [B,2] fp32).
    ws (optional, moe_workspace_size bytes) lets a small batch split its expert sweep."""
    _dev(x, "x")
    B, d = x.shape
    _dev(w_gate, "w_gate")
    n = w_gate.shape[0]
    _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
    _dev(gate_bias, "gate_bias", torch.float32, (n,))
    _dev(eps, "eps", torch.float32, (B, n))
    dims = _gate_dims(x, w_gate, k)
    opts = make_opts(train, noise_floor, gate_order=gate_order)
    dev = x.device
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    gate = torch.empty((B, k), dtype=torch.float32, device=dev)
    thr = torch.empty((B, 2), dtype=torch.float32, device=dev)
    st = lib().moe_gate(ctypes.byref(dims), ctypes.byref(opts), _ptr(x), _ptr(w_gate),
                        _ptr(w_noise), _ptr(gate_bias), _ptr(eps), _ptr(idx), _ptr(gate), _ptr(thr),
                        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "moe_gate")
    return idx, gate, thr


def moe_route(topk_idx, topk_gate, n_experts: int, *, d_model: int = 64,
              ws: Optional[torch.Tensor] = None, with_importance: bool = True, capacity: int = 0,
              stream=None) -> Dict[str, torch.Tensor]:
    """Stable expert-major routing: counts, offsets, perm_token, perm_gate, slot_pos, importance.
    capacity > 0: slots past the first `capacity` rows of their expert get slot_pos -1."""
    _dev(topk_idx, "topk_idx", torch.int32)
    B, k = topk_idx.shape
    _dev(topk_gate, "topk_gate", torch.float32, (B, k))
    dims = make_dims(B, d_model, 128, n_experts, k, MOE_F32, MOE_F32, MOE_F32, capacity)
    dev = topk_idx.device
    if ws is None:
        ws = workspace(dims, None, dev)
    out = {"counts": torch.empty(n_experts, dtype=torch.int32, device=dev),
           "offsets": torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
           "perm_token": torch.empty(B * k, dtype=torch.int32, device=dev),
           "perm_gate": torch.empty(B * k, dtype=torch.float32, device=dev),
           "slot_pos": torch.empty(B * k, dtype=torch.int32, device=dev)}
    if with_importance:
        out["importance"] = torch.empty(n_experts, dtype=torch.float32, device=dev)
    st = lib().moe_route(ctypes.byref(dims), _ptr(topk_idx), _ptr(topk_gate), _ptr(out["counts"]),
                         _ptr(out["offsets"]), _ptr(out["perm_token"]), _ptr(out["perm_gate"]),
                         _ptr(out["slot_pos"]), _ptr(out.get("importance")), _ptr(ws), ws.numel(),
                         _stream(stream))
    _check(st, "moe_route")
    return out


def moe_expert_ffn(x, offsets, perm_token, w1, w2, k: int, *, b1=None, b2=None,
                   ws: Optional[torch.Tensor] = None, out=None, capacity: int = 0,
                   expert_layout: int = 0, stream=None) -> torch.Tensor:
    """expert_out [B*k, d] in permutation order: E_e(x[perm_token[p]]) per segment (with
    capacity > 0 only the first `capacity` rows of each segment are computed; with
    expert_layout=1, w1 and w2 come from moe_pack_expert_weights)."""
    _dev(x, "x")
    B, d = x.shape
    _dev(w1, "w1", x.dtype)
    n, h, _ = w1.shape
    _dev(w2, "w2", x.dtype, (n, d, h))
    _dev(b1, "b1", x.dtype, (n, h))
    _dev(b2, "b2", x.dtype, (n, d))
    _dev(offsets, "offsets", torch.int32, (n + 1,))
    _dev(perm_token, "perm_token", torch.int32, (B * k,))
    dims = make_dims(B, d, h, n, k, _dt(x), _dt(w1), _dt(x), capacity, expert_layout)
    if ws is None:
        ws = workspace(dims, None, x.device)
    if out is None:
        out = torch.empty((B * k, d), dtype=x.dtype, device=x.device)
    _dev(out, "expert_out", x.dtype, (B * k, d))
    st = lib().moe_expert_ffn(ctypes.byref(dims), _ptr(x), _ptr(offsets), _ptr(perm_token),
                              _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out), _ptr(ws),
                              ws.numel(), _stream(stream))
    _check(st, "moe_expert_ffn")
    return out


def moe_combine(expert_out, slot_pos, topk_gate, *, n_experts: int = 1, out=None,
                stream=None) -> torch.Tensor:
    """y [B, d] = sum_j topk_gate[t, j] * expert_out[slot_pos[t*k + j]]."""
    _dev(topk_gate, "topk_gate", torch.float32)
    B, k = topk_gate.shape
    _dev(expert_out, "expert_out")
    d = expert_out.shape[1]
    _dev(slot_pos, "slot_pos", torch.int32, (B * k,))
    dims = make_dims(B, d, 128, max(n_experts, k), k, _dt(expert_out), _dt(expert_out),
                     _dt(expert_out))
    if out is None:
        out = torch.empty((B, d), dtype=expert_out.dtype, device=expert_out.device)
    _dev(out, "y", expert_out.dtype, (B, d))
    st = lib().moe_combine(ctypes.byref(dims), _ptr(expert_out), _ptr(slot_pos), _ptr(topk_gate),
                           _ptr(out), _stream(stream))
    _check(st, "moe_combine")
    return out


def moe_aux_losses(x, w_gate, w_noise, thresh, offsets, perm_token, importance, k: int, *,
                   train: bool = True, noise_floor: float = 1e-2, w_importance: float = 0.1,
                   w_load: float = 0.1, gate_bias=None, ws: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(load [n], losses [3] = CV2(imp), CV2(load), weighted sum). ``thresh`` comes from
    moe_gate; ``offsets``, ``perm_token`` and ``importance`` from moe_route of its selection."""
    _dev(x, "x")
    B, d = x.shape
    _dev(w_gate, "w_gate")
    n = w_gate.shape[0]
    _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
    _dev(gate_bias, "gate_bias", torch.float32, (n,))
    _dev(thresh, "thresh", torch.float32, (B, 2))
    _dev(offsets, "offsets", torch.int32, (n + 1,))
    _dev(perm_token, "perm_token", torch.int32, (B * k,))
    _dev(importance, "importance", torch.float32, (n,))
    dims = _gate_dims(x, w_gate, k)
    opts = make_opts(train, noise_floor, w_importance, w_load)
    if ws is None:
        ws = workspace(dims, opts, x.device)
    load = torch.empty(n, dtype=torch.float32, device=x.device)
    losses = torch.empty(3, dtype=torch.float32, device=x.device)
    st = lib().moe_aux_losses(ctypes.byref(dims), ctypes.byref(opts), _ptr(x), _ptr(w_gate),
                              _ptr(w_noise), _ptr(gate_bias), _ptr(thresh), _ptr(offsets),
                              _ptr(perm_token), _ptr(importance), _ptr(load), _ptr(losses),
                              _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_aux_losses")
    return load, losses


class MoeForward:
    """Holds the layer's weights, options and a workspace for repeated
    ``moe_forward`` calls. Tensors stay owned by the caller."""

    def __init__(self, x_shape, w_gate, w_noise, w1, w2, k: int, *, b1=None, b2=None,
                 gate_bias=None, train: bool = True, noise_floor: float = 1e-2,
                 w_importance: float = 0.1, w_load: float = 0.1, act_dtype=None,
                 capacity: int = 0, gate_order: int = 0, expert_layout: int = 0):
        """expert_layout=1: w1 and w2 come from moe_pack_expert_weights."""
        B, d = x_shape
        n, h, _ = w1.shape
        self.w_gate, self.w_noise, self.w1, self.w2, self.b1, self.b2 = w_gate, w_noise, w1, w2, b1, b2
        self.gate_bias = gate_bias
        _dev(w_gate, "w_gate", shape=(n, d))
        _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
        _dev(w1, "w1")
        _dev(w2, "w2", w1.dtype, (n, d, h))
        _dev(b1, "b1", w1.dtype, (n, h))
        _dev(b2, "b2", w1.dtype, (n, d))
        _dev(gate_bias, "gate_bias", torch.float32, (n,))
        adt = _dt(w1) if act_dtype is None else act_dtype
        self.dims = make_dims(B, d, h, n, k, adt, _dt(w1), _dt(w_gate), capacity, expert_layout)
        self.opts = make_opts(train, noise_floor, w_importance, w_load, gate_order)
        dev = w1.device
        self.ws = workspace(self.dims, self.opts, dev)
        self.importance = torch.empty(n, dtype=torch.float32, device=dev)
        self.load = torch.empty(n, dtype=torch.float32, device=dev)
        self.losses = torch.empty(3, dtype=torch.float32, device=dev)

    def __call__(self, x, eps, y=None, *, topk_idx=None, topk_gate=None, thresh=None, counts=None,
                 perm_token=None, stream=None):
        d = self.dims
        _dev(x, "x", self.w1.dtype, (d.tokens, d.d_model))
        _dev(eps, "eps", torch.float32, (d.tokens, d.n_experts))
        if y is None:
            y = torch.empty((d.tokens, d.d_model), dtype=x.dtype, device=x.device)
        _dev(y, "y", x.dtype, (d.tokens, d.d_model))
        for name, t, dt, shp in (("topk_idx", topk_idx, torch.int32, (d.tokens, d.k)),
                                 ("topk_gate", topk_gate, torch.float32, (d.tokens, d.k)),
                                 ("thresh", thresh, torch.float32, (d.tokens, 2)),
                                 ("counts", counts, torch.int32, (d.n_experts,)),
                                 ("perm_token", perm_token, torch.int32, (d.tokens * d.k,))):
            _dev(t, name, dt, shp)
        st = lib().moe_forward(ctypes.byref(self.dims), ctypes.byref(self.opts), _ptr(x),
                               _ptr(self.w_gate), _ptr(self.w_noise), _ptr(self.gate_bias),
                               _ptr(eps), _ptr(self.w1), _ptr(self.b1), _ptr(self.w2),
                               _ptr(self.b2), _ptr(y), _ptr(self.importance), _ptr(self.load),
                               _ptr(self.losses), _ptr(topk_idx), _ptr(topk_gate), _ptr(thresh),
                               _ptr(counts), _ptr(perm_token), _ptr(self.ws), self.ws.numel(),
                               _stream(stream))
        _check(st, "moe_forward")
        return y


def moe_forward(x, w_gate, w_noise, eps, w1, w2, k: int, *, b1=None, b2=None, gate_bias=None,
                train: bool = True, noise_floor: float = 1e-2, w_importance: float = 0.1,
                w_load: float = 0.1, return_routing: bool = False, capacity: int = 0,
                gate_order: int = 0, expert_layout: int = 0, stream=None):
    """One call of the whole forward pass; returns a dict of device tensors."""
    f = MoeForward(tuple(x.shape), w_gate, w_noise, w1, w2, k, b1=b1, b2=b2, gate_bias=gate_bias,
                   train=train, noise_floor=noise_floor, w_importance=w_importance, w_load=w_load,
                   capacity=capacity, gate_order=gate_order, expert_layout=expert_layout)
    B, n = x.shape[0], w1.shape[0]
    extra = {}
    if return_routing:
        dev = x.device
        extra = {"topk_idx": torch.empty((B, k), dtype=torch.int32, device=dev),
                 "topk_gate": torch.empty((B, k), dtype=torch.float32, device=dev),
                 "thresh": torch.empty((B, 2), dtype=torch.float32, device=dev),
                 "counts": torch.empty(n, dtype=torch.int32, device=dev),
                 "perm_token": torch.empty(B * k, dtype=torch.int32, device=dev)}
    y = f(x, eps, **extra, stream=stream)
    out = {"y": y, "importance": f.importance, "load": f.load, "losses": f.losses}
    out.update(extra)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def moe_forward_noalloc(x, w_gate, w_noise, eps, w1, w2, k: int, *, y=None, importance=None,
                        load=None, losses=None, b1=None, b2=None, gate_bias=None,
                        train: bool = True, noise_floor: float = 1e-2, w_importance: float = 0.1,
                        w_load: float = 0.1, capacity: int = 0, gate_order: int = 0,
                        topk_idx=None, topk_gate=None, thresh=None, counts=None, perm_token=None,
                        expert_layout: int = 0, stream=None):
    """The whole forward pass through ``moe_forward_noalloc``: the library
    takes its workspace from its static per-device scratch (no allocation by
    the library; outputs not given are allocated here by torch). Returns a dict
    of the outputs."""
    B, d = x.shape
    n, h, _ = w1.shape
    _dev(x, "x", w1.dtype, (B, d))
    _dev(w_gate, "w_gate", shape=(n, d))
    _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
    _dev(w2, "w2", w1.dtype, (n, d, h))
    _dev(b1, "b1", w1.dtype, (n, h))
    _dev(b2, "b2", w1.dtype, (n, d))
    _dev(gate_bias, "gate_bias", torch.float32, (n,))
    _dev(eps if train else None, "eps", torch.float32, (B, n))
    dev = x.device
    y = torch.empty((B, d), dtype=x.dtype, device=dev) if y is None else y
    importance = torch.empty(n, dtype=torch.float32, device=dev) if importance is None else importance
    load = torch.empty(n, dtype=torch.float32, device=dev) if load is None else load
    losses = torch.empty(3, dtype=torch.float32, device=dev) if losses is None else losses
    _dev(y, "y", x.dtype, (B, d))
    for name, t, dt, shp in (("importance", importance, torch.float32, (n,)),
                             ("load", load, torch.float32, (n,)),
                             ("losses", losses, torch.float32, (3,)),
                             ("topk_idx", topk_idx, torch.int32, (B, k)),
                             ("topk_gate", topk_gate, torch.float32, (B, k)),
                             ("thresh", thresh, torch.float32, (B, 2)),
                             ("counts", counts, torch.int32, (n,)),
                             ("perm_token", perm_token, torch.int32, (B * k,))):
        _dev(t, name, dt, shp)
    dims = make_dims(B, d, h, n, k, _dt(x), _dt(w1), _dt(w_gate), capacity, expert_layout)
    opts = make_opts(train, noise_floor, w_importance, w_load, gate_order)
    st = lib().moe_forward_noalloc(ctypes.byref(dims), ctypes.byref(opts), _ptr(x), _ptr(w_gate),
                                   _ptr(w_noise), _ptr(gate_bias), _ptr(eps if train else None),
                                   _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(y),
                                   _ptr(importance), _ptr(load), _ptr(losses), _ptr(topk_idx),
                                   _ptr(topk_gate), _ptr(thresh), _ptr(counts), _ptr(perm_token),
                                   _stream(stream))
    _check(st, "moe_forward_noalloc")
    out = {"y": y, "importance": importance, "load": load, "losses": losses}
    for name, t in (("topk_idx", topk_idx), ("topk_gate", topk_gate), ("thresh", thresh),
                    ("counts", counts), ("perm_token", perm_token)):
        if t is not None:
            out[name] = t
    return out


def moe_backward(x, w_gate, w_noise, eps, w1, w2, k: int, topk_idx, topk_gate, thresh, importance,
                 load, dy, *, b1=None, b2=None, gate_bias=None, train: bool = True,
                 noise_floor: float = 1e-2, w_importance: float = 0.1, w_load: float = 0.1,
                 aux_scale: float = 1.0, ws: Optional[torch.Tensor] = None,
                 stream=None) -> Dict[str, torch.Tensor]:
    """Gradients (fp32) of sum dy . y + aux_scale * (weighted losses) for x and
    every parameter, from a forward pass's selection, thresholds, Importance
    and Load: dx, dw_gate, dw_noise, dw1, dw2, plus dgate_bias / db1 / db2 for
    the biases that are given."""
    B, d = x.shape
    n, h, _ = w1.shape
    _dev(x, "x", w1.dtype, (B, d))
    _dev(w_gate, "w_gate", shape=(n, d))
    _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
    _dev(w2, "w2", w1.dtype, (n, d, h))
    _dev(b1, "b1", w1.dtype, (n, h))
    _dev(b2, "b2", w1.dtype, (n, d))
    _dev(gate_bias, "gate_bias", torch.float32, (n,))
    _dev(eps if train else None, "eps", torch.float32, (B, n))
    _dev(topk_idx, "topk_idx", torch.int32, (B, k))
    _dev(topk_gate, "topk_gate", torch.float32, (B, k))
    _dev(thresh, "thresh", torch.float32, (B, 2))
    _dev(importance, "importance", torch.float32, (n,))
    _dev(load, "load", torch.float32, (n,))
    _dev(dy, "dy", x.dtype, (B, d))
    dims = make_dims(B, d, h, n, k, _dt(x), _dt(w1), _dt(w_gate))
    opts = make_opts(train, noise_floor, w_importance, w_load)
    dev = x.device
    if ws is None:
        nbytes = int(lib().moe_backward_workspace_size(ctypes.byref(dims), ctypes.byref(opts)))
        if nbytes == 0:
            _check(1, "moe_backward_workspace_size")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    f32 = torch.float32
    out = {"dx": torch.empty((B, d), dtype=f32, device=dev),
           "dw_gate": torch.empty((n, d), dtype=f32, device=dev),
           "dw_noise": torch.empty((n, d), dtype=f32, device=dev),
           "dw1": torch.empty((n, h, d), dtype=f32, device=dev),
           "dw2": torch.empty((n, d, h), dtype=f32, device=dev)}
    if gate_bias is not None:
        out["dgate_bias"] = torch.empty(n, dtype=f32, device=dev)
    if b1 is not None:
        out["db1"] = torch.empty((n, h), dtype=f32, device=dev)
    if b2 is not None:
        out["db2"] = torch.empty((n, d), dtype=f32, device=dev)
    st = lib().moe_backward(ctypes.byref(dims), ctypes.byref(opts), _ptr(x), _ptr(w_gate),
                            _ptr(w_noise), _ptr(gate_bias), _ptr(eps if train else None),
                            _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(topk_idx),
                            _ptr(topk_gate), _ptr(thresh), _ptr(importance), _ptr(load), _ptr(dy),
                            ctypes.c_float(aux_scale), _ptr(out["dx"]), _ptr(out["dw_gate"]),
                            _ptr(out["dw_noise"]), _ptr(out.get("dgate_bias")), _ptr(out["dw1"]),
                            _ptr(out.get("db1")), _ptr(out["dw2"]), _ptr(out.get("db2")),
                            _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_backward")
    return out


class MoeBatchwiseForward:
    """Holds the weights, options and workspace for repeated
    ``moe_batchwise_forward`` calls: batchwise gating, where every expert takes
    its ``rows_per_expert`` best rows of the batch (above ``expert_threshold``
    [n] fp32 if given). Tensors stay owned by the caller."""

    def __init__(self, x_shape, w_gate, w_noise, w1, w2, rows_per_expert: int, *, b1=None,
                 b2=None, gate_bias=None, expert_threshold=None, train: bool = True,
                 noise_floor: float = 1e-2, w_importance: float = 0.1, w_load: float = 0.1,
                 act_dtype=None, expert_layout: int = 0):
        B, d = x_shape
        n, h, _ = w1.shape
        self.w_gate, self.w_noise, self.w1, self.w2, self.b1, self.b2 = w_gate, w_noise, w1, w2, b1, b2
        self.gate_bias, self.threshold = gate_bias, expert_threshold
        _dev(w_gate, "w_gate", shape=(n, d))
        _dev(w_noise, "w_noise", w_gate.dtype, (n, d))
        _dev(w1, "w1")
        _dev(w2, "w2", w1.dtype, (n, d, h))
        _dev(b1, "b1", w1.dtype, (n, h))
        _dev(b2, "b2", w1.dtype, (n, d))
        _dev(gate_bias, "gate_bias", torch.float32, (n,))
        _dev(expert_threshold, "expert_threshold", torch.float32, (n,))
        adt = _dt(w1) if act_dtype is None else act_dtype
        self.m = int(rows_per_expert)
        self.dims = make_dims(B, d, h, n, 1, adt, _dt(w1), _dt(w_gate), 0, expert_layout)
        self.opts = make_opts(train, noise_floor, w_importance, w_load)
        size = lib().moe_batchwise_workspace_size(ctypes.byref(self.dims), ctypes.byref(self.opts),
                                                  self.m)
        if size == 0:
            raise MoeError(f"moe_batchwise_workspace_size: invalid shape or options "
                           f"(B={B}, n={n}, m={self.m})")
        dev = w1.device
        self.ws = torch.empty(size, dtype=torch.uint8, device=dev)
        self.counts = torch.empty(n, dtype=torch.int32, device=dev)
        self.sel_token = torch.empty(n * self.m, dtype=torch.int32, device=dev)
        self.sel_score = torch.empty(n * self.m, dtype=torch.float32, device=dev)
        self.sel_gate = torch.empty(n * self.m, dtype=torch.float32, device=dev)
        self.importance = torch.empty(n, dtype=torch.float32, device=dev)
        self.load = torch.empty(n, dtype=torch.float32, device=dev)
        self.losses = torch.empty(3, dtype=torch.float32, device=dev)

    def __call__(self, x, eps, y=None, *, stream=None):
        d = self.dims
        _dev(x, "x", self.w1.dtype, (d.tokens, d.d_model))
        _dev(eps, "eps", torch.float32, (d.tokens, d.n_experts))
        if y is None:
            y = torch.empty((d.tokens, d.d_model), dtype=x.dtype, device=x.device)
        _dev(y, "y", x.dtype, (d.tokens, d.d_model))
        st = lib().moe_batchwise_forward(
            ctypes.byref(self.dims), ctypes.byref(self.opts), self.m, _ptr(self.threshold),
            _ptr(x), _ptr(self.w_gate), _ptr(self.w_noise), _ptr(self.gate_bias), _ptr(eps),
            _ptr(self.w1), _ptr(self.b1), _ptr(self.w2), _ptr(self.b2), _ptr(y),
            _ptr(self.counts), _ptr(self.sel_token), _ptr(self.sel_score), _ptr(self.sel_gate),
            _ptr(self.importance), _ptr(self.load), _ptr(self.losses), _ptr(self.ws),
            self.ws.numel(), _stream(stream))
        _check(st, "moe_batchwise_forward")
        return y


def moe_batchwise_forward(x, w_gate, w_noise, eps, w1, w2, rows_per_expert: int, *, b1=None,
                          b2=None, gate_bias=None, expert_threshold=None, train: bool = True,
                          noise_floor: float = 1e-2, w_importance: float = 0.1,
                          w_load: float = 0.1, expert_layout: int = 0, stream=None):
    """One call of the batchwise-gated forward pass; returns a dict of device
    tensors (y, counts, sel_token, sel_score, sel_gate [n * m], importance,
    load, losses)."""
    f = MoeBatchwiseForward(tuple(x.shape), w_gate, w_noise, w1, w2, rows_per_expert, b1=b1, b2=b2,
                            gate_bias=gate_bias, expert_threshold=expert_threshold, train=train,
                            noise_floor=noise_floor, w_importance=w_importance, w_load=w_load,
                            expert_layout=expert_layout)
    y = f(x, eps, stream=stream)
    return {"y": y, "counts": f.counts, "sel_token": f.sel_token, "sel_score": f.sel_score,
            "sel_gate": f.sel_gate, "importance": f.importance, "load": f.load,
            "losses": f.losses}


class MoeHierForward:
    """Holds a hierarchical layer's weights, options and workspace for repeated
    ``moe_hier_forward`` calls (section "Hierarchical MoE"): primary gate
    ``w_gate1``/``w_noise1`` [a, d], secondary gates ``w_gate2``/``w_noise2``
    [a, b, d], leaves ``w1`` [a*b, h, d] and ``w2`` [a*b, d, h]."""

    def __init__(self, x_shape, w_gate1, w_noise1, w_gate2, w_noise2, w1, w2, k1: int, k2: int, *,
                 b1=None, b2=None, train: bool = True, noise_floor: float = 1e-2,
                 w_importance: float = 0.1, w_load: float = 0.1, expert_layout: int = 0):
        B, d = x_shape
        a, b, _ = w_gate2.shape
        n, h, _ = w1.shape
        if n != a * b:
            raise MoeError(f"w1 has {n} leaves, expected groups * group_experts = {a * b}")
        _dev(w_gate1, "w_gate1", shape=(a, d))
        _dev(w_noise1, "w_noise1", w_gate1.dtype, (a, d))
        _dev(w_gate2, "w_gate2", w_gate1.dtype, (a, b, d))
        _dev(w_noise2, "w_noise2", w_gate1.dtype, (a, b, d))
        _dev(w1, "w1")
        _dev(w2, "w2", w1.dtype, (n, d, h))
        _dev(b1, "b1", w1.dtype, (n, h))
        _dev(b2, "b2", w1.dtype, (n, d))
        self.w = (w_gate1, w_noise1, w_gate2, w_noise2, w1, b1, w2, b2)
        self.dims = MoeHierDims(B, d, h, a, b, k1, k2, _dt(w1), _dt(w1), _dt(w_gate1),
                                expert_layout)
        self.opts = make_opts(train, noise_floor, w_importance, w_load)
        dev = w1.device
        nbytes = int(lib().moe_hier_workspace_size(ctypes.byref(self.dims), ctypes.byref(self.opts)))
        if nbytes == 0:
            _check(1, "moe_hier_workspace_size")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.importance = torch.empty(n, dtype=torch.float32, device=dev)
        self.load = torch.empty(n, dtype=torch.float32, device=dev)
        self.losses = torch.empty(3, dtype=torch.float32, device=dev)

    def output_shapes(self) -> Dict[str, Tuple[Tuple[int, ...], torch.dtype]]:
        """Shape and dtype of every optional output."""
        d = self.dims
        B, a, b, k1, k2 = d.tokens, d.groups, d.group_experts, d.k1, d.k2
        i32, f32 = torch.int32, torch.float32
        return {"topk_idx": ((B, k1 * k2), i32), "topk_gate": ((B, k1 * k2), f32),
                "counts": ((a * b,), i32), "group_idx": ((B, k1), i32),
                "group_gate": ((B, k1), f32), "group_thresh": ((B, 2), f32),
                "group_rows": ((a,), i32), "group_importance": ((a,), f32),
                "group_load": ((a,), f32), "sub_idx": ((B, k1, k2), i32),
                "sub_gate": ((B, k1, k2), f32), "sub_thresh": ((B, k1, 2), f32),
                "sub_load": ((a * b,), f32)}

    def __call__(self, x, eps1, eps2, y=None, *, stream=None, **extra):
        d = self.dims
        w_gate1, w_noise1, w_gate2, w_noise2, w1, b1, w2, b2 = self.w
        _dev(x, "x", w1.dtype, (d.tokens, d.d_model))
        train = bool(self.opts.train)
        _dev(eps1 if train else None, "eps1", torch.float32, (d.tokens, d.groups))
        _dev(eps2 if train else None, "eps2", torch.float32, (d.tokens, d.k1, d.group_experts))
        if y is None:
            y = torch.empty((d.tokens, d.d_model), dtype=x.dtype, device=x.device)
        _dev(y, "y", x.dtype, (d.tokens, d.d_model))
        shapes = self.output_shapes()
        outs = MoeHierOutputs()
        for name, t in extra.items():
            if name not in shapes:
                raise MoeError(f"unknown output {name}")
            shp, dt = shapes[name]
            _dev(t, name, dt, shp)
            setattr(outs, name, t.data_ptr() if t is not None else None)
        st = lib().moe_hier_forward(
            ctypes.byref(self.dims), ctypes.byref(self.opts), _ptr(x), _ptr(w_gate1),
            _ptr(w_noise1), _ptr(eps1 if train else None), _ptr(w_gate2), _ptr(w_noise2),
            _ptr(eps2 if train else None), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(y),
            _ptr(self.importance), _ptr(self.load), _ptr(self.losses), ctypes.byref(outs),
            _ptr(self.ws), self.ws.numel(), _stream(stream))
        _check(st, "moe_hier_forward")
        return y


def moe_hier_forward(x, w_gate1, w_noise1, eps1, w_gate2, w_noise2, eps2, w1, w2, k1: int, k2: int,
                     *, b1=None, b2=None, train: bool = True, noise_floor: float = 1e-2,
                     w_importance: float = 0.1, w_load: float = 0.1, return_all: bool = False,
                     expert_layout: int = 0, stream=None):
    """One call of the hierarchical forward pass; returns a dict of device tensors
    (with ``return_all`` also every optional output of the C call)."""
    f = MoeHierForward(tuple(x.shape), w_gate1, w_noise1, w_gate2, w_noise2, w1, w2, k1, k2,
                       b1=b1, b2=b2, train=train, noise_floor=noise_floor,
                       w_importance=w_importance, w_load=w_load, expert_layout=expert_layout)
    extra = {}
    if return_all:
        extra = {name: torch.empty(shp, dtype=dt, device=x.device)
                 for name, (shp, dt) in f.output_shapes().items()}
    y = f(x, eps1, eps2, **extra, stream=stream)
    out = {"y": y, "importance": f.importance, "load": f.load, "losses": f.losses}
    out.update(extra)
    return out
