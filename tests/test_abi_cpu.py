"""The C ABI on the host: the library loads, exports every symbol that
include/moe.h declares, sizes workspaces, and rejects invalid arguments with
the documented status before touching the device. No call here passes
validation, so nothing is ever launched (the pointers are fake)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("sparsely_gated_mixture_moe_amd")
from sparsely_gated_mixture_moe_amd import _binding as B  # noqa: E402

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|int|const char\*|size_t)\s+(moe_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_symbols_are_exported():
    L = B.lib()
    names = declared_functions()
    assert "moe_forward" in names and len(names) >= 10
    for name in names:
        assert hasattr(L, name), f"{name} declared in moe.h but not exported"
    assert L.moe_abi_version() == 6


def dims(**kw):
    base = dict(tokens=1024, d_model=512, d_hidden=1024, n_experts=64, k=4, act_dtype=1,
                expert_dtype=1, gate_dtype=1, capacity=0, expert_layout=0)
    base.update(kw)
    return B.MoeDims(*[base[f] for f, _ in B.MoeDims._fields_])


def opts(**kw):
    base = dict(train=1, noise_floor=0.01, w_importance=0.1, w_load=0.1, gate_order=0)
    base.update(kw)
    return B.MoeGateOpts(*[base[f] for f, _ in B.MoeGateOpts._fields_])


def P(v=FAKE):
    return ctypes.c_void_p(v)


def call_gate(d, o, x=FAKE, eps=FAKE, out=FAKE):
    L = B.lib()
    return L.moe_gate(ctypes.byref(d) if d is not None else None,
                      ctypes.byref(o) if o is not None else None, P(x), P(), P(), None, P(eps),
                      P(out), P(out), P(out), None, 0, None)


def last_error():
    return B.lib().moe_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    ({"k": 0}, INVALID, "k = 0"),
    ({"k": 65}, INVALID, "k = 65"),
    ({"k": 9, "n_experts": 100}, UNSUPPORTED, "k = 9"),
    ({"tokens": -1}, INVALID, "tokens"),
    ({"n_experts": 0}, INVALID, "n_experts"),
    ({"n_experts": 40000}, INVALID, "n_experts"),
    ({"d_model": 96}, UNSUPPORTED, "d_model"),
    ({"d_model": 1024}, UNSUPPORTED, "d_model"),
    ({"d_hidden": 100}, UNSUPPORTED, "d_hidden"),
    ({"act_dtype": 0, "expert_dtype": 0, "gate_dtype": 1}, UNSUPPORTED, "bf16 gate"),
    ({"expert_dtype": 0}, UNSUPPORTED, "expert_dtype"),
    ({"act_dtype": 7}, INVALID, "dtype"),
    ({"tokens": 600_000_000}, INVALID, "int32"),
    ({"capacity": -1}, INVALID, "capacity"),
])
def test_invalid_dims(kw, status, msg):
    assert call_gate(dims(**kw), opts()) == status
    assert msg in last_error()
    assert B.lib().moe_workspace_size(ctypes.byref(dims(**kw)), ctypes.byref(opts())) == 0


def test_null_and_misaligned_pointers():
    assert call_gate(None, opts()) == INVALID and "dims" in last_error()
    assert call_gate(dims(), None) == INVALID and "opts" in last_error()
    assert call_gate(dims(), opts(), x=0) == INVALID and "x is NULL" in last_error()
    assert call_gate(dims(), opts(), x=FAKE + 4) == INVALID and "aligned" in last_error()
    assert call_gate(dims(), opts(), eps=0) == INVALID and "eps" in last_error()
    # biases and noise rows are copied 16 bytes at a time: a 4-byte offset view is refused
    assert call_gate(dims(), opts(), eps=FAKE + 4) == INVALID and "eps is not 16-byte" in last_error()
    L = B.lib()
    st = L.moe_gate(ctypes.byref(dims()), ctypes.byref(opts()), P(), P(), P(), P(FAKE + 4), P(),
                    P(), P(), P(), None, 0, None)
    assert st == INVALID and "bias is not 16-byte" in last_error()
    assert call_gate(dims(), opts(train=2)) == INVALID
    assert call_gate(dims(), opts(noise_floor=-1.0)) == INVALID
    assert call_gate(dims(), opts(noise_floor=float("nan"))) == INVALID
    assert call_gate(dims(), opts(gate_order=2)) == INVALID


def test_workspace_checks():
    L = B.lib()
    d, o = dims(), opts()
    need = L.moe_workspace_size(ctypes.byref(d), ctypes.byref(o))
    # the forward pass holds the routing and one bf16 expert output row per (token, slot)
    assert need >= 1024 * 4 * 512 * 2
    args = [ctypes.byref(d), ctypes.byref(o)] + [P()] * 3 + [None] + [P()] + [P()] + [None] + \
        [P()] + [None] + [P()] * 4 + [None] * 5
    st = L.moe_forward(*args, P(), need - 256, None)
    assert st == WORKSPACE and "needed" in last_error()
    st = L.moe_forward(*args, None, need, None)
    assert st == WORKSPACE
    st = L.moe_forward(*args, P(FAKE + 16), need, None)
    assert st == INVALID and "256-byte" in last_error()
    # route needs its block histograms
    st = L.moe_route(ctypes.byref(d), P(), P(), P(), P(), P(), P(), P(), None, P(), 16, None)
    assert st == WORKSPACE


def test_workspace_size_scales_with_workload():
    L = B.lib()
    small = L.moe_workspace_size(ctypes.byref(dims(tokens=1000)), ctypes.byref(opts()))
    big = L.moe_workspace_size(ctypes.byref(dims(tokens=65536, n_experts=4096)),
                               ctypes.byref(opts()))
    assert 0 < small < big
    infer = L.moe_workspace_size(ctypes.byref(dims(tokens=65536, n_experts=4096)),
                                 ctypes.byref(opts(train=0)))
    assert infer < big  # no Load partial sums without noise
    assert L.moe_workspace_size(ctypes.byref(dims(tokens=0)), ctypes.byref(opts())) > 0


def test_timing_argument_checks():
    L = B.lib()
    assert L.moe_ffn_timing(2) == 1 and L.moe_ffn_timing(-1) == 1  # MOE_ERR_INVALID
    assert L.moe_ffn_timing_read(None, None) == 1


def test_status_strings():
    L = B.lib()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def hdims(**kw):
    base = dict(tokens=1024, d_model=512, d_hidden=1024, groups=16, group_experts=32, k1=2, k2=2,
                act_dtype=1, expert_dtype=1, gate_dtype=1, expert_layout=0)
    base.update(kw)
    return B.MoeHierDims(*[base[f] for f, _ in B.MoeHierDims._fields_])


def call_hier(d, o, ws=FAKE, ws_bytes=1 << 40, eps2=FAKE, extra=None):
    L = B.lib()
    return L.moe_hier_forward(ctypes.byref(d), ctypes.byref(o), P(), P(), P(), P(), P(), P(),
                              P(eps2), P(), None, P(), None, P(), P(), P(), P(),
                              ctypes.byref(extra) if extra is not None else None, P(ws), ws_bytes,
                              None)


@pytest.mark.parametrize("kw,status,msg", [
    ({"groups": 0}, INVALID, "groups"),
    ({"k1": 0}, INVALID, "k1"),
    ({"k1": 17}, INVALID, "k1"),
    ({"k2": 33}, INVALID, "k2"),
    ({"k1": 3, "k2": 3}, UNSUPPORTED, "k1 * k2"),
    ({"groups": 256, "group_experts": 256}, INVALID, "32768"),
    ({"d_model": 96}, UNSUPPORTED, "d_model"),
    ({"tokens": -5}, INVALID, "tokens"),
])
def test_hier_invalid_dims(kw, status, msg):
    assert call_hier(hdims(**kw), opts()) == status
    assert msg in last_error()
    assert B.lib().moe_hier_workspace_size(ctypes.byref(hdims(**kw)), ctypes.byref(opts())) == 0


def test_hier_pointer_and_workspace_checks():
    L = B.lib()
    d, o = hdims(), opts()
    need = L.moe_hier_workspace_size(ctypes.byref(d), ctypes.byref(o))
    # the leaf layer's expert outputs alone take B * k1 * k2 bf16 rows
    assert need >= 1024 * 4 * 512 * 2
    assert call_hier(d, o, eps2=0) == INVALID and "eps2" in last_error()
    assert call_hier(d, opts(train=0), eps2=0, ws_bytes=0) == WORKSPACE
    assert call_hier(d, o, ws_bytes=need - 256) == WORKSPACE and "needed" in last_error()
    assert call_hier(d, o, ws=FAKE + 16, ws_bytes=need) == INVALID
    bad = B.MoeHierOutputs()
    bad.sub_load = FAKE + 2
    assert call_hier(d, o, extra=bad) == INVALID and "sub_load" in last_error()
    infer = L.moe_hier_workspace_size(ctypes.byref(d), ctypes.byref(opts(train=0)))
    assert 0 < infer < need


def call_batchwise(d, o, m, ws=FAKE, ws_bytes=1 << 40, y=FAKE, counts=FAKE):
    L = B.lib()
    return L.moe_batchwise_forward(ctypes.byref(d), ctypes.byref(o), m, None, P(), P(), P(), None,
                                   P(), P(), None, P(), None, P(y), P(counts), P(), P(), P(), P(),
                                   P(), P(), P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,okw,m,status,msg", [
    ({}, {}, 0, INVALID, "rows_per_expert"),
    ({"tokens": 70000}, {}, 64, UNSUPPORTED, "65536"),
    ({"capacity": 8}, {}, 64, UNSUPPORTED, "capacity"),
    ({}, {"gate_order": 1}, 64, UNSUPPORTED, "gate_order"),
    ({"n_experts": 32768, "tokens": 65536}, {}, 65536, INVALID, "int32"),
    ({"d_hidden": 100}, {}, 64, UNSUPPORTED, "d_hidden"),
])
def test_batchwise_invalid_arguments(kw, okw, m, status, msg):
    d, o = dims(**kw), opts(**okw)
    assert call_batchwise(d, o, m) == status
    assert msg in last_error()
    assert B.lib().moe_batchwise_workspace_size(ctypes.byref(d), ctypes.byref(o), m) == 0


def test_batchwise_pointer_and_workspace_checks():
    L = B.lib()
    d, o = dims(tokens=65536, n_experts=4096), opts()
    need = L.moe_batchwise_workspace_size(ctypes.byref(d), ctypes.byref(o), 64)
    # the fp32 score matrix [n, B] and one bf16 expert output row per slot
    assert need >= 4096 * 65536 * 4 + 4096 * 64 * 512 * 2
    assert call_batchwise(d, o, 64, counts=0) == INVALID and "counts is NULL" in last_error()
    assert call_batchwise(d, o, 64, y=FAKE + 2) == INVALID and "aligned" in last_error()
    assert call_batchwise(d, o, 64, ws_bytes=need - 1) == WORKSPACE
    assert call_batchwise(d, o, 64, ws=FAKE + 16, ws_bytes=need) == INVALID


def test_noalloc_rejects_dims_beyond_its_scratch():
    """moe_forward_noalloc refuses dims whose workspace exceeds the static
    scratch before any device call (the pointers here are fake)."""
    L = B.lib()
    d, o = dims(tokens=65536, n_experts=4096), opts()
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(o)) > B.NOALLOC_SCRATCH_BYTES
    st = L.moe_forward_noalloc(ctypes.byref(d), ctypes.byref(o), *([P()] * 18), None)
    assert st == WORKSPACE
    assert "static" in last_error() and str(B.NOALLOC_SCRATCH_BYTES) in last_error()


def call_backward(d, o, ws=FAKE, ws_bytes=1 << 40, aux=1.0, dw1=FAKE, dy=FAKE, topk=FAKE):
    L = B.lib()
    return L.moe_backward(ctypes.byref(d), ctypes.byref(o), P(), P(), P(), None, P(), P(), None,
                          P(), None, P(topk), P(), P(), P(), P(), P(dy), ctypes.c_float(aux), P(),
                          P(), P(), None, P(dw1), None, P(), None, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,okw,aux,status,msg", [
    ({"capacity": 8}, {}, 1.0, UNSUPPORTED, "capacity"),
    ({}, {"gate_order": 1}, 1.0, UNSUPPORTED, "gate_order"),
    ({}, {}, float("inf"), INVALID, "aux_scale"),
    ({"k": 9, "n_experts": 100}, {}, 1.0, UNSUPPORTED, "k = 9"),
    ({"d_hidden": 100}, {}, 1.0, UNSUPPORTED, "d_hidden"),
])
def test_backward_invalid_arguments(kw, okw, aux, status, msg):
    assert call_backward(dims(**kw), opts(**okw), aux=aux) == status
    assert msg in last_error()


def test_backward_pointer_and_workspace_checks():
    L = B.lib()
    d, o = dims(), opts()
    need = L.moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(o))
    # recomputed hidden rows, their gradients and the dense gate-logit gradients
    assert need >= 1024 * 4 * 1024 * 4 + 1024 * 2 * 64 * 4
    assert call_backward(d, o, dw1=0) == INVALID and "dw1 is NULL" in last_error()
    assert call_backward(d, o, dy=FAKE + 4) == INVALID and "dy" in last_error()
    assert call_backward(d, o, topk=0) == INVALID and "topk_idx" in last_error()
    assert call_backward(d, o, ws_bytes=need - 256) == WORKSPACE and "needed" in last_error()
    assert call_backward(d, o, ws=FAKE + 16, ws_bytes=need) == INVALID


def test_pack_expert_weights_and_layout_rejections():
    L = B.lib()
    d = dims()
    nbytes = 64 * 1024 * 512 * 2  # each of w1, w2 at these dims
    w1, w2, p1, p2 = FAKE, FAKE + nbytes, FAKE + 2 * nbytes, FAKE + 3 * nbytes

    def pack(*ptrs, dd=d):
        return L.moe_pack_expert_weights(ctypes.byref(dd), *[P(v) for v in ptrs], None)

    assert pack(w1, w2, p1 + 8, p2) == INVALID and "16-byte" in last_error()
    assert pack(w1, w2, w1 + 16, p2) == INVALID and "overlaps an input" in last_error()
    assert pack(w1, w2, p1, w2 + nbytes - 16) == INVALID and "overlaps an input" in last_error()
    assert pack(w1, w2, p1, p1 + 1024) == INVALID and "overlap" in last_error()
    assert pack(w1, w2, p1, p2, dd=dims(d_model=96)) == UNSUPPORTED
    assert pack(w1, w2, p1, p2, dd=dims(expert_layout=2)) == INVALID
    assert "expert_layout" in last_error()
    assert call_gate(dims(expert_layout=-1), opts()) == INVALID
