"""moe_forward_noalloc (the forward pass for callers that cannot allocate:
its workspace is the library's static per-device scratch) through the C ABI,
against moe_forward with a workspace of the caller's. Both run the same
kernels on the same inputs, so every output must agree bit for bit. Each case
makes two calls in a row, the second on a smaller batch, so the second call
runs on what the first left in the scratch."""
import pytest

import datagen as dg
from parity import announce, gpu_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsely_gated_mixture_moe_amd as moe  # noqa: E402

FLOOR = 1e-2

# (workload, first call's overrides, second call's overrides, train, expert/gate biases)
CASES = [
    ("flat_bf16_n4096", {"tokens": 3000, "n_experts": 256, "d_hidden": 256},
     {"tokens": 700, "n_experts": 256, "d_hidden": 256}, True, False),
    # the second call takes the small-batch paths (split gate sweep and FFN units)
    ("flat_bf16_n4096", {"tokens": 2048, "n_experts": 512}, {"tokens": 5, "n_experts": 512},
     False, False),
    ("zipf_bf16_n256", {"tokens": 4096, "gate_dtype": dg.BF16}, {"tokens": 1000, "n_experts": 64},
     True, True),
    ("tiny_fp32", {"tokens": 4000}, {"tokens": 300, "n_experts": 9, "k": 3}, True, True),
]


def one_call(w, train, bias):
    inp = dg.make_inputs(w, with_bias=bias)
    g = gpu_inputs(inp)
    B, n, k = w.tokens, w.n_experts, w.k
    dev = g["x"].device
    outs = {"topk_idx": torch.empty((B, k), dtype=torch.int32, device=dev),
            "topk_gate": torch.empty((B, k), dtype=torch.float32, device=dev),
            "thresh": torch.empty((B, 2), dtype=torch.float32, device=dev),
            "counts": torch.empty(n, dtype=torch.int32, device=dev),
            "perm_token": torch.empty(B * k, dtype=torch.int32, device=dev)}
    got = moe.moe_forward_noalloc(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"],
                                  k, b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                                  train=train, noise_floor=FLOOR, **outs)
    ref = moe.moe_forward(g["x"], g["w_gate"], g["w_noise"], g["eps"], g["w1"], g["w2"], k,
                          b1=g.get("b1"), b2=g.get("b2"), gate_bias=g.get("gate_bias"),
                          train=train, noise_floor=FLOOR, return_routing=True)
    torch.cuda.synchronize()
    for key in ("y", "importance", "load", "losses", "topk_idx", "topk_gate", "thresh", "counts",
                "perm_token"):
        assert torch.equal(got[key], ref[key]), f"{key} differs"


@pytest.mark.parametrize("case", CASES, ids=[c[0] + f"-{c[1]['tokens']}-then-{c[2]['tokens']}"
                                             for c in CASES])
def test_noalloc_matches_forward(case):
    name, kw1, kw2, train, bias = case
    for kw in (kw1, kw2):
        w = dg.workload(name, **kw)
        announce(f"moe_forward_noalloc {name} {kw} train={train}")
        one_call(w, train, bias)


def test_noalloc_rejects_dims_beyond_the_scratch():
    """The whole benchmark workload needs far more than the static scratch:
    the call returns MOE_ERR_WORKSPACE and launches nothing."""
    dims = moe.make_dims(65536, 512, 1024, 4096, 4, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16)
    assert moe.moe_workspace_size(dims, moe.make_opts()) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.empty((65536, 512), dtype=torch.bfloat16, device="cuda")
    wg = torch.empty((4096, 512), dtype=torch.bfloat16, device="cuda")
    eps = torch.empty((65536, 4096), dtype=torch.float32, device="cuda")
    w1 = torch.empty((4096, 1024, 512), dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty((4096, 512, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="MOE_ERR_WORKSPACE.*static"):
        moe.moe_forward_noalloc(x, wg, wg, eps, w1, w2, 4)
