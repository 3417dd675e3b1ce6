"""The seeded input generator: deterministic, sliceable, standard normal."""
import numpy as np
import pytest
from scipy import stats

import datagen as dg


def test_deterministic_and_sliceable():
    a = dg.normal(7, 3, 0, 10001)
    b = dg.normal(7, 3, 0, 10001)
    assert np.array_equal(a, b)
    for off, cnt in [(1, 5), (2, 7), (9999, 2), (5000, 1)]:
        assert np.array_equal(dg.normal(7, 3, off, cnt), a[off:off + cnt])


def test_streams_differ_by_seed_and_tensor():
    a = dg.normal(1, 1, 0, 4096)
    assert not np.array_equal(a, dg.normal(2, 1, 0, 4096))
    assert not np.array_equal(a, dg.normal(1, 2, 0, 4096))
    assert abs(np.corrcoef(a, dg.normal(1, 2, 0, 4096))[0, 1]) < 0.1


def test_standard_normal_distribution():
    z = dg.normal(11, 4, 0, 400_000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # neighbouring draws (cos / sin branches of one pair, and across pairs) are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 0.01


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 dtype=np.float32)
    b = dg.f32_to_bf16(x)
    back = dg.bf16_to_f32(b)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    assert back[5] == 1.0 and back[6] == np.float32(1.0 + 2 ** -6)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)
    bf = dg.normal(5, 5, 0, 1000, dtype=dg.BF16)
    assert np.array_equal(bf, dg.f32_to_bf16(dg.normal(5, 5, 0, 1000)))


def test_workload_shapes():
    w = dg.workload("tiny_fp32")
    inp = dg.make_inputs(w, with_bias=True)
    assert inp["x"].shape == (256, 64) and inp["eps"].shape == (256, 16)
    assert inp["w1"].shape == (16, 128, 64) and inp["w2"].shape == (16, 64, 128)
    small = dg.make_inputs(dg.workload("tiny_fp32", tokens=100), experts=False)
    assert np.array_equal(small["x"], inp["x"][:100])
    assert np.array_equal(small["eps"], inp["eps"][:100])
    w4 = dg.WORKLOADS["flat_bf16_n4096"]
    assert w4.n_experts * w4.d_hidden * 2 * w4.d_model == 4_294_967_296
