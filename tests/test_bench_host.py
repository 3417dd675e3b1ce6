"""Host-side arithmetic of bench.py (no GPU): the median of the timed steps
and the per-stage roof fractions."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_median():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 3.0, 2.0]) == 2.5


def test_roof_mfma_bound_stage():
    # 0.55 TFLOP in 0.5 ms on a 2500 TFLOP/s roof: 1100 TFLOP/s, 44 %; the
    # 1.15 GB it reads would take 0.144 ms at 8 TB/s, so the MFMA roof binds
    r = bench.roof("gate", 0.5, 0.55e12, 1.15e9, 2500.0)
    assert r["bound"] == "mfma"
    assert r["tflops"] == pytest.approx(1100.0)
    assert r["mfma_frac"] == pytest.approx(0.44)
    assert r["roof_ms"] == pytest.approx(0.22)
    assert r["frac"] == pytest.approx(0.44)
    assert r["hbm_frac"] == pytest.approx(1.15e9 / 0.5e-3 / 8e12)


def test_roof_hbm_bound_stage():
    # 9.13 GB and 0.55 TFLOP in 1.74 ms: the bytes take 1.141 ms at 8 TB/s,
    # the flops 0.22 ms at 2500 TFLOP/s, so HBM binds
    r = bench.roof("ffn", 1.74, 0.55e12, 9.13e9, 2500.0)
    assert r["bound"] == "hbm"
    assert r["gbs"] == pytest.approx(9.13e9 / 1.74e-3 / 1e9)
    assert r["frac"] == pytest.approx(9.13e9 / 8e12 * 1e3 / 1.74)


def test_roof_latency_stage():
    r = bench.roof("route", 0.046)
    assert r["bound"] == "latency" and r["frac"] is None and r["roof_ms"] == 0.0
