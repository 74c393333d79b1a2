"""CPU checks of the seeded input generator (the recipe both sides consume)."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import workloads


def test_generator_is_deterministic_and_shaped():
    a = workloads.small("bf16", 2, 3, 128, 64, seed=4, fox=True)
    b = workloads.small("bf16", 2, 3, 128, 64, seed=4, fox=True)
    for k in ("q", "k", "v", "w", "beta", "logf"):
        assert np.array_equal(a[k], b[k])
    assert a["q"].shape == (2, 3, 128, 64) and a["beta"].shape == (2, 3, 128)
    assert a["logf"].dtype == np.float32 and a["beta"].dtype == np.float32


def test_bf16_values_are_representable():
    a = workloads.small("bf16", 1, 2, 64, 64, seed=1)
    for k in ("q", "k", "v", "w"):
        bits = a[k].view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)


def test_bf16_round_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)], dtype=np.float32)
    y = workloads.bf16_round(x)
    assert list(y) == [1.0, 1.0 + 2 ** -6, 1.0, -1.0]


def test_w_unit_and_beta_range():
    a = workloads.small("f32", 1, 2, 256, 128, seed=2, beta_sigma=1.5)
    n = np.linalg.norm(a["w"].astype(np.float64), axis=-1)
    assert np.max(np.abs(n - 1)) < 1e-6
    assert np.all(a["beta"] > 0) and np.all(a["beta"] < 2)


def test_near_two_fraction_and_gate():
    wl = dataclasses.replace(workloads.MID_D128_NEAR2, B=2, H=2, T=4096)
    a = workloads.generate(wl)
    frac = np.mean(a["beta"] >= 1.9)
    assert 0.09 < frac < 0.14     # 10 % forced plus the natural tail above 1.9
    assert np.all(a["beta"] < 2)
    f = workloads.generate(dataclasses.replace(workloads.FOX_D128, B=1, H=2, T=2048))["logf"]
    assert np.all(f < 0) and -0.2 < f.mean() < 0


def test_workload_table_matches_stated_shapes():
    shapes = [(w.dtype, w.B, w.H, w.T, w.d, w.fox) for w in workloads.WORKLOADS]
    assert shapes == [("f32", 1, 2, 256, 64, False), ("bf16", 16, 16, 2048, 64, False),
                      ("bf16", 16, 8, 2048, 128, False), ("bf16", 2, 16, 16384, 64, False),
                      ("bf16", 4, 8, 8192, 128, True)]
    assert [w.seed for w in workloads.WORKLOADS] == [0, 1, 2, 3, 4]
    long = workloads.LONG_D64
    assert long.flops_path() == pytest.approx(1.649e12, rel=1e-3)
    assert long.flops_attn() == pytest.approx(1.0995e12, rel=1e-3)
