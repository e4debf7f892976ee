"""The seeded input generators: shapes, determinism and the built spectrum."""
import numpy as np

import workloads


def test_standard_shapes():
    wl = workloads.standard_workloads()
    assert wl["c1_fp32_256x512"].shapes == ((256, 512),)
    assert wl["c2_96x2048x6144"].shapes == ((2048, 6144),) * 96
    c3 = wl["c3_rank_222_experts"].shapes
    assert len(c3) == 222
    assert c3[:3] == ((6144, 2048), (6144, 2048), (2048, 6144))
    assert sum(1 for s in c3 if s == (6144, 2048)) == 148
    c4 = wl["c4_dense_attn"].shapes
    assert c4.count((6144, 6144)) == 16 and c4.count((6144, 1024)) == 16
    c5 = wl["c5_mixed_illcond"]
    assert c5.batch == 128 and c5.steps == 10 and c5.nesterov
    assert {d for s in c5.shapes for d in s} <= set(workloads.MIXED_DIMS)


def test_generation_is_deterministic_per_matrix():
    wl = workloads.standard_workloads()["c2_96x2048x6144"].with_shapes([(64, 96)] * 3)
    a = workloads.matrix_inputs(wl, 1)
    b = workloads.matrix_inputs(wl, 1)
    c = workloads.matrix_inputs(wl, 2)
    for k in ("w", "m", "g"):
        assert np.array_equal(a[k], b[k])
        assert not np.array_equal(a[k], c[k])
    assert abs(float(a["g"].std()) - 1e-3) < 1e-4
    assert abs(float(a["w"].std()) - 0.02) < 2e-3


def test_illcond_spectrum_is_built():
    wl = workloads.standard_workloads()["c5_mixed_illcond"].with_shapes([(96, 160), (160, 64)])
    for j, (r, c) in enumerate(wl.shapes):
        g = workloads.matrix_inputs(wl, j)["g"].astype(np.float64)
        want = np.sort(workloads.illcond_spectrum(wl.seed, j, min(r, c)))[::-1]
        got = np.linalg.svd(g, compute_uv=False)
        assert want.min() >= 1e-4 and want.max() <= 1.0
        assert np.abs(got - want).max() < 1e-6


def test_bf16_cast_rounds_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], np.float32)
    got = workloads.as_float64(workloads.cast(x, "bf16"))
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, 1.0]
