"""Host logic of the SPRINT timing model (SPRINT report section 3.3, eqs. 4-6).

The fits are checked against known coefficients: times generated from a
chosen eq. 6 (or eq. 5 line) must give those coefficients back, and eq. 4's
sums over synthetic profile records must group a product's launches and add
the per-kernel models as the equation writes them.
"""
import numpy as np
import pytest

from sgd_cnns_amd import timing_model as TM

# a plausible eq. 6: 60 TFLOP/s asymptote, bandwidth-like mn/mk/nk terms, 5 us floor (ms units)
ALPHA = np.array([2 / 60e9, 4 / 4e9, 4 / 6e9, 4 / 6e9, 1e-7, 2e-7, 3e-8, 5e-3])


def test_grid_points_follow_the_bounds():
    pts = TM.grid_points()
    assert len(pts) == len(set(pts))
    for m, n, k in pts:
        for v in (m, n, k):
            assert v & (v - 1) == 0 and 8 <= v <= 2 ** 22
        assert m * n * k <= 2 ** 38 and max(m * n, m * k, n * k) <= 2 ** 29
    assert (8, 8, 8) in pts and (2 ** 22, 8, 8) in pts and (4096, 4096, 2 ** 14) in pts
    assert (2 ** 22, 2 ** 8, 8) not in pts       # an operand of 2^30 elements


def test_offgrid_points_lie_between_the_grid():
    pts = TM.offgrid_points(200, seed=3)
    assert len(pts) == 200
    for m, n, k in pts:
        for v in (m, n, k):
            assert v in {round(2.0 ** (x + 0.25)) for x in range(3, 22)}    # 2^(x + 1/4), rounded
    assert TM.offgrid_points(200, seed=3) == pts


def test_eq6_fit_recovers_known_coefficients():
    m, n, k = np.array(TM.grid_points()).T
    t = TM.eq6(ALPHA, m, n, k)
    a = TM.fit_eq6(m, n, k, t)
    assert np.allclose(a, ALPHA, rtol=1e-6, atol=0)


def test_eq6_features_are_the_eight_terms():
    f = TM.eq6_features(2, 3, 5)
    assert list(f) == [30, 6, 10, 15, 2, 3, 5, 1]
    assert TM.EQ6_TERMS == ("mnk", "mn", "mk", "nk", "m", "n", "k", "1")


def test_eq6_fit_under_noise_predicts_within_the_noise():
    rng = np.random.default_rng(0)
    m, n, k = np.array(TM.grid_points()).T
    t = TM.eq6(ALPHA, m, n, k) * np.exp(rng.normal(0, 0.02, m.size))
    a = TM.fit_eq6(m, n, k, t)
    off = np.array(TM.offgrid_points(300, seed=1)).T
    err = TM.rel_errors(TM.eq6(a, *off), TM.eq6(ALPHA, *off))
    assert np.median(np.abs(err)) < 0.01


def test_linear_fit_recovers_line_and_handles_one_size():
    x = np.array([1e3, 1e5, 1e7, 1e9])
    a, b = TM.fit_linear(x, 2e-9 * x + 3e-3)
    assert a == pytest.approx(2e-9, rel=1e-9) and b == pytest.approx(3e-3, rel=1e-9)
    assert TM.fit_linear([5.0, 5.0], [1.0, 3.0]) == (0.0, 2.0)


def test_fit_rejects_too_few_or_nonpositive_samples():
    with pytest.raises(ValueError):
        TM.fit_eq6([1, 2], [1, 2], [1, 2], [1.0, 2.0])
    m, n, k = np.array(TM.grid_points()[:20]).T
    t = np.ones(20)
    t[3] = 0.0
    with pytest.raises(ValueError):
        TM.fit_eq6(m, n, k, t)


def rec(name, ms, nbytes=0.0, shape=(0, 0, 0, -1)):
    return (name, 0, 0, ms, 0.0, nbytes, shape)


def test_products_and_eq4_sums():
    recs = [rec("im2col", 0.5, 1e6),
            rec("gemm_dma_128x128_nt", 1.0, shape=(4096, 64, 576, 0)),
            rec("maxpool_fwd", 0.2, 2e6),
            rec("gemm_dma_128x64_tn", 2.0, shape=(64, 577, 4096, 1)),
            rec("gemm_sk_fixup", 0.25, shape=(64, 577, 4096, 1)),
            rec("gemm_staged_64x128_nn", 0.75, shape=(4096, 576, 64, 2)),
            rec("splitk_reduce", 0.125, shape=(4096, 576, 64, 2)),
            rec("im2col", 0.3, 5e5)]
    prods, others = TM.products_of(recs)
    assert [(p["family"], p["form"], p["m"], p["n"], p["k"], p["ms"]) for p in prods] == [
        ("dma", "nt", 4096, 64, 576, 1.0), ("dma", "tn", 64, 577, 4096, 2.25),
        ("staged", "nn", 4096, 576, 64, 0.875)]
    assert others == [("im2col", 1e6, 0.5), ("maxpool_fwd", 2e6, 0.2), ("im2col", 5e5, 0.3)]

    models = TM.fit_kernel_models(recs)
    a, b = models["im2col"]
    assert a * 1e6 + b == pytest.approx(0.5) and a * 5e5 + b == pytest.approx(0.3)
    assert models["maxpool_fwd"] == (0.0, 0.2)

    alphas = {fam: {f: ALPHA * (i + 1) * (j + 1) for i, f in enumerate(("nt", "tn", "nn"))}
              for j, fam in enumerate(("dma", "staged"))}
    p = TM.predict_step(recs, alphas, models)
    want_sg = sum(float(TM.eq6(alphas[fam][f], m, n, k)) for fam, f, m, n, k in
                  [("dma", "nt", 4096, 64, 576), ("dma", "tn", 64, 577, 4096), ("staged", "nn", 4096, 576, 64)])
    assert p["sgemm_pred"] == pytest.approx(want_sg)
    assert p["sgemm_meas"] == pytest.approx(1.0 + 2.25 + 0.875)
    assert p["cuda_pred"] == pytest.approx(1.0) and p["cuda_meas"] == pytest.approx(1.0)
    assert p["pred"] == pytest.approx(want_sg + 1.0)
    with pytest.raises(KeyError):
        TM.predict_step(recs, {"dma": alphas["dma"]}, models)
    with pytest.raises(KeyError):
        TM.predict_step(recs, alphas, {"im2col": (0.0, 0.1)})


def test_kernel_forms():
    assert TM.form_of_kernel("gemm_dma_128x128_tn") == "tn"
    assert TM.form_of_kernel("gemm_staged_64x128_nt") == "nt"
    assert TM.form_of_kernel("gemm_conv_fwd_128x64") == "nt"
    assert TM.form_of_kernel("gemm_conv_dw_128x128") == "tn"
    assert TM.form_of_kernel("gemm_conv_dx_64x128") == "nn"
    assert TM.form_of_kernel("gemm_sk_fixup") is None
    assert TM.family_of_kernel("gemm_staged_128x64_nn") == "staged"
    assert TM.family_of_kernel("gemm_conv_dx_64x128") == "dma"


def test_staged_shapes_break_the_direct_load_alignment():
    for f in ("nt", "nn"):
        assert TM.staged_shape(f, 64, 32, 128) == (64, 32, 130)     # A stored [m][k]: k % 4 != 0
    for f in ("tn", "tt"):
        assert TM.staged_shape(f, 64, 32, 128) == (66, 32, 128)     # A stored [k][m]: m % 4 != 0
