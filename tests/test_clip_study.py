"""The CPU clipping study (oracle/clip_study.py) against the FORGE
assessment's P2 claims ("Math verified, not asserted"): exact global-norm
clipping keeps the second moment bounded through a gradient spike, while
clipping the update after the optimizer, or clipping with the previous
step's norm, leave sqrt(v) inflated as much as no clipping at all. The page
quotes 3.18x ten steps after the spike without its setup; with a 100x spike
at steady state this study gives 3.41x for sqrt(mean v_hat) and 2.91x for
mean sqrt(v_hat), bracketing it (magnitude: parity unpinned)."""
import numpy as np
import pytest

from oracle import clip_study


@pytest.fixture(scope="module")
def study():
    return clip_study.run()


def test_clip_update_leaves_v_exactly_as_no_clipping(study):
    runs = study["runs"]
    assert np.array_equal(runs["clip_update"]["v"], runs["none"]["v"])
    assert np.array_equal(runs["clip_update"]["m"], runs["none"]["m"])
    # ... while the parameters do differ (the update itself was clipped)
    assert not np.array_equal(runs["clip_update"]["W"], runs["none"]["W"])


def test_delayed_norm_is_no_better_than_no_clipping(study):
    r = study["ratios"]
    for key in ("rms_sqrt_v", "mean_sqrt_v"):
        assert abs(r["delayed"][key] / r["none"][key] - 1.0) < 0.01


def test_spike_inflation_magnitude(study):
    r = study["ratios"]
    assert r["exact"]["rms_sqrt_v"] == 1.0
    # the page's 3.18x lies between the two definitions of "sqrt(v) bar"
    assert 2.5 < r["none"]["mean_sqrt_v"] < 3.18 < r["none"]["rms_sqrt_v"] < 4.0


def test_exact_clipping_keeps_second_moment_at_steady_state(study):
    ex = study["runs"]["exact"]["rms_sqrt_v"]
    warm, after = study["setup"]["warm"], study["setup"]["after"]
    pre = ex[warm - 1]
    assert abs(ex[warm + after] / pre - 1.0) < 0.05
    # without clipping the spike step itself moves it by ~sqrt(1 + (1 - beta2) spike^2)
    none = study["runs"]["none"]["rms_sqrt_v"]
    expect = np.sqrt(1.0 + (1 - 0.999) * 100.0 ** 2)
    assert abs(none[warm] / pre / expect - 1.0) < 0.05
