"""Host-side checks of the budget-sweep speedup model: the fit recovers a known
correction constant, and the error figures behave as the model implies."""
import numpy as np

from rl_rollout_amd.budget_sweep import fit_kappa, held_out, mape, model_speedup


def test_fit_recovers_kappa_from_exact_model_values():
    g = 4
    f = np.array([0.80, 0.85, 0.92, 0.97])
    rho = np.array([0.07, 0.12, 0.27, 0.52])
    true_kappa = 0.35
    meas = model_speedup(g, f, rho, true_kappa)
    k = fit_kappa(g, f, rho, meas)
    assert abs(k - true_kappa) < 1e-6
    assert mape(model_speedup(g, f, rho, k), meas) < 1e-6
    # without the correction the model overstates every speedup
    assert np.all(model_speedup(g, f, rho, 0.0) > meas)
    assert mape(model_speedup(g, f, rho, 0.0), meas) > 10.0


def test_model_shape_matches_the_reported_trend():
    """More budget: more accepted drafts but a larger read ratio; with reads
    growing faster than acceptance the modelled speedup falls."""
    g = 4
    f = np.array([0.804, 0.853, 0.918, 0.967])
    rho = np.array([0.05, 0.10, 0.25, 0.50])
    s = model_speedup(g, f, rho, 0.3)
    assert np.all(np.diff(s) < 0)
    assert s[0] > 1.0


def test_fit_with_noisy_measurements_is_least_squares():
    g = 4
    rng = np.random.default_rng(0)
    f = np.array([0.8, 0.85, 0.9, 0.95])
    rho = np.array([0.06, 0.11, 0.26, 0.51])
    meas = model_speedup(g, f, rho, 0.5) * (1 + rng.normal(0, 0.01, 4))
    k = fit_kappa(g, f, rho, meas)

    def loss(x):
        return np.sum((model_speedup(g, f, rho, x) - meas) ** 2)

    for d in (1e-3, -1e-3):
        assert loss(k) <= loss(k + d) + 1e-15


def test_held_out_predictions():
    """Leave-one-out: on exact model values every fold recovers kappa and predicts
    the held-out point; with noise the held-out error is at least the in-sample one
    and each fold's kappa is the least-squares fit of the other points."""
    g = 4
    f = np.array([0.80, 0.85, 0.92, 0.97])
    rho = np.array([0.07, 0.12, 0.27, 0.52])
    meas = model_speedup(g, f, rho, 0.4)
    pred, err, kappas = held_out(g, f, rho, meas)
    np.testing.assert_allclose(kappas, 0.4, atol=1e-6)
    assert err < 1e-4
    noisy = meas * (1 + np.array([0.02, -0.015, 0.01, -0.02]))
    pred, err, kappas = held_out(g, f, rho, noisy)
    k_all = fit_kappa(g, f, rho, noisy)
    assert err >= mape(model_speedup(g, f, rho, k_all), noisy) - 1e-9
    for i in range(4):
        keep = np.arange(4) != i
        assert abs(kappas[i] - fit_kappa(g, f[keep], rho[keep], noisy[keep])) < 1e-12
        assert abs(pred[i] - model_speedup(g, f[i], rho[i], kappas[i])) < 1e-12
