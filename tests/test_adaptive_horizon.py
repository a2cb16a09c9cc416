"""Host-side checks of the adaptive draft-horizon controller and of the
position-dependent draft-noise profiles."""
import numpy as np

from rl_rollout_amd import workloads as W
from rl_rollout_amd.adaptive import HorizonController
from rl_rollout_amd.calibrate import acceptance, linear_profile


def _controller(alpha, cost, gm=6):
    c = HorizonController(gm, cost, explore_every=0)
    c.reach[:] = 1e6
    c.keep[:] = np.asarray(alpha) * 1e6
    return c


def test_choice_maximises_expected_tokens_per_time():
    alpha = [0.95, 0.9, 0.84, 0.79, 0.73, 0.68]
    cost = lambda g: 10.0 + 1.5 * g
    c = _controller(alpha, cost)
    best = max(range(1, 7), key=lambda g: (1 + np.sum(np.cumprod(alpha[:g]))) / cost(g))
    assert c.choose() == best
    assert abs(c.expected_tokens(2) - (1 + 0.95 + 0.95 * 0.9)) < 1e-12


def test_horizon_shrinks_when_late_positions_deteriorate_or_drafts_get_dearer():
    cost = lambda g: 10.0 + 1.5 * g
    early = _controller([0.96, 0.9, 0.85, 0.79, 0.73, 0.68], cost).choose()
    late = _controller([0.94, 0.6, 0.4, 0.3, 0.2, 0.1], cost).choose()
    assert late < early
    dear = _controller([0.96, 0.9, 0.85, 0.79, 0.73, 0.68], lambda g: 10.0 + 6.0 * g).choose()
    assert dear < early


def test_measured_step_times_correct_a_wrong_cost_model():
    """A model that underestimates the cost of the longest horizon picks it; measured
    step times at that horizon move the choice to the best one."""
    alpha = [0.93, 0.89, 0.78, 0.72, 0.68, 0.63]
    true_cost = lambda g: 10.0 + 0.3 * g + (2.0 if g == 6 else 0.0)
    c = _controller(alpha, lambda g: 10.0 + 0.3 * g)
    best = max(range(1, 7), key=lambda g: (1 + np.sum(np.cumprod(alpha[:g]))) / true_cost(g))
    assert c.choose() == 6 and best == 5
    for _ in range(5):
        c.observe_time(6, true_cost(6))
    assert abs(c.step_time(6) - true_cost(6)) < 0.5
    assert c.choose() == best


def test_update_tracks_the_observed_keep_rate_per_position():
    c = HorizonController(4, lambda g: 1.0 + g, prior=0.5, prior_weight=1.0, decay=1.0, explore_every=0)
    rng = np.random.default_rng(0)
    true = np.array([0.9, 0.8, 0.7, 0.6])
    for _ in range(400):
        a = np.zeros(256, dtype=np.int64)
        alive = np.ones(256, dtype=bool)
        for j in range(4):
            kept = alive & (rng.random(256) < true[j])
            a += kept
            alive = kept
        c.update(a, 4)
    assert np.allclose(c.alpha(), true, atol=0.01)
    # a step at horizon 2 observes positions 1 and 2 only
    before = c.reach.copy()
    c.update(np.array([0, 1, 2, 2]), 2)
    assert np.all(c.reach[2:] == before[2:])
    assert c.reach[0] == before[0] + 4 and c.reach[1] == before[1] + 3


def test_position_profiles_are_linear_in_position_and_reproduce_the_checkpoint_rate():
    prof = linear_profile(0.958, 0.679, 6)
    assert abs(prof[0] - 0.958) < 1e-12 and abs(prof[5] - 0.679) < 1e-12
    assert abs(np.mean(prof) - 0.819) < 1e-3       # printed checkpoint-level rate 81.9%
    late = linear_profile(0.942, 0.613, 6)
    assert abs(np.mean(late) - 0.775) < 3e-3       # printed 77.5%


def test_stored_noise_gives_the_profile_acceptance():
    """The stored per-position noise of the 8B-like profile reproduces its first-
    and last-position acceptance (estimated on fresh rows)."""
    w = W.QWEN3_8B_24K_POSITIONS
    a1 = acceptance(w.position_noise[0], rows=8, seed=7)
    a6 = acceptance(w.position_noise[5], rows=8, seed=7)
    assert abs(a1 - 0.958) < 0.004 and abs(a6 - 0.679) < 0.006
    assert all(x < y for x, y in zip(w.position_noise, w.position_noise[1:]))
