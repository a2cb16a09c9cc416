"""Host-side checks of the per-sequence budget allocation: Dinkelbach's search
against brute force over every choice on small batches, the ordering a cost
proportional to length implies, its limits, and the key counts it prices
against the oracle's selection count."""
import itertools

import numpy as np
import pytest

import oracle
from rl_rollout_amd.budget_alloc import allocate, draft_keys_per_step, pages_selected, ratio
from rl_rollout_amd.measure import draft_keys


def _brute(E, C, fixed):
    B, M = E.shape
    return max(ratio(E, C, fixed, np.array(ch)) for ch in itertools.product(range(M), repeat=B))


@pytest.mark.parametrize("seed", range(12))
def test_allocation_is_the_best_of_every_choice(seed):
    rng = np.random.default_rng(seed)
    B, M = int(rng.integers(1, 6)), int(rng.integers(1, 5))
    E = rng.uniform(1.0, 5.0, (B, M))
    C = rng.uniform(0.0, 3.0, (B, M))
    fixed = float(rng.uniform(0.1, 5.0))
    choice, rate, rounds = allocate(E, C, fixed)
    assert rate == pytest.approx(ratio(E, C, fixed, choice), rel=1e-12)
    assert rate == pytest.approx(_brute(E, C, fixed), rel=1e-12)
    assert rounds >= 1


def test_shared_token_curve_with_cost_proportional_to_length():
    """Same tokens per budget for every sequence, draft cost s x length: the
    allocation gives a shorter sequence a budget at least as large as a longer
    one, and beats every single budget for the batch."""
    S = np.array([0.05, 0.10, 0.25, 0.50])
    E = 1 + 4 * np.array([0.60, 0.69, 0.81, 0.92])
    rng = np.random.default_rng(1)
    n = rng.integers(1024, 16385, 64).astype(np.float64)
    C = 4 * S[None, :] * n[:, None] * 1e-9
    fixed = 1.3 * n.sum() * 1e-9
    choice, rate, _ = allocate(E, C, fixed)
    order = np.argsort(n)
    assert np.all(np.diff(choice[order]) <= 0)
    uniform = [ratio(np.broadcast_to(E, C.shape), C, fixed, np.full(64, m)) for m in range(4)]
    assert rate >= max(uniform)
    assert len(set(choice)) > 1


def test_limits_of_the_fixed_time():
    E = np.array([[1.0, 2.0, 3.0], [1.0, 2.0, 3.0]])
    C = np.array([[0.0, 1.0, 2.0], [0.0, 4.0, 8.0]])
    # a fixed time that dwarfs the drafts: the most tokens for everyone
    choice, _, _ = allocate(E, C, 1e9)
    assert list(choice) == [2, 2]
    # a tiny fixed time: rate ~ sum E / sum C, the free first budget everywhere
    # would divide by ~0, which is the best ratio
    choice, _, _ = allocate(E, C, 1e-9)
    assert list(choice) == [0, 0]


def test_input_checks():
    with pytest.raises(ValueError):
        allocate([1.0, 2.0], [[0.0, 1.0]], 0.0)
    with pytest.raises(ValueError):
        allocate([1.0, 2.0], [[0.0, -1.0]], 1.0)
    with pytest.raises(ValueError):
        allocate([1.0, np.nan], [[0.0, 1.0]], 1.0)


def test_pages_selected_is_the_oracle_selection_count():
    for s in (0.02, 0.05, 0.1, 0.25, 0.3, 0.5, 1.0, 1.5):
        for n in list(range(0, 70)) + [999, 1000, 1001, 1536]:
            assert int(pages_selected(n, s)) == oracle.num_selected(n, s), (n, s)


def test_draft_keys_per_step_sums_the_draft_steps():
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 20000, 50)
    for s in (0.05, 0.5):
        nsel = pages_selected(lens // 16, s)
        want = sum(draft_keys(lens, nsel, j) for j in range(1, 5))
        np.testing.assert_array_equal(draft_keys_per_step(lens, s, 4), want)


def test_horizon_model_pieces():
    from rl_rollout_amd.horizon_alloc import draft_keys_by_position, expected_tokens, horizon_costs
    E = expected_tokens([0.9, 0.8, 0.5], 3)
    np.testing.assert_allclose(E, [1.0, 1.9, 1.9 + 0.72, 1.9 + 0.72 + 0.36])
    lens = np.array([0, 17, 100])
    k = draft_keys_by_position(lens, np.array([0, 1, 2]), 3)
    np.testing.assert_array_equal(k, [[1, 2, 3], [16 + 1 + 1, 16 + 1 + 2, 16 + 1 + 3], [32 + 4 + 1, 32 + 4 + 2, 32 + 4 + 3]])
    np.testing.assert_array_equal(k.sum(axis=0), [sum(draft_keys(lens, np.array([0, 1, 2]), j)) for j in (1, 2, 3)])
    c = horizon_costs(k, 2.0, 5.0)
    np.testing.assert_allclose(c[:, 0], 0.0)
    np.testing.assert_allclose(c[1], [0, 2 * 18 + 10, 2 * (18 + 19) + 20, 2 * (18 + 19 + 20) + 30])


def test_horizon_allocation_gives_long_sequences_shorter_horizons():
    """Shared expected tokens, costs growing with length: horizons never increase
    with length, and the allocation is the brute-force optimum on a small batch."""
    from rl_rollout_amd.horizon_alloc import draft_keys_by_position, expected_tokens, horizon_costs
    E = expected_tokens([0.95, 0.9, 0.83, 0.77, 0.72, 0.68], 6)
    lens = np.array([1000, 3000, 6000, 9000, 16000])
    C = horizon_costs(draft_keys_by_position(lens, pages_selected(lens // 16, 0.05), 6), 2e-9, 3e-8)
    choice, rate, _ = allocate(E, C, 1e-5)
    assert np.all(np.diff(choice) <= 0)
    assert rate == pytest.approx(_brute(np.broadcast_to(E, C.shape).copy(), C, 1e-5), rel=1e-12)
