"""Pins for the oracle's exact speculative accept: hand-worked cases, the p == q
and one-hot closed forms, exact enumeration against the dense autoregressive
joint, and a Monte Carlo chi-square of the sampler. No GPU."""
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import enumeration
from rl_rollout_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_small.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    tl = np.log(np.array(case["p"], dtype=np.float64))[None]
    dl = np.log(np.array(case["q"], dtype=np.float64))[None]
    a, out = oracle.spec_accept(tl, dl, np.array([case["draft_tokens"]]), np.array([case["u_accept"]], np.float32),
                                np.array([case["u_sample"]], np.float32), 1.0)
    assert a[0] == case["num_accepted"]
    assert list(out[0]) == case["out_tokens"]


def test_p_equals_q_accepts_every_draft_and_draws_bonus_from_last_row():
    rng = np.random.default_rng(5)
    B, gamma, V = 40, 4, 300
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = tl[:, :gamma].copy()
    d = rng.integers(0, V, (B, gamma))
    ua = rng.random((B, gamma), dtype=np.float32)
    ua[0] = np.float32(1.0 - 2 ** -24)          # the largest float32 below 1
    us = rng.random(B, dtype=np.float32)
    a, out = oracle.spec_accept(tl, dl, d, ua, us, 1.0)
    assert (a == gamma).all()
    np.testing.assert_array_equal(out[:, :gamma], d)
    for b in range(B):
        p_last = oracle.softmax_row(tl[b, gamma], 1.0)
        assert out[b, gamma] == oracle.inverse_cdf(p_last, us[b])


def test_one_hot_draft_closed_form():
    """q one-hot at x: keep x with probability p(x); otherwise the correction is p
    with x removed, renormalised."""
    rng = np.random.default_rng(9)
    V, x = 12, 5
    tl = rng.normal(0, 1, (1, 2, V))
    dl = np.full((1, 1, V), -1e4)
    dl[0, 0, x] = 0.0                                   # exp(-1e4) == 0 in float64
    p = np.exp(tl[0, 0] - tl[0, 0].max())
    p /= p.sum()
    us_grid = (np.arange(200) + 0.5) / 200
    for u in (p[x] - 0.01, p[x] + 0.01):
        a, out = oracle.spec_accept(tl, dl, np.array([[x]]), np.array([[u]], np.float32),
                                    np.array([0.5], np.float32), 1.0)
        assert a[0] == (1 if u < p[x] else 0)
    resid = p.copy()
    resid[x] = 0
    resid /= resid.sum()
    cdf = np.cumsum(resid)
    for us in us_grid:
        a, out = oracle.spec_accept(tl, dl, np.array([[x]]), np.array([[0.999]], np.float32),
                                    np.array([us], np.float32), 1.0)
        us32 = float(np.float32(us))
        assert out[0, 0] == int(np.searchsorted(cdf, us32, side="right"))
        assert out[0, 0] != x


def test_temperature_divides_logits():
    rng = np.random.default_rng(2)
    tl = rng.normal(0, 2, (3, 3, 50)).astype(np.float32)
    dl = (tl[:, :2] + rng.normal(0, 0.5, (3, 2, 50))).astype(np.float32)
    d = rng.integers(0, 50, (3, 2))
    ua = rng.random((3, 2), dtype=np.float32)
    us = rng.random(3, dtype=np.float32)
    T = 0.5
    r1 = oracle.spec_accept(tl, dl, d, ua, us, T)
    r2 = oracle.spec_accept(tl.astype(np.float64) / T, dl.astype(np.float64) / T, d, ua, us, 1.0)
    np.testing.assert_array_equal(r1[0], r2[0])
    np.testing.assert_array_equal(r1[1], r2[1])


@pytest.mark.parametrize("gamma", [1, 2, 3])
@pytest.mark.parametrize("n", [2, 3])
def test_enumeration_equals_dense_autoregressive_joint(gamma, n):
    p, q = synth.markov_tables(16, seed=100 + gamma)
    for prev in (0, 7):
        joint = enumeration.joint_first_tokens(p, q, prev, gamma, n)
        dense = enumeration.dense_joint(p, prev, n)
        np.testing.assert_allclose(joint, dense, rtol=0, atol=1e-12)
        assert abs(joint.sum() - 1) < 1e-12


def test_planted_residual_sign_error_breaks_enumeration(monkeypatch):
    """A plausible mistake (residual max(0, q - p)) must fail the enumeration pin."""
    p, q = synth.markov_tables(16, seed=3)

    def wrong(p_row, q_row):
        r = np.maximum(0.0, q_row - p_row)
        return r / r.sum()

    monkeypatch.setattr(enumeration, "corrected_distribution", wrong)
    joint = enumeration.joint_first_tokens(p, q, 0, 2, 2)
    assert np.abs(joint - enumeration.dense_joint(p, 0, 2)).max() > 1e-3


def test_planted_accept_ratio_inversion_breaks_enumeration(monkeypatch):
    p, q = synth.markov_tables(16, seed=4)
    monkeypatch.setattr(enumeration, "accept_probability", lambda pr, qr, x: min(1.0, qr[x] / pr[x]))
    joint = enumeration.joint_first_tokens(p, q, 0, 2, 2)
    assert np.abs(joint - enumeration.dense_joint(p, 0, 2)).max() > 1e-3


# ------------------------------------------------------------- Monte Carlo of the sampler

def markov_step_inputs(p_tab, q_tab, prev, gamma, rng):
    """Inputs of one S3R step per trial: drafts drawn from the q chain (inverse CDF
    on a uniform, done here in the test), logits = log of the table rows."""
    B = prev.shape[0]
    V = p_tab.shape[0]
    ctx = np.empty((B, gamma + 1), dtype=np.int64)
    ctx[:, 0] = prev
    d = np.empty((B, gamma), dtype=np.int64)
    qc = np.cumsum(q_tab, axis=1)
    for j in range(gamma):
        u = rng.random(B)
        d[:, j] = np.minimum((qc[ctx[:, j]] <= u[:, None]).sum(axis=1), V - 1)
        ctx[:, j + 1] = d[:, j]
    with np.errstate(divide="ignore"):         # a zero table entry is a masked (-inf) logit
        tl = np.log(p_tab[ctx])                # [B][G1][V]
        dl = np.log(q_tab[ctx[:, :gamma]])     # [B][gamma][V]
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    return tl, dl, d, ua, us


def chi_square_pooled(counts, probs, min_expected=5.0):
    """Pearson chi-square with cells of expected count < min_expected pooled."""
    n = counts.sum()
    exp = probs * n
    small = exp < min_expected
    c = np.append(counts[~small], counts[small].sum())
    e = np.append(exp[~small], exp[small].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    stat = ((c - e) ** 2 / e).sum()
    return stat, len(e) - 1


def sample_two_tokens(sampler, p_tab, q_tab, gamma, trials, seed, prev0=0):
    rng = np.random.default_rng(seed)
    prev = np.full(trials, prev0)
    a, out = sampler(*markov_step_inputs(p_tab, q_tab, prev, gamma, rng))
    first = out[:, 0].copy()
    second = out[:, 1].copy()
    need = a == 0                       # the step emitted a single token: run the next step
    if need.any():
        a2, out2 = sampler(*markov_step_inputs(p_tab, q_tab, first[need], gamma, rng))
        second[need] = out2[:, 0]
    return first, second


def test_oracle_sampler_matches_exact_distribution_chi_square():
    """1e6 trials of the oracle's sampler (rows split over worker processes)."""
    from oracle_parallel import spec_accept_rows
    p, q = synth.markov_tables(16, seed=21, alpha=4.0)
    gamma, trials = 2, 1_000_000
    first, second = sample_two_tokens(lambda *x: spec_accept_rows(*x, 1.0), p, q, gamma, trials, seed=77)
    exact = enumeration.joint_first_tokens(p, q, 0, gamma, 2)
    c1 = np.bincount(first, minlength=16)
    stat1, df1 = chi_square_pooled(c1, exact.sum(axis=1))
    assert stat1 < stats.chi2.ppf(1 - 0.001, df1), (stat1, df1)
    c2 = np.bincount(first * 16 + second, minlength=256)
    stat2, df2 = chi_square_pooled(c2, exact.reshape(-1))
    assert stat2 < stats.chi2.ppf(1 - 0.001, df2), (stat2, df2)


def _masked_tables(vocab, seed, n_mask):
    """Markov tables whose rows each give zero probability (a -inf logit) to n_mask
    tokens, chosen independently for p and q, so some tokens only the draft can
    propose (always rejected) and some only the target can emit (never drafted)."""
    p, q = synth.markov_tables(vocab, seed=seed, alpha=4.0)
    rng = np.random.default_rng(seed + 1)
    for t in (p, q):
        for row in t:
            row[rng.choice(vocab, size=n_mask, replace=False)] = 0.0
            row /= row.sum()
    return p, q


def test_masked_enumeration_still_equals_the_dense_joint():
    p, q = _masked_tables(16, seed=31, n_mask=5)
    for gamma, n in [(1, 2), (2, 3), (3, 2)]:
        np.testing.assert_allclose(enumeration.joint_first_tokens(p, q, 0, gamma, n), enumeration.dense_joint(p, 0, n),
                                   rtol=0, atol=1e-12)


def test_oracle_sampler_with_masked_logits_matches_exact_distribution_chi_square():
    """1e6 trials with -inf logits in both rows (5 of 16 tokens masked per row, p and
    q independently): the two-token joint matches the exact one, and no trial emits
    a token pair the dense chain gives zero probability."""
    from oracle_parallel import spec_accept_rows
    p, q = _masked_tables(16, seed=41, n_mask=5)
    gamma, trials = 2, 1_000_000
    first, second = sample_two_tokens(lambda *x: spec_accept_rows(*x, 1.0), p, q, gamma, trials, seed=78)
    exact = enumeration.joint_first_tokens(p, q, 0, gamma, 2)
    np.testing.assert_allclose(exact, enumeration.dense_joint(p, 0, 2), rtol=0, atol=1e-12)
    c2 = np.bincount(first * 16 + second, minlength=256)
    assert c2[exact.reshape(-1) == 0].sum() == 0
    c1 = np.bincount(first, minlength=16)
    stat1, df1 = chi_square_pooled(c1, exact.sum(axis=1))
    assert stat1 < stats.chi2.ppf(1 - 0.001, df1), (stat1, df1)
    stat2, df2 = chi_square_pooled(c2, exact.reshape(-1))
    assert stat2 < stats.chi2.ppf(1 - 0.001, df2), (stat2, df2)


def test_masked_logits_emit_only_tokens_the_target_row_allows():
    """Random masks on both sides (about half of 64 tokens per row), drafts drawn
    from the draft rows: every kept draft and every final token has a finite target
    logit in its row, kept drafts are the drafted tokens, and -1 fills the rest."""
    rng = np.random.default_rng(5)
    B, V, gamma = 4000, 64, 4
    tl = rng.normal(0, 2, (B, gamma + 1, V))
    dl = tl[:, :gamma] + rng.normal(0, 1, (B, gamma, V))
    tl[rng.random(tl.shape) < 0.5] = -np.inf
    dl[rng.random(dl.shape) < 0.5] = -np.inf
    tl[:, :, 0] = np.where(np.isinf(tl).all(axis=2), 0.0, tl[:, :, 0])  # every row keeps a token
    dl[:, :, 0] = np.where(np.isinf(dl).all(axis=2), 0.0, dl[:, :, 0])
    qd = np.exp(dl - dl.max(axis=2, keepdims=True))
    qc = np.cumsum(qd / qd.sum(axis=2, keepdims=True), axis=2)
    u = rng.random((B, gamma, 1))
    d = np.minimum((qc <= u).sum(axis=2), V - 1)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    a, out = oracle.spec_accept(tl, dl, d, ua, us, 1.0)
    for b in range(B):
        k = int(a[b])
        assert (out[b, :k] == d[b, :k]).all()
        assert all(np.isfinite(tl[b, j, d[b, j]]) for j in range(k))
        assert np.isfinite(tl[b, k, out[b, k]])
        assert (out[b, k + 1:] == -1).all()


def test_a_draft_its_own_row_masks_is_kept_exactly_when_the_target_allows_it():
    """q(d) = 0 (the draft row masks its own token): the test u * q(d) < p(d) reads
    0 < p(d), so the draft is kept iff the target row gives it mass, whatever u."""
    V, gamma = 8, 2
    tl = np.zeros((2, gamma + 1, V))
    dl = np.zeros((2, gamma, V))
    d = np.array([[3, 5], [3, 5]])
    dl[:, 0, 3] = -np.inf
    dl[:, 1, 5] = -np.inf
    tl[1, 1, 5] = -np.inf  # sequence 1: the target masks the second draft
    ua = np.full((2, gamma), 0.999, dtype=np.float32)
    us = np.array([0.5, 0.5], dtype=np.float32)
    a, out = oracle.spec_accept(tl, dl, d, ua, us, 1.0)
    assert list(a) == [2, 1]
    assert list(out[0, :2]) == [3, 5] and list(out[1, :1]) == [3]
    assert out[1, 1] != 5 and np.isfinite(tl[1, 1, out[1, 1]])


def test_commit_advances_by_accepted_plus_one():
    np.testing.assert_array_equal(oracle.commit([10, 20, 30], [0, 4, 2]), [11, 25, 33])
