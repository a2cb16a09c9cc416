"""Exact output distribution of repeated S3R steps on a Markov toy policy.

TEST INFRASTRUCTURE (see oracle/s3r_oracle.py). This module computes, by exact
enumeration, the joint distribution of the first n tokens that repeated
speculative steps emit when the dense policy is p(.|prev) and the draft policy is
q(.|prev) over a small vocabulary. It is written from the definition of the
accept rule (accept a draft token x with probability min(1, p(x)/q(x))) and of
the correction (a draw from max(0, p - q) normalised), which the pages describe
in prose (rebasdaily.com, "草稿可以稀疏，交卷必须完整"; rit.work, "Как разреженный
черновик сохраняет ответы плотной модели"), and shares no code with the sampler in
s3r_oracle.py. The abstract claims the emitted responses follow the dense
policy; the tests check that this enumeration equals the product of p along the
sequence, and that the sampler's Monte Carlo frequencies match it.

Because drafts after the first rejection are discarded and the toy is Markov,
drawing d_j lazily from q(.|previous accepted token) gives the same law as
drawing the whole draft chain first.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np


def accept_probability(p_row: np.ndarray, q_row: np.ndarray, x: int) -> float:
    if q_row[x] == 0.0:
        return 1.0
    return min(1.0, p_row[x] / q_row[x])


def corrected_distribution(p_row: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    r = np.maximum(0.0, p_row - q_row)
    R = r.sum()
    return r / R if R > 0 else p_row.copy()


def joint_first_tokens(p_table: np.ndarray, q_table: np.ndarray, prev: int, gamma: int, n: int) -> np.ndarray:
    """Exact joint distribution of the first n emitted tokens, as an array of shape
    [V] * n, starting a fresh step (gamma drafts) after token `prev`."""
    V = p_table.shape[0]
    p_table = np.asarray(p_table, dtype=np.float64)
    q_table = np.asarray(q_table, dtype=np.float64)

    @lru_cache(maxsize=None)
    def dist(prev_tok: int, drafts_left: int, k: int):
        # distribution over the next k tokens, flattened, given drafts_left drafts
        # remain to be verified in the current step
        if k == 0:
            return np.ones(1)
        res = np.zeros(V ** k)
        p_row, q_row = p_table[prev_tok], q_table[prev_tok]
        if drafts_left == 0:
            # every draft of the step accepted: one extra token from p
            for x in range(V):
                tail = dist(x, gamma, k - 1)
                res[x * V ** (k - 1):(x + 1) * V ** (k - 1)] += p_row[x] * tail
            return res
        corr = corrected_distribution(p_row, q_row)
        reject_mass = 0.0
        for d in range(V):
            a = accept_probability(p_row, q_row, d)
            tail = dist(d, drafts_left - 1, k - 1)
            res[d * V ** (k - 1):(d + 1) * V ** (k - 1)] += q_row[d] * a * tail
            reject_mass += q_row[d] * (1.0 - a)
        for x in range(V):
            if corr[x] == 0.0:
                continue
            tail = dist(x, gamma, k - 1)
            res[x * V ** (k - 1):(x + 1) * V ** (k - 1)] += reject_mass * corr[x] * tail
        return res

    return dist(int(prev), int(gamma), int(n)).reshape([V] * n)


def dense_joint(p_table: np.ndarray, prev: int, n: int) -> np.ndarray:
    """prod_t p(x_t | x_{t-1}) for all sequences of length n (autoregressive target)."""
    V = p_table.shape[0]
    out = np.asarray(p_table[prev], dtype=np.float64)
    for _ in range(n - 1):
        out = out[..., None] * p_table.reshape([1] * (out.ndim - 1) + [V, V])
        # out[..., x_prev, x_next]: multiply by p(x_next | x_prev) along the last axis
    return out
