"""One sparse budget per sequence.

The pages show draft acceptance rising with the sparse budget while the drafts'
reads grow with it until they outweigh the gain, and name adaptive budgets as
future work (wispaper.ai, "What to watch before adopting S3R" and "Where the
speedup claim holds"). Under one budget for the batch every sequence drafts from
the same fraction of its history. A sequence's draft reads are that fraction of
its length, while its gain in tokens from a larger budget does not depend on its
length (the acceptance-versus-budget relation the pages print for a batch, read
as holding per sequence). The step's time is shared by the batch, so a larger
budget costs less step time per token gained on a short sequence than on a long
one.

allocate() picks one budget per sequence from a candidate set to maximise the
emitted tokens per second of step time,
    R = sum_b E_b(s_b) / (T0 + sum_b c_b(s_b)),
where E_b(s) is the expected number of tokens a step emits for sequence b at
budget s, c_b(s) the step time of its drafts at that budget and T0 the step time
that does not depend on the budgets (verify, accept, selection, fixed launch
costs). It uses Dinkelbach's method for ratio objectives: with lambda the ratio
of the current choice, every sequence independently takes the budget that
maximises E_b(s) - lambda c_b(s), and lambda becomes the ratio of the new
choice. F(lambda) = max over choices of sum_b (E_b - lambda c_b) - lambda T0 is
zero exactly at the optimal ratio and positive below it; each round raises
lambda strictly while F > 0, and the inner maximum separates per sequence, so it
is exact. The search ends when F is zero (to rounding), at the optimum over all
M^B choices.

run(): on the ragged workload (256 sequences, lengths uniform in 1K..16K), measures
each budget of the calibrated set as one budget for the batch, fits the step
time as T0 + beta x draft keys per step, takes each budget's measured tokens per
step as E(s), allocates, and measures the allocation, each sequence drafting with
the calibrated draft noise of its own budget.
Run: python -m rl_rollout_amd.budget_alloc [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def pages_selected(n_full, budget):
    """Full pages a sequence with n_full full pages keeps at a budget ratio: the
    budget's share rounded up, at least one, at most n_full (0 without a full page)."""
    n = np.asarray(n_full, dtype=np.int64)
    k = np.ceil(np.asarray(budget, dtype=np.float64) * n - 1e-9).astype(np.int64)
    return np.where(n > 0, np.minimum(n, np.maximum(1, k)), 0)


def draft_keys_per_step(lens, budget, gamma, page_size=16):
    """Keys one step's gamma drafts attend for each sequence at committed lengths
    lens: the selected full pages plus the tail of draft j, 16 * floor(L / 16) <=
    t <= L + j - 1."""
    L = np.asarray(lens, dtype=np.int64)
    n_full = L // page_size
    tail = L - n_full * page_size
    sel = pages_selected(n_full, budget) * page_size
    return gamma * (sel + tail) + gamma * (gamma + 1) // 2


def ratio(tokens, cost, fixed, choice):
    rows = np.arange(tokens.shape[0])
    return float(np.sum(tokens[rows, choice]) / (fixed + np.sum(cost[rows, choice])))


def allocate(tokens, cost, fixed, max_rounds=1000):
    """tokens, cost: [B][M] (or [M], shared by every sequence): expected tokens per
    step and draft step time of each sequence at each of M budgets; fixed: the
    budget-independent step time (> 0). Returns (choice [B] of budget indices,
    tokens per unit of step time of that choice, rounds)."""
    E, C = (np.atleast_2d(np.asarray(x, dtype=np.float64)) for x in (tokens, cost))
    E, C = (np.ascontiguousarray(x) for x in np.broadcast_arrays(E, C))
    if not fixed > 0 or np.any(C < 0) or not np.all(np.isfinite(E)) or not np.all(np.isfinite(C)):
        raise ValueError("allocate needs a positive fixed time and finite, non-negative costs")
    B, M = E.shape
    # start from the best single budget for every sequence
    uniform = [ratio(E, C, fixed, np.full(B, m)) for m in range(M)]
    choice = np.full(B, int(np.argmax(uniform)))
    lam = ratio(E, C, fixed, choice)
    rows = np.arange(B)
    for rounds in range(1, max_rounds + 1):
        v = E - lam * C
        best = np.argmax(v, axis=1)
        F = float(np.sum(v[rows, best])) - lam * fixed
        if F <= 1e-12 * max(1.0, float(np.sum(E[rows, best]))):
            return choice, lam, rounds
        choice = best
        lam = ratio(E, C, fixed, choice)
    raise RuntimeError("Dinkelbach iteration did not settle")


def run(steps, warmup, seed, warm_cache):
    import torch

    from . import workloads as W
    from .budget_sweep import run_budget
    from .measure import cache_flush

    torch.cuda.set_device(0)
    sweep = cache_flush(torch)

    def flush():
        if not warm_cache:
            sweep()

    base = W.RAGGED_SWEEP
    S, sigma = np.asarray(base.budgets), np.asarray(base.sweep_noise)
    uniform = []
    for s, sg in zip(S, sigma):
        r = run_budget(base.with_(budget=float(s), draft_noise=float(sg)), seed, steps, warmup, flush)
        uniform.append(r)
        print(json.dumps({"budget": float(s), "draft_noise": float(sg), "step_us": r["step_us"],
                          "draft_keys_per_step": r["draft_keys_per_step"], "tokens_per_step": r["tokens_per_step"],
                          "emitted_tokens_per_s": r["emitted_tokens_per_s"]}), flush=True)
    T = np.array([r["step_us"] for r in uniform]) * 1e-6
    K = np.array([r["draft_keys_per_step"] for r in uniform])
    beta, T0 = np.polyfit(K, T, 1)
    fit_err = float(np.max(np.abs(T0 + beta * K - T) / T)) * 100.0
    E = np.array([r["tokens_per_step"] for r in uniform])
    lens = uniform[0]["lens_at_start"]
    cost = beta * np.stack([draft_keys_per_step(lens, s, base.gamma) for s in S], axis=1)
    choice, pred, rounds = allocate(E, cost, T0)
    r = run_budget(base.with_(budget=float(S[choice].max())), seed, steps, warmup, flush,
                   budgets=S[choice].astype(np.float64), seq_noise=sigma[choice].astype(np.float32))
    best = max(uniform, key=lambda x: x["emitted_tokens_per_s"])
    per_class = {}
    for m, s in enumerate(S):
        idx = choice == m
        if idx.any():
            per_class[str(float(s))] = {
                "sequences": int(idx.sum()),
                "length_range": [int(lens[idx].min()), int(lens[idx].max())],
                "acceptance": float(np.mean(r["accepted_per_seq"][idx]) / base.gamma),
                "acceptance_at_this_budget_for_the_batch": uniform[m]["acceptance"],
            }
    out = {
        "workload": base.name, "steps": steps,
        "step_time_fit": {"T0_us": T0 * 1e6, "ns_per_draft_key": beta * 1e9, "max_rel_err_pct": fit_err},
        "dinkelbach_rounds": rounds,
        "allocation": per_class,
        "predicted_emitted_tokens_per_s": pred,
        "measured_emitted_tokens_per_s": r["emitted_tokens_per_s"],
        "step_us": r["step_us"],
        "best_uniform_budget": best["budget"],
        "best_uniform_emitted_tokens_per_s": best["emitted_tokens_per_s"],
        "vs_best_uniform": r["emitted_tokens_per_s"] / best["emitted_tokens_per_s"],
    }
    print(json.dumps(out), flush=True)
    return uniform, out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=6)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--warm-cache", action="store_true")
    args = ap.parse_args(argv)
    return run(args.steps, args.warmup, args.seed, args.warm_cache)


if __name__ == "__main__":
    main(sys.argv[1:])
