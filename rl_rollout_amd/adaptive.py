"""Adaptive draft horizon from position-dependent acceptance.

The pages report that draft acceptance falls with the draft position and that
late positions decline further as training proceeds, and suggest a draft
horizon that shortens when late-position acceptance deteriorates (wispaper.ai,
"Acceptance falls at later draft positions"; they leave it to future work).

HorizonController keeps a running estimate of the acceptance alpha_j of each
draft position j (the fraction of sequences that reached position j whose draft
j was kept, with exponential forgetting) and picks, before each step, the
horizon gamma in 1 .. gamma_max that maximises the expected tokens per unit of
step time:
    E[tokens](gamma) = 1 + sum_{k <= gamma} prod_{j <= k} alpha_j
    time(gamma)      = a running mean of the measured step times at gamma, which
                       starts from a model (fixed cost + gamma x per-draft cost +
                       the accept pass, whose rows grow with gamma, all measured
                       at gamma_max) and follows the steps actually run at gamma.
The measured times matter where the model is off: the verify block of gamma + 1
queries changes mode with gamma (one or two MFMA column tiles), which a cost
linear in gamma does not see.
Positions beyond the current horizon stop producing observations, so every
`explore_every`-th step runs the full horizon to refresh them.

run(): on a position-profile workload, measures every fixed horizon and the
adaptive controller, first with the earlier-training profile and then with the
later one. Run: python -m rl_rollout_amd.adaptive [--workload NAME] [--steps K]
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Callable, Sequence

import numpy as np


class HorizonController:
    def __init__(self, gamma_max: int, cost: Callable[[int], float], prior: float = 0.8, prior_weight: float = 4.0,
                 decay: float = 0.9, explore_every: int = 16, time_prior_weight: float = 2.0,
                 time_decay: float = 0.8):
        self.gamma_max = gamma_max
        self.cost = cost
        self.decay = decay
        self.explore_every = explore_every
        self.reach = np.full(gamma_max, prior_weight, dtype=np.float64)
        self.keep = np.full(gamma_max, prior * prior_weight, dtype=np.float64)
        # step time per horizon: weighted sum and weight, the model's value as prior
        self.time_decay = time_decay
        self.t_weight = np.full(gamma_max, time_prior_weight, dtype=np.float64)
        self.t_sum = np.array([cost(g) for g in range(1, gamma_max + 1)], dtype=np.float64) * self.t_weight
        self.steps = 0

    def step_time(self, gamma: int) -> float:
        return float(self.t_sum[gamma - 1] / self.t_weight[gamma - 1])

    def observe_time(self, gamma: int, seconds: float) -> None:
        """The measured GPU time of one step run at horizon gamma."""
        self.t_sum[gamma - 1] = self.time_decay * self.t_sum[gamma - 1] + seconds
        self.t_weight[gamma - 1] = self.time_decay * self.t_weight[gamma - 1] + 1.0

    def alpha(self) -> np.ndarray:
        return self.keep / np.maximum(self.reach, 1e-12)

    def expected_tokens(self, gamma: int, alpha: Sequence[float] = None) -> float:
        a = self.alpha() if alpha is None else np.asarray(alpha, dtype=np.float64)
        return 1.0 + float(np.sum(np.cumprod(a[:gamma])))

    def choose(self) -> int:
        self.steps += 1
        if self.explore_every and self.steps % self.explore_every == 0:
            return self.gamma_max
        rates = [self.expected_tokens(g) / self.step_time(g) for g in range(1, self.gamma_max + 1)]
        return int(np.argmax(rates)) + 1

    def update(self, num_accepted: np.ndarray, gamma: int) -> None:
        """Observations of one step run at horizon gamma: a_b drafts kept per sequence."""
        a = np.asarray(num_accepted)
        self.reach[:gamma] *= self.decay
        self.keep[:gamma] *= self.decay
        for j in range(1, gamma + 1):
            self.reach[j - 1] += float(np.sum(a >= j - 1))
            self.keep[j - 1] += float(np.sum(a >= j))


def _run_steps(st, timer, steps, s0, gamma_of, ctx, init_lens, torch, on_step=None, warm_gamma=None):
    """steps steps from uniform index s0 + 1, after one untimed step at warm_gamma
    (which also loads the kernels that horizon uses: HIP loads a kernel's code on
    its first launch); returns (emitted tokens, GPU op seconds, horizons,
    per-position counts)."""
    gm = st.gamma
    ctx.copy_(init_lens)
    st.seed_scores()
    if warm_gamma is not None:
        st.run(s0, None if warm_gamma == gm else warm_gamma)
    s0 += 1
    torch.cuda.synchronize()
    timer.reset()
    reach, keep = np.zeros(gm), np.zeros(gm)
    used = []
    start = ctx.clone()
    for i in range(steps):
        g = gamma_of()
        used.append(g)
        n_before = {o: len(v) for o, v in timer.pairs.items()}
        st.run(s0 + i, None if g == gm else g)
        a = st.num_accepted.cpu().numpy()  # synchronises: this step's events are complete
        step_s = sum(s_.elapsed_time(e_) for o, v in timer.pairs.items() for s_, e_ in v[n_before.get(o, 0):]) / 1e3
        for j in range(1, g + 1):
            reach[j - 1] += np.sum(a >= j - 1)
            keep[j - 1] += np.sum(a >= j)
        if on_step is not None:
            on_step(a, g, step_s)
    torch.cuda.synchronize()
    emitted = int((ctx - start).sum().item())
    op_s = sum(sum(timer.ms(o)) for o in list(timer.pairs)) / 1e3
    return emitted, op_s, used, reach, keep


def run(workload: str, steps: int, seed: int, warm_cache: bool):
    import torch

    from . import synth
    from . import workloads as W
    from .measure import OpTimer, cache_flush
    from .step import DecodeStep, build_inputs

    torch.cuda.set_device(0)
    w = W.BY_NAME[workload]
    gm = w.gamma
    profiles = [("early", w.position_noise)] + ([("late", w.late_position_noise)] if w.late_position_noise else [])
    n_runs = len(profiles) * (gm + 2)
    total = (steps + 1) * n_runs + 16
    layers, table, ctx, acc, max_pages, _ = build_inputs(w, seed, total)
    init_lens = ctx.clone()
    sweep = cache_flush(torch)

    def flush():
        if not warm_cache:
            sweep()

    timer = OpTimer(torch)
    st = DecodeStep(layers, table, ctx, acc, gm, w.budget, w.temperature, before_attn=flush, run=timer.run)
    B = w.num_seqs
    results = []
    s0 = 0
    for pname, noise in profiles:
        if pname != "early":
            st.replace_accept(synth.device_accept_inputs(w.with_(position_noise=noise), seed, total))
        # per-op costs at the full horizon, for the controller's time model
        emitted, op_s, _, _, _ = _run_steps(st, timer, 4, s0, lambda: gm, ctx, init_lens, torch, warm_gamma=gm)
        s0 += 5
        t = {o: float(np.mean(timer.ms(o))) * 1e-3 for o in timer.pairs}
        # an append launch per draft only when the drafts do not read their rows
        # from the draft-row buffers; the verify block's append in either mode
        per_draft = float(np.mean([t[f"draft{j}"] for j in range(1, gm + 1)]))
        if not st.draft_rows:
            per_draft += t.get("append", 0.0)
        fixed = t["verify"] + t["select"] + t.get("append", 0.0)

        def cost(g, t=t, per_draft=per_draft, fixed=fixed):
            return fixed + g * per_draft + t["accept"] * (2 * g + 1) / (2 * gm + 1)

        for g in range(1, gm + 1):
            emitted, op_s, used, reach, keep = _run_steps(st, timer, steps, s0, lambda g=g: g, ctx, init_lens, torch,
                                                          warm_gamma=g)
            s0 += steps + 1
            r = {"profile": pname, "horizon": g, "emitted_tokens_per_s": emitted / op_s,
                 "tokens_per_step": emitted / (B * steps),
                 "alpha_per_position": [round(float(k / r_), 4) if r_ else None for k, r_ in zip(keep, reach)]}
            results.append(r)
            print(json.dumps(r), flush=True)
        ctl = HorizonController(gm, cost)
        def observe(a, g, step_s):
            ctl.update(a, g)
            ctl.observe_time(g, step_s)

        emitted, op_s, used, reach, keep = _run_steps(st, timer, steps, s0, ctl.choose, ctx, init_lens, torch,
                                                      on_step=observe)
        s0 += steps + 1
        fixed_best = max((r for r in results if r["profile"] == pname), key=lambda r: r["emitted_tokens_per_s"])
        r = {"profile": pname, "horizon": "adaptive", "emitted_tokens_per_s": emitted / op_s,
             "tokens_per_step": emitted / (B * steps), "mean_horizon": float(np.mean(used)),
             "horizon_counts": {int(k): int(v) for k, v in zip(*np.unique(used, return_counts=True))},
             "alpha_estimate": [round(float(x), 4) for x in ctl.alpha()],
             "best_fixed_horizon": fixed_best["horizon"],
             "vs_best_fixed": (emitted / op_s) / fixed_best["emitted_tokens_per_s"],
             "vs_full_horizon": (emitted / op_s) / next(x["emitted_tokens_per_s"] for x in results
                                                          if x["profile"] == pname and x["horizon"] == gm)}
        results.append(r)
        print(json.dumps(r), flush=True)
    return results


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="qwen3_8b_like_gqa32x8_d128_ctx24k_b128_position_profile")
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--warm-cache", action="store_true")
    args = ap.parse_args(argv)
    return run(args.workload, args.steps, args.seed, args.warm_cache)


if __name__ == "__main__":
    main(sys.argv[1:])
