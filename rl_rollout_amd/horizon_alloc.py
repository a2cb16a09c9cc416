"""A draft horizon per sequence.

The pages report acceptance falling with the draft position and leave a shorter,
adaptive horizon to future work (wispaper.ai, "Acceptance falls at later draft
positions"). With the ragged entry points every sequence b can draft its own
gamma_b tokens in one step: the drafts skip the sequences whose horizon is
reached, the verify block of b is its first gamma_b + 1 queries and the accept
tests b's first gamma_b drafts.

Choosing gamma_b: a draft at position k adds prod_{j<=k} alpha_j expected tokens
to its sequence whatever the sequence's length, while its reads grow with the
length (the budget's share of the history plus the tail), and the accept reads
two more logit rows. The step's time is shared by the batch, so the choice is the
ratio problem of rl_rollout_amd.budget_alloc with horizons as the choices:
    E_b(g) = 1 + sum_{k<=g} prod_{j<=k} alpha_j
    c_b(g) = beta_key x (keys b's drafts 1..g attend) + beta_row x 2 g
and the budget-independent remainder T0 of the step (verify, selection, the
fixed part of every launch).

run(): on the ragged workload with the 1.7B-like position profile (256
sequences, lengths 1K..16K, gamma_max = 6, s = 0.05):
  1. every uniform horizon g = 1 .. 6: emitted tokens per second of GPU time and
     the per-position acceptance alpha_j (at g = 6);
  2. the draft kernel's time against the keys it attends, from draft steps with
     the longest 0, 1/4, 1/2 and 3/4 of the sequences skipped;
  3. the accept kernel's time against the logit rows it reads, from the uniform
     runs;
  4. for every block size G = max_b gamma_b (which sets the verify launch, so
     the remainder T0 is the uniform step at G less the modelled per-sequence
     costs), the allocation within 0 .. G; the best, and a measured run with it.
Run: python -m rl_rollout_amd.horizon_alloc [--steps K]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from .budget_alloc import allocate


def expected_tokens(alpha, gamma_max):
    """E(g) for g = 0 .. gamma_max from per-position acceptance alpha_1.."""
    a = np.asarray(alpha, dtype=np.float64)[:gamma_max]
    return np.concatenate([[1.0], 1.0 + np.cumsum(np.cumprod(a))])


def draft_keys_by_position(lens, nsel, gamma_max, page_size=16):
    """[B][gamma_max]: keys draft j attends for each sequence (selected full
    pages, the partial last page of the history and the j in-flight rows)."""
    L = np.asarray(lens, dtype=np.int64)
    base = np.asarray(nsel, dtype=np.int64) * page_size + L % page_size
    return base[:, None] + np.arange(1, gamma_max + 1)[None, :]


def horizon_costs(keys_by_pos, beta_key, beta_row):
    """[B][gamma_max + 1]: the step time sequence b adds at each horizon g."""
    cum = np.concatenate([np.zeros((keys_by_pos.shape[0], 1)), np.cumsum(keys_by_pos, axis=1)], axis=1)
    g = np.arange(keys_by_pos.shape[1] + 1)[None, :]
    return beta_key * cum + beta_row * 2 * g


def run(workload, steps, seed, warm_cache):
    import torch

    from . import workloads as W
    from .measure import OpTimer, cache_flush
    from .step import DecodeStep, build_inputs

    torch.cuda.set_device(0)
    w = W.BY_NAME[workload]
    gm, B = w.gamma, w.num_seqs
    n_runs = gm + 3
    total = (steps + 1) * n_runs + 8
    layers, table, ctx, acc, max_pages, _ = build_inputs(w, seed, total)
    init_lens = ctx.clone()
    sweep = cache_flush(torch)

    def flush():
        if not warm_cache:
            sweep()

    timer = OpTimer(torch)
    st = DecodeStep(layers, table, ctx, acc, gm, w.budget, w.temperature, before_attn=flush, run=timer.run)
    s0 = [0]

    def run_steps(n, gamma, horizons=None):
        """n timed steps after one untimed one (which also loads the kernels it uses)."""
        ctx.copy_(init_lens)
        st.seed_scores()
        hz = None if horizons is None else torch.from_numpy(np.asarray(horizons, dtype=np.int32)).cuda()
        g_arg = None if gamma == gm else gamma
        st.run(s0[0], g_arg, hz)
        torch.cuda.synchronize()
        start = ctx.clone()
        timer.reset()
        A = []
        for i in range(1, n + 1):
            st.run(s0[0] + i, g_arg, hz)
            A.append(st.num_accepted.clone())
        torch.cuda.synchronize()
        s0[0] += n + 1
        emitted = int((ctx - start).sum().item())
        op_s = sum(sum(timer.ms(o)) for o in timer.pairs) / 1e3
        ops = {o: float(np.mean(timer.ms(o))) * 1e-3 for o in timer.pairs}
        return emitted, op_s, np.stack([a.cpu().numpy() for a in A]), ops

    lens0 = init_lens.cpu().numpy().astype(np.int64)
    uniform = []
    for g in range(1, gm + 1):
        emitted, op_s, A, ops = run_steps(steps, g)
        r = {"horizon": g, "emitted_tokens_per_s": emitted / op_s, "step_us": op_s / steps * 1e6,
             "accept_us": ops["accept"] * 1e6, "verify_us": ops["verify"] * 1e6,
             "draft_us": [round(ops[f"draft{j}"] * 1e6, 1) for j in range(1, g + 1)]}
        if g == gm:
            reach = np.array([np.sum(A >= j - 1) for j in range(1, gm + 1)], dtype=np.float64)
            keep = np.array([np.sum(A >= j) for j in range(1, gm + 1)], dtype=np.float64)
            r["alpha_per_position"] = [round(float(x), 4) for x in keep / reach]
        uniform.append(r)
        print(json.dumps(r), flush=True)
    alpha = uniform[-1]["alpha_per_position"]

    # draft kernel time against attended keys: the longest fraction f of the
    # sequences skipped (horizon 0) at every draft step of a full-horizon step
    ctx.copy_(init_lens)
    st.seed_scores()
    torch.cuda.synchronize()
    nsel0 = st.nsel[0].cpu().numpy()
    keys = draft_keys_by_position(lens0, nsel0, gm)
    order = np.argsort(-lens0, kind="stable")
    pts_k, pts_t = [], []
    for frac in (0.0, 0.25, 0.5, 0.75):
        hz = np.full(B, gm, dtype=np.int32)
        hz[order[: int(frac * B)]] = 0
        hz_t = torch.from_numpy(hz).cuda()
        for rep in range(2):
            timer.reset()
            for j in range(1, gm + 1):
                st.draft_phase(j, hz_t)
            torch.cuda.synchronize()
            for j in range(1, gm + 1):
                pts_k.append(float(np.sum(keys[hz >= j, j - 1])))
                pts_t.append(timer.ms(f"draft{j}")[0] * 1e-3)
    beta_key, draft_fixed = np.polyfit(pts_k, pts_t, 1)
    fit_draft = float(np.max(np.abs(draft_fixed + beta_key * np.array(pts_k) - pts_t) / np.array(pts_t))) * 100
    rows = np.array([B * (2 * g + 1) for g in range(1, gm + 1)], dtype=np.float64)
    acc_t = np.array([r["accept_us"] for r in uniform]) * 1e-6
    beta_row, acc_fixed = np.polyfit(rows, acc_t, 1)

    # The block size G = max_b gamma_b sets the verify launch (its query tile and
    # staging), so the remainder T0 is taken per G from the uniform step at G, and
    # the horizons are allocated within 0 .. G for every G; the best G wins.
    cost = horizon_costs(keys, beta_key, beta_row)            # [B][gm + 1]
    E = expected_tokens(alpha, gm)                            # [gm + 1]
    per_block = []
    for G in range(1, gm + 1):
        T0_G = uniform[G - 1]["step_us"] * 1e-6 - float(np.sum(cost[:, G]))
        ch, rate, rounds = allocate(E[:G + 1], cost[:, :G + 1], T0_G)
        per_block.append((rate, G, ch, T0_G, rounds))
    pred, G, choice, T0, rounds = max(per_block, key=lambda x: x[0])
    emitted, op_s, A, _ = run_steps(steps, G, choice)
    best = max(uniform, key=lambda x: x["emitted_tokens_per_s"])
    classes = {}
    for g in range(gm + 1):
        idx = choice == g
        if idx.any():
            classes[str(g)] = {"sequences": int(idx.sum()), "length_range": [int(lens0[idx].min()),
                                                                               int(lens0[idx].max())]}
    out = {
        "workload": w.name, "steps": steps,
        "draft_fit": {"us_fixed": draft_fixed * 1e6, "ns_per_key": beta_key * 1e9, "max_rel_err_pct": fit_draft},
        "accept_fit": {"us_fixed": acc_fixed * 1e6, "ns_per_row": beta_row * 1e9},
        "block_size": G, "T0_us": T0 * 1e6,
        "predicted_by_block_size": [round(x[0], 1) for x in per_block],
        "expected_tokens_by_horizon": [round(float(x), 4) for x in E],
        "dinkelbach_rounds": rounds, "allocation": classes,
        "predicted_emitted_tokens_per_s": pred,
        "measured_emitted_tokens_per_s": emitted / op_s, "step_us": op_s / steps * 1e6,
        "best_uniform_horizon": best["horizon"],
        "best_uniform_emitted_tokens_per_s": best["emitted_tokens_per_s"],
        "vs_best_uniform": (emitted / op_s) / best["emitted_tokens_per_s"],
    }
    print(json.dumps(out), flush=True)
    return uniform, out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="ragged_b256_ctx1k_16k_position_profile")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--seed", type=int, default=5)
    ap.add_argument("--warm-cache", action="store_true")
    args = ap.parse_args(argv)
    return run(args.workload, args.steps, args.seed, args.warm_cache)


if __name__ == "__main__":
    main(sys.argv[1:])
