"""Draft-noise calibration for the synthetic acceptance profiles.

The synthetic draft logits are target logits plus N(0, sigma^2) noise. For a
draft token drawn from q the probability that exact speculative sampling keeps
it is sum_x min(p(x), q(x)) (one minus the total-variation distance of p and q),
so the acceptance a sigma gives can be computed directly. This tool estimates
that acceptance over seeded target rows and inverts it by bisection; its results
are the constants stored in workloads.py (it is not imported by the kernels'
path or by the input generators).

Profiles it is used for (wispaper.ai, "Acceptance falls at later draft
positions"): Qwen3-8B at training step 20 keeps 95.8% of first-position drafts
and 67.9% of sixth-position drafts, and at step 100 1.6 and 6.6 points fewer;
Qwen3-1.7B 95.0% and 62.9%. Intermediate
positions are not printed; the reading taken is linear in position, which
reproduces the printed checkpoint-level rate (the mean of 95.8 and 67.9 is 81.85,
printed 81.9).

Run: python -m rl_rollout_amd.calibrate
"""
from __future__ import annotations

import json

import numpy as np


def acceptance(sigma: float, vocab: int = 151936, target_std: float = 2.0, rows: int = 48, seed: int = 0,
               temperature: float = 1.0, bf16: bool = True) -> float:
    """Mean over seeded rows of sum_x min(p(x), q(x)), with target logits
    ~ N(0, target_std^2) and draft logits = target + N(0, sigma^2), both rounded
    to bf16 as the workloads store them."""
    from .synth import bf16_bits_to_f32, f32_to_bf16_bits

    rng = np.random.Generator(np.random.PCG64(seed))
    acc = 0.0
    for _ in range(rows):
        t = (rng.standard_normal(vocab, dtype=np.float32) * np.float32(target_std))
        d = t + rng.standard_normal(vocab, dtype=np.float32) * np.float32(sigma)
        if bf16:
            t = bf16_bits_to_f32(f32_to_bf16_bits(t))
            d = bf16_bits_to_f32(f32_to_bf16_bits(d))
        lt = t.astype(np.float64) / temperature
        ld = d.astype(np.float64) / temperature
        p = np.exp(lt - lt.max())
        p /= p.sum()
        q = np.exp(ld - ld.max())
        q /= q.sum()
        acc += float(np.minimum(p, q).sum())
    return acc / rows


def sigma_for_acceptance(alpha: float, lo: float = 0.0, hi: float = 4.0, iters: int = 40, **kw) -> float:
    """Noise sigma whose acceptance is alpha (acceptance falls as sigma grows)."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if acceptance(mid, **kw) > alpha:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def linear_profile(first: float, sixth: float, positions: int) -> list:
    """Acceptance at positions 1..positions, linear between the printed first- and
    sixth-position values."""
    return [first + (sixth - first) * (j - 1) / 5.0 for j in range(1, positions + 1)]


def main():
    out = {}
    for name, first, sixth in (("qwen3_8b_step20", 0.958, 0.679), ("qwen3_8b_step100", 0.942, 0.613),
                               ("qwen3_1.7b", 0.950, 0.629)):
        prof = linear_profile(first, sixth, 6)
        sig = [round(sigma_for_acceptance(a, rows=16, iters=24), 4) for a in prof]
        out[name] = {"acceptance": [round(a, 4) for a in prof], "sigma": sig,
                     "check": [round(acceptance(s, rows=16, seed=1), 4) for s in sig]}
        print(json.dumps({name: out[name]}), flush=True)
    return out


if __name__ == "__main__":
    main()
