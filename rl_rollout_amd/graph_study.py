"""Wall-clock time per step, eager launches against one HIP-graph replay per step
(rl_rollout_amd.step.StepGraph), warm cache.

A step issues about 8 launches per layer plus the accept's 3 (drafts, block
append, verify and its page-score pass, selection). With short histories or few
sequences the kernels take microseconds, and the host's launch path (Python,
the C ABI's checks, the runtime) sets the step time. A graph replay issues the
whole step at once. Measured after one eager step and the capture, with a host
sync before and after each timed run of `steps` steps.
Run: python -m rl_rollout_amd.graph_study [--steps K]
"""
from __future__ import annotations

import argparse
import json
import sys
import time


CASES = [
    # name, workload overrides
    ("8 seqs, 1K-3K ctx, 1 layer", dict(num_seqs=8, ctx_range=(1000, 3000))),
    ("8 seqs, 1K-3K ctx, 28 layers", dict(num_seqs=8, ctx_range=(1000, 3000), num_layers=28)),
    ("64 seqs, 16K ctx, 1 layer", dict()),
]


def run(steps: int, seed: int):
    import torch

    from . import workloads as W
    from .step import DecodeStep, StepGraph, build_inputs

    torch.cuda.set_device(0)
    rows = []
    for name, over in CASES:
        w = W.QWEN3_1P7B_16K.with_(**over)
        layers, table, ctx, acc, _, _ = build_inputs(w, seed, 2 * steps + 4)
        st = DecodeStep(layers, table, ctx, acc, w.gamma, w.budget, w.temperature)
        st.seed_scores()
        st.run(0)
        torch.cuda.synchronize()
        graph = StepGraph(st)
        init = ctx.clone()

        def timed(fn, first):
            ctx.copy_(init)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                fn(first + i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / steps

        eager = timed(st.run, 1)
        replay = timed(graph.replay, 1 + steps)
        r = {"case": name, "layers": w.num_layers, "steps": steps, "eager_ms_per_step": eager * 1e3,
             "graph_ms_per_step": replay * 1e3, "speedup": eager / replay}
        rows.append(r)
        print(json.dumps(r), flush=True)
        del st, graph, layers, table, ctx, acc
        torch.cuda.empty_cache()
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--seed", type=int, default=6)
    args = ap.parse_args(argv)
    return run(args.steps, args.seed)


if __name__ == "__main__":
    main(sys.argv[1:])
