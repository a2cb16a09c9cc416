"""KV-aware admission study: pages moved per 1,000 generated tokens and the
attention-path throughput of a rollout batch under a fixed concurrency cap and
under the AIMD limit, with offload or recompute of paused requests.

The pages report, against a fixed cap of 256 with offload, 18.0 -> 1.3 pages
moved per 1,000 tokens and 6014.9 -> 6362.1 generated tokens per GPU-second
(rebasdaily.com, "真正难搬的，还是那叠完整笔记"; wispaper.ai, "Where the speedup
claim holds": 0.144M recompute-plus-moved pages against 5.362M for recompute and
2.024M for offload).

Method:
  1. on the GPU, the page moves of this library: s3r_pack_pages of 2048 random
     blocks of a 1.7B-like layer (8 kv heads, d 128, bf16: 64 KB per page) into a
     device staging buffer, then a copy into pinned host memory (offload), and the
     reverse (restore): event-timed, bytes per second each way;
  2. on the host, rl_rollout_amd.kv_scheduler runs one rollout batch (256 prompts
     x 8 responses, prompts 128..1024 tokens, responses log-normal around 3000,
     at most 16384) to completion for each pool size, controller and policy; each
     running request emits 1 + a tokens per step, a the accepted drafts of gamma =
     4 with per-position acceptance 0.88 (the 1.7B-like workload's measured rate);
  3. time of the attention path: per step and layer, the verify's and drafts'
     bytes at the rates measured by bench.py (6.45 and 5.26 TB/s), a fixed
     25 us per layer (selection, append and launch gaps), the accept at 1 us per
     request once per step, over 28 layers; plus the moved pages' bytes (28 layers)
     at the measured move rates. Recompute's prefill is not priced: its count is
     reported as pages recomputed.
Run: python -m rl_rollout_amd.kv_sched_study
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from .kv_scheduler import AIMD, FixedCap, rollout_batch, simulate

LAYERS = 28
PAGE_BYTES_LAYER = 8 * 16 * 128 * 2 * 2      # K and V tiles of 8 kv heads, d 128, bf16
VERIFY_BPS = 6.45e12
DRAFT_BPS = 5.26e12
LAYER_FIXED_S = 25e-6
ACCEPT_PER_REQ_S = 1.0e-6
ALPHA = 0.88
GAMMA = 4
BUDGET = 0.05


def measure_moves(pages=2048, reps=5):
    """Event-timed offload (pack + device-to-host) and restore (host-to-device +
    unpack) of `pages` random pages; returns bytes per second each way."""
    import torch

    from . import s3r

    torch.cuda.set_device(0)
    nb = 8192
    k = torch.randn((nb, 8, 16, 128), device="cuda").to(torch.bfloat16)
    v = torch.randn((nb, 8, 128, 16), device="cuda").to(torch.bfloat16)
    table = torch.zeros((1, nb), dtype=torch.int32, device="cuda")
    lens = torch.zeros((1,), dtype=torch.int32, device="cuda")
    kv = s3r.KVCache(k, v, table, lens)
    rng = np.random.default_rng(0)
    blocks = torch.from_numpy(rng.choice(nb, size=pages, replace=False).astype(np.int32)).cuda()
    pb = s3r.page_bytes(kv)
    staging = torch.empty((pages, pb), dtype=torch.uint8, device="cuda")
    host = torch.empty((pages, pb), dtype=torch.uint8, pin_memory=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    off, res = [], []
    for _ in range(reps + 1):
        ev[0].record()
        s3r.s3r_pack_pages(kv, blocks, staging)
        ev[1].record()
        host.copy_(staging, non_blocking=True)
        ev[2].record()
        staging.copy_(host, non_blocking=True)
        ev[3].record()
        s3r.s3r_unpack_pages(kv, blocks, staging)
        ev[4].record()
        torch.cuda.synchronize()
        off.append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])))
        res.append((ev[2].elapsed_time(ev[3]), ev[3].elapsed_time(ev[4])))
    off, res = np.array(off[1:]), np.array(res[1:])
    nbytes = pages * pb
    return {
        "pages": pages, "page_bytes": pb,
        "pack_us": float(np.median(off[:, 0]) * 1e3), "device_to_host_us": float(np.median(off[:, 1]) * 1e3),
        "host_to_device_us": float(np.median(res[:, 0]) * 1e3), "unpack_us": float(np.median(res[:, 1]) * 1e3),
        "offload_bytes_per_s": nbytes / (np.median(off.sum(axis=1)) * 1e-3),
        "restore_bytes_per_s": nbytes / (np.median(res.sum(axis=1)) * 1e-3),
    }


def tokens_per_step(rng, n):
    """1 + accepted drafts of gamma drafts, each kept with ALPHA while the prefix holds."""
    a = np.zeros(n, dtype=np.int64)
    alive = np.ones(n, dtype=bool)
    for _ in range(GAMMA):
        alive &= rng.random(n) < ALPHA
        a += alive
    return a + 1


def attention_seconds(trace):
    """Modelled attention-path time of the steps in a simulate() trace."""
    running, kv = trace[:, 0].astype(np.float64), trace[:, 1].astype(np.float64)
    G1 = GAMMA + 1
    tok_bytes = PAGE_BYTES_LAYER / 16
    verify = (kv + running * G1) * tok_bytes / VERIFY_BPS
    drafts = GAMMA * (BUDGET * kv + running * 16) * tok_bytes / DRAFT_BPS
    return float(np.sum(LAYERS * (verify + drafts + LAYER_FIXED_S) + running * ACCEPT_PER_REQ_S))


def run(pool_tokens, seed, moves):
    rows = []
    for pool in pool_tokens:
        for ctl_name in ("fixed256", "aimd"):
            for policy in ("offload", "recompute"):
                reqs = rollout_batch(256, 8, seed)
                ctl = FixedCap(256) if ctl_name == "fixed256" else AIMD()
                s, tr = simulate(reqs, pool // 16, ctl, policy, tokens_per_step, seed + 1)
                gen = int(tr[:, 2].sum())
                t_attn = attention_seconds(tr)
                off_b = s.pages_offloaded * PAGE_BYTES_LAYER * LAYERS
                res_b = s.pages_restored * PAGE_BYTES_LAYER * LAYERS
                t_move = off_b / moves["offload_bytes_per_s"] + res_b / moves["restore_bytes_per_s"]
                r = {"pool_tokens": pool, "controller": ctl_name, "policy": policy, "steps": s.steps,
                     "generated_tokens": gen,
                     "pages_moved_per_1k_tokens": (s.pages_offloaded + s.pages_restored) / gen * 1000,
                     "pages_recomputed_per_1k_tokens": s.pages_recomputed / gen * 1000,
                     "pages_moved_or_recomputed": s.pages_offloaded + s.pages_restored + s.pages_recomputed,
                     "mean_running": float(tr[:, 0].mean()), "mean_kv_utilisation": float(tr[:, 1].mean() / pool),
                     "attention_s": t_attn, "move_s": t_move,
                     # recompute's prefill is not priced, so it gets no throughput figure
                     "tokens_per_s_attention_path": gen / (t_attn + t_move) if policy == "offload" else None}
                rows.append(r)
                print(json.dumps(r), flush=True)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--pools", default="400000,700000,1000000", help="pool sizes in tokens")
    ap.add_argument("--no-gpu", action="store_true", help="skip the move measurement (assume 25 GB/s each way)")
    args = ap.parse_args(argv)
    if args.no_gpu:
        moves = {"offload_bytes_per_s": 25e9, "restore_bytes_per_s": 25e9, "measured": False}
    else:
        moves = measure_moves()
    print(json.dumps({"page_moves": moves}), flush=True)
    return run([int(x) for x in args.pools.split(",")], args.seed, moves)


if __name__ == "__main__":
    main(sys.argv[1:])
