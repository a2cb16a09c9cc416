"""Page sets per sequence vs per kv head: what the sparse draft keeps.

Selection is by summed attention scores (rit.work, "Как разреженный черновик
сохраняет ответы плотной модели"); the pages leave context selection itself to
future work (wispaper.ai, "What to watch before adopting S3R"). With one page
set per sequence, every kv head attends the pages the heads chose together; with
one set per kv head, each head keeps the pages its own query heads weight most.
Both read the same number of pages, so the draft moves the same bytes.

For one verify step of a workload this measures, per (sequence, kv head):
  * captured mass: the share of the head's verify softmax mass over the full
    pages that lies on the selected pages;
  * the draft error: the relative error of the first draft step's attention
    output against dense attention of the same query (the verify kernel with a
    one-query block at the draft position);
  * the draft launch time of both selections.

Run: python -m rl_rollout_amd.selection_study [--workload NAME] [--budget S]
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np


def run(workload: str, budget: float, seed: int):
    import torch

    from . import s3r
    from . import workloads as W
    from .measure import FLUSH_BYTES
    from .step import build_inputs

    torch.cuda.set_device(0)
    w = W.BY_NAME[workload].with_(budget=budget)
    layers, table, ctx, acc, max_pages, _ = build_inputs(w, seed, 2)
    lay = layers[0]
    kv = s3r.KVCache(lay["k_cache"], lay["v_cache"], table, ctx)
    B, H, G1 = w.num_seqs, w.num_kv_heads, w.block_len
    s3r.s3r_append_kv(kv, lay["k_block"], lay["v_block"], offset=0)
    _, hs = s3r.s3r_dense_verify_attn_head_scores(kv, lay["q_verify"])      # [B][H][P]
    shared = hs.sum(dim=1).contiguous()                                       # [B][P]
    max_sel = max(1, math.ceil(budget * max_pages))
    sel_s, ns_s = s3r.s3r_select_budget(shared, ctx, budget, max_sel)
    lens_rows = ctx.repeat_interleave(H).contiguous()
    sel_h, ns_h = s3r.s3r_select_budget(hs.view(B * H, -1), lens_rows, budget, max_sel)
    sel_h, ns_h = sel_h.view(B, H, max_sel), ns_h.view(B, H)

    # captured mass of each head's full-page scores
    n_full = (ctx // 16).long()
    P = hs.shape[2]
    full = (torch.arange(P, device="cuda")[None, :] < n_full[:, None]).float()          # [B][P]
    total = (hs * full[:, None, :]).sum(dim=2)                                           # [B][H]

    def captured(sel, ns):
        s = sel.long().clamp_min(0)
        valid = (torch.arange(sel.shape[-1], device="cuda") < ns[..., None]).float()
        return (torch.gather(hs, 2, s) * valid).sum(dim=2) / total.clamp_min(1e-30)

    cap_s = captured(sel_s[:, None, :].expand(B, H, max_sel).contiguous(), ns_s[:, None].expand(B, H))
    cap_h = captured(sel_h, ns_h)

    # first draft step: both selections against dense attention of the same query
    j = 1
    q = lay["q_draft"][j - 1]
    s3r.s3r_append_kv(kv, lay["k_draft"][j - 1], lay["v_draft"][j - 1], offset=j - 1)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(5):
            flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r = fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return r, float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3

    o_s, t_s = timed(lambda: s3r.s3r_sparse_draft_attn(kv, q, sel_s, ns_s, j))
    o_h, t_h = timed(lambda: s3r.s3r_sparse_draft_attn_head_sel(kv, q, sel_h.contiguous(), ns_h.contiguous(), j))
    kv_d = s3r.KVCache(kv.k_cache, kv.v_cache, table, (ctx + (j - 1)).contiguous())
    dense, _ = s3r.s3r_dense_verify_attn(kv_d, q[:, None].contiguous(), want_scores=False)
    dense = dense[:, 0].float()

    def rel_err(o):
        o = o.float()
        return ((o - dense).norm(dim=-1) / dense.norm(dim=-1).clamp_min(1e-30)).view(B, H, -1)

    e_s, e_h = rel_err(o_s), rel_err(o_h)
    res = {
        "workload": w.name, "budget": budget, "pages_per_set_mean": float(ns_s.float().mean()),
        "captured_mass_shared_mean": float(cap_s.mean()), "captured_mass_per_head_mean": float(cap_h.mean()),
        "captured_mass_gain_min": float((cap_h - cap_s).min()),
        "draft_rel_err_shared_mean": float(e_s.mean()), "draft_rel_err_per_head_mean": float(e_h.mean()),
        "draft_rel_err_shared_max": float(e_s.max()), "draft_rel_err_per_head_max": float(e_h.max()),
        "draft_us_shared": t_s, "draft_us_per_head": t_h,
    }
    print(json.dumps(res), flush=True)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="qwen3_1.7b_like_gqa16x8_d128_ctx16k_b64")
    ap.add_argument("--budget", type=float, nargs="+", default=[0.05, 0.25])
    ap.add_argument("--seed", type=int, default=4)
    args = ap.parse_args(argv)
    return [run(args.workload, s, args.seed) for s in args.budget]


if __name__ == "__main__":
    main(sys.argv[1:])
