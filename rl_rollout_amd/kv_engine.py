"""The KV-aware admission scheduler driving the real decode step on the GPU.

rl_rollout_amd.kv_scheduler decides which requests run; this loop runs them:
  * a fixed set of `slots` rows of one DecodeStep (one attention layer of the
    1.7B-like shape); a running request occupies a slot, whose page-table row
    holds the request's blocks (block 0 of the pool is a scratch block that every
    unused entry points at) and whose committed length is the request's; an empty
    slot has length 0, so the kernels read only its scratch page;
  * the step's own accept decides how many tokens each request emits (synthetic
    logits with the 1.7B-like draft noise, a fresh uniform per step and slot);
  * when the scheduler pauses a request its pages are packed (s3r_pack_pages) and
    copied into pinned host memory; when it restores one, they are copied back and
    unpacked (s3r_unpack_pages) into its new blocks;
  * a slot that takes a new request starts with an empty page selection, so its
    first drafts read only their tail (its previous scores belong to another
    request).
Measured per batch: GPU time of the step's kernels and of the page moves (events),
tokens generated, pages moved.
Run: python -m rl_rollout_amd.kv_engine [--pool TOKENS] [--controller aimd|fixed256]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def run(controller: str, pool_tokens: int, seed: int = 1, slots: int = 256, num_prompts: int = 256, group: int = 8,
        max_steps: int = 40000, verify_moves: bool = False, median_response: int = 3000):
    """One rollout batch to completion. verify_moves: after every restore, pack the
    new blocks again and compare them byte for byte with the pages that were
    offloaded (a check for tests; it adds work outside the timed events)."""
    import torch

    from . import s3r, synth
    from . import workloads as W
    from .kv_scheduler import AIMD, FixedCap, Scheduler, pages_for, rollout_batch
    from .measure import OpTimer
    from .step import DecodeStep

    torch.cuda.set_device(0)
    w = W.QWEN3_1P7B_16K.with_(num_seqs=slots)
    G1 = w.block_len
    reqs = rollout_batch(num_prompts, group, seed, median_response=median_response)
    max_len = max(r.prompt + r.response for r in reqs)
    maxp = pages_for(max_len + G1) + 1
    nb = pool_tokens // 16 + 1                     # block 0: scratch
    k, v = synth.device_layer_kv(w, seed, nb)
    layer = dict(k_cache=k, v_cache=v)
    layer.update(synth.device_layer_queries(w, seed, slots))
    acc = synth.device_accept_inputs(w, seed, max_steps)
    table_h = np.zeros((slots, maxp), dtype=np.int32)
    ctx_h = np.zeros((slots,), dtype=np.int32)
    table = torch.from_numpy(table_h).cuda()
    ctx = torch.from_numpy(ctx_h).cuda()
    timer = OpTimer(torch)
    st = DecodeStep([layer], table, ctx, acc, w.gamma, w.budget, w.temperature, run=timer.run)
    kv = st.kv[0]
    pb = s3r.page_bytes(kv)
    staging = torch.empty((maxp, pb), dtype=torch.uint8, device="cuda")
    host_pages = {}
    move_events = []
    slot_of = {}
    free_slots = list(range(slots - 1, -1, -1))
    fresh = []
    checked = [0]

    def blocks_tensor(blocks):
        return torch.tensor([b + 1 for b in blocks], dtype=torch.int32, device="cuda")

    def on_pause(r, blocks):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = len(blocks)
        dst = torch.empty((n, pb), dtype=torch.uint8, pin_memory=True)
        bt = blocks_tensor(blocks)
        e0.record()
        s3r.s3r_pack_pages(kv, bt, staging)
        dst.copy_(staging[:n], non_blocking=True)
        e1.record()
        # stream order keeps the copy ahead of any later write to these blocks
        host_pages[r.rid] = dst
        move_events.append(("offload", n, e0, e1))
        sl = slot_of.pop(r.rid, None)         # a request admitted this round has no slot yet
        if sl is not None:
            free_slots.append(sl)

    def on_restore(r):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        src = host_pages.pop(r.rid)
        n = src.shape[0]
        bt = blocks_tensor(r.blocks[:n])
        e0.record()
        staging[:n].copy_(src, non_blocking=True)
        s3r.s3r_unpack_pages(kv, bt, staging)
        e1.record()
        move_events.append(("restore", n, e0, e1))
        if verify_moves:
            check = s3r.s3r_pack_pages(kv, bt)
            if not torch.equal(check.cpu(), src):
                raise RuntimeError(f"request {r.rid}: restored pages differ from the offloaded ones")
            checked[0] += n

    ctl = AIMD() if controller == "aimd" else FixedCap(slots)
    sch = Scheduler(reqs, nb - 1, ctl, "offload", G1, on_pause=on_pause, on_restore=on_restore)
    generated = 0
    gpu_step_ms = 0.0
    step = 0
    while not sch.done:
        sch.admit()
        sch.ensure_room()
        for r in sch.running:
            if r.rid not in slot_of:
                slot_of[r.rid] = free_slots.pop()
                fresh.append(slot_of[r.rid])
        occupied = {slot_of[r.rid]: r for r in sch.running}
        table_h[:] = 0
        ctx_h[:] = 0
        for sl, r in occupied.items():
            table_h[sl, :len(r.blocks)] = np.asarray(r.blocks, dtype=np.int32) + 1
            ctx_h[sl] = r.length
        table.copy_(torch.from_numpy(table_h), non_blocking=False)
        ctx.copy_(torch.from_numpy(ctx_h), non_blocking=False)
        if fresh:
            st.nsel[0][torch.tensor(fresh, dtype=torch.int64, device="cuda")] = 0
            fresh.clear()
        timer.reset()
        st.run(step % max_steps)
        a = st.num_accepted.cpu().numpy()
        gpu_step_ms += sum(sum(timer.ms(o)) for o in timer.pairs)
        generated += sch.step({r.rid: int(a[sl]) + 1 for sl, r in occupied.items()})
        for r in reqs:
            if r.state == "done" and r.rid in slot_of:
                free_slots.append(slot_of.pop(r.rid))
        step += 1
        if step % 2000 == 0:
            print(json.dumps({"step": step, "running": len(sch.running), "paused": len(sch.paused),
                              "waiting": len(sch.waiting), "limit": sch.limit}), flush=True)
        if step >= max_steps:
            raise RuntimeError("batch did not finish")
    torch.cuda.synchronize()
    move_ms = sum(e0.elapsed_time(e1) for _, _, e0, e1 in move_events)
    moved = sch.pages_offloaded + sch.pages_restored
    out = {"controller": controller, "pool_tokens": pool_tokens, "slots": slots, "requests": len(reqs),
           "steps": step, "generated_tokens": generated,
           "pages_moved_per_1k_tokens": moved / generated * 1000,
           "gpu_step_s": gpu_step_ms / 1e3, "gpu_move_s": move_ms / 1e3,
           "tokens_per_gpu_s": generated / ((gpu_step_ms + move_ms) / 1e3),
           "mean_step_us": gpu_step_ms / step * 1e3, "pages_checked_after_restore": checked[0],
           "all_finished": all(r.state == "done" and r.generated == r.response for r in reqs)}
    print(json.dumps(out), flush=True)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--pool", type=int, default=700000, help="pool size in tokens")
    ap.add_argument("--controller", default="aimd", choices=["aimd", "fixed256"])
    ap.add_argument("--prompts", type=int, default=256)
    ap.add_argument("--seed", type=int, default=1)
    args = ap.parse_args(argv)
    return run(args.controller, args.pool, args.seed, num_prompts=args.prompts)


if __name__ == "__main__":
    main(sys.argv[1:])
