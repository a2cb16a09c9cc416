#!/usr/bin/env python3
"""Benchmark of the S3R decode hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, one
attention layer: gamma sparse draft attention calls (each reading the draft rows
in flight from the draft-row buffers), the append of the verify block, dense
verify attention with page scores, exact speculative accept with commit, and
budget selection for the next step. Inputs are resident
in HBM before timing starts. Before every attention call a 1 GiB read sweep
evicts L2 and the 256 MB Infinity Cache (as the other layers of a model would),
so the attention kernels are measured cold.

Printed value: verify + draft attention bandwidth = algorithmic bytes of the
verify and the gamma draft calls / their summed kernel time (HIP events on the
launch stream, created with hipEventDisableSystemFence: timing-only events that
add no cache write-back and invalidate around the op). Also reported: emitted and accepted tokens/s over the whole
path's GPU time, per-op times, a dense autoregressive reference (verify with one
query), the roofline of the dominant kernel and the fp64 oracle timed on host
cores over a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from rl_rollout_amd.measure import (FLUSH_BYTES, HBM_PEAK_GBS, OpTimer, cache_flush, draft_bytes,  # noqa: E402
                                    verify_bytes)

METRIC = "verify+draft attn HBM GB/s (% peak) and accepted tokens/s at 16K ctx, 1 GPU"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_1.7b_like_gqa16x8_d128_ctx16k_b64")
    ap.add_argument("--budget", type=float, default=None,
                    help="override the sparse budget (a budget of the workload's sweep also takes its draft noise)")
    ap.add_argument("--draft-noise", type=float, default=None)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--warm-cache", action="store_true", help="skip the cache flush before attention calls")
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="how the 1 GiB cache flush before each attention call evicts the caches: by reading the "
                         "buffer (default), or by writing it, which also leaves dirty lines whose write-back lands in "
                         "the next kernel")
    ap.add_argument("--fused-append", action="store_true",
                    help="write K/V rows inside the attention launches (the *_append entry points) instead of "
                         "separate s3r_append_kv launches")
    ap.add_argument("--draft-appends", action="store_true",
                    help="append each draft token's K/V row before its draft (s3r_append_kv) instead of the "
                         "default, where the drafts read the in-flight rows from the draft-row buffers "
                         "(s3r_sparse_draft_attn_rows)")
    ap.add_argument("--events", choices=("system", "nofence", "device"), default="nofence",
                    help="timing events around each op: hipEventDisableSystemFence (default: timing-only "
                         "events, no cache write-back and invalidate at each record), torch's (a system-scope "
                         "fence at each record), or a device-scope release")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=64)
    ap.add_argument("--cpu-workers", type=int, default=min(16, len(os.sched_getaffinity(0))),
                    help="worker processes of the oracle baseline (default: the CPUs this process may run on, at "
                         "most 16, the host share one GPU is given)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


KERNEL_HEADERS = ("common.hpp", "kernels.hpp")


def source_hash(path):
    """First 16 hex digits of the sha256 of a kernel source followed by the
    headers beside it that it includes (those present)."""
    h = hashlib.sha256(open(path, "rb").read())
    for name in KERNEL_HEADERS:
        hp = os.path.join(os.path.dirname(path), name)
        if os.path.exists(hp):
            h.update(open(hp, "rb").read())
    return h.hexdigest()[:16]


def read_counter_traffic(kernel_src, workload):
    """HBM bytes per verify launch from the committed counter summary, if it was
    taken on the current kernel source and on this workload; else None."""
    path = os.path.join(PROFILE_DIR, "verify_attn_qwen3_1.7b_ctx16k_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_wl = re.search(r"workload:\s*(\S+)", text)
    if not m_hash or not m_bytes or not m_wl or m_hash.group(1) != source_hash(kernel_src):
        return None
    if m_wl.group(1) != workload:
        return None
    return float(m_bytes.group(1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_pool_context():
    """A forkserver started before this process touches the GPU: the oracle's
    worker processes fork from it, so none of them holds GPU state."""
    import multiprocessing as mp
    from multiprocessing import forkserver

    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy"])
    forkserver.ensure_running()
    return ctx


# Worker side of the oracle baseline: each worker maps the sample's arrays from
# the files the parent wrote and runs the oracle on one chunk of sequences.
_ORACLE_DATA = {}
_ORACLE_LIMITS = []
_ORACLE_BARRIER = []


def _oracle_worker_init(path, barrier):
    from threadpoolctl import threadpool_limits

    _ORACLE_BARRIER.append(barrier)
    _ORACLE_LIMITS.append(threadpool_limits(limits=1))  # one BLAS thread per worker process
    for name in os.listdir(path):
        if name.endswith(".npy"):
            _ORACLE_DATA[name[:-4]] = np.load(os.path.join(path, name), mmap_mode="r")


def _oracle_task(task):
    """(the worker's pid, the op's result); "ready" waits until every worker of the
    pool holds one such task, so that each worker is up before the timing starts."""
    import oracle

    op, idx, j, temperature = task
    D = _ORACLE_DATA
    res = None
    if op == "verify":
        res = oracle.dense_verify_attn(D["qv"][idx], D["k"], D["v"], D["table"][idx], D["lens"][idx])[1]
    elif op == "draft":
        sel = [D["sel"][b, :D["ns"][b]] for b in idx]
        oracle.sparse_draft_attn(D["qd"][j - 1][idx], D["k"], D["v"], D["table"][idx], D["lens"][idx], sel, j)
    elif op == "accept":
        res = oracle.spec_accept(D["tl"][idx], D["dl"][idx], D["dt"][idx], D["ua"][idx], D["us"][idx],
                                 temperature)[0]
    else:
        _ORACLE_BARRIER[0].wait(timeout=120)
    return os.getpid(), res


def cpu_baseline(mp_ctx, dev_inputs, acc_inputs, w, max_pages, nsel_dev, sel_dev, n_seqs, workers):
    """Time the fp64 oracle on the first n_seqs sequences of the workload: one
    verify, gamma draft steps, one accept and one selection. The oracle runs as it
    is, in `workers` processes (one BLAS thread each), each over a contiguous chunk
    of the sequences; the arrays reach the workers as memory-mapped files."""
    import shutil
    import tempfile

    import torch

    import oracle

    B = w.num_seqs
    n = min(n_seqs, B)
    G1 = w.block_len
    lens = dev_inputs["ctx_lens"].cpu().numpy()[:n].astype(np.int64)
    table = dev_inputs["page_table"].cpu().numpy()[:n]
    used = np.unique(table[table >= 0])
    remap = np.full(int(table.max()) + 2, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    small_table = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
    idx = torch.from_numpy(used.astype(np.int64)).cuda()

    def to_np(t):
        t = t.contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    sel = sel_dev.cpu().numpy()[:n]
    ns = nsel_dev.cpu().numpy()[:n]
    arrays = {
        "k": to_np(dev_inputs["k_cache"].index_select(0, idx)),
        "v": to_np(dev_inputs["v_cache"].index_select(0, idx)),
        "qv": to_np(dev_inputs["q_verify"][:n]),
        "qd": to_np(dev_inputs["q_draft"][:, :n]),
        "table": small_table, "lens": lens, "sel": sel, "ns": ns,
        "tl": to_np(acc_inputs["target_logits"][:n]),
        "dl": to_np(acc_inputs["draft_logits"][:n]),
        "dt": acc_inputs["draft_tokens"][:n].cpu().numpy(),
        "ua": acc_inputs["u_accept"][0, :n].cpu().numpy(),
        "us": acc_inputs["u_sample"][0, :n].cpu().numpy(),
    }
    chunks = [c for c in np.array_split(np.arange(n), max(1, min(workers, n))) if len(c)]
    tmp = tempfile.mkdtemp(prefix="s3r_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for name, arr in arrays.items():
            np.save(os.path.join(tmp, name + ".npy"), np.ascontiguousarray(arr))
        del arrays
        T = w.temperature
        barrier = mp_ctx.Barrier(len(chunks))
        with mp_ctx.Pool(len(chunks), initializer=_oracle_worker_init, initargs=(tmp, barrier)) as pool:
            pool.map(_oracle_task, [("ready", None, 0, T)] * len(chunks), chunksize=1)
            pids = set()

            def each(op, j=0):
                out = pool.map(_oracle_task, [(op, c, j, T) for c in chunks], chunksize=1)
                pids.update(pid for pid, _ in out)
                return [r for _, r in out]

            t0 = time.perf_counter()
            scores = np.concatenate(each("verify"))
            t1 = time.perf_counter()
            for j in range(1, w.gamma + 1):
                each("draft", j)
            t2 = time.perf_counter()
            a = np.concatenate(each("accept"))
            t3 = time.perf_counter()
        oracle.select_budget(scores, oracle.commit(lens, a), 16, w.budget)
        t4 = time.perf_counter()
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    attn_bytes = verify_bytes(lens, G1, w, max_pages) + sum(draft_bytes(lens, ns, j, w) for j in range(1, w.gamma + 1))
    attn_s = (t1 - t0) + (t2 - t1)
    return {
        "value": attn_bytes / attn_s / 1e9,
        "unit": "GB/s",
        "cores": len(chunks),
        "kind": "oracle",
        "sample": f"first {n} of {B} sequences, one step: verify + {w.gamma} drafts (timed for value), "
                  f"accept (timed, reported) in {len(chunks)} worker processes over sequence chunks, one BLAS "
                  f"thread each; select (timed, reported) in the parent; float64 NumPy",
        "worker_processes": len(chunks),
        "distinct_worker_pids": len(pids),
        "host_cpus": os.cpu_count(),
        "cpus_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "verify_s": t1 - t0, "draft_s": t2 - t1, "accept_s": t3 - t2, "select_s": t4 - t3,
        "emitted_tokens_per_s": float(np.sum(a + 1)) / (t4 - t0),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    mp_ctx = None
    if not (args.no_cpu_baseline or args.calibrate_copy):
        try:
            mp_ctx = oracle_pool_context()
        except Exception as e:  # the baseline then reports the failure; the GPU measurement goes on
            print(f"[bench] no oracle worker pool: {e!r}", file=sys.stderr, flush=True)
    import torch

    from rl_rollout_amd import s3r
    from rl_rollout_amd import workloads as W
    from rl_rollout_amd.step import DecodeStep, build_inputs

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": FLUSH_BYTES, "copy_bytes_written": FLUSH_BYTES, "launches": 5}))
        return

    w = W.BY_NAME[args.workload]
    if args.budget is not None:
        w = w.with_(budget=args.budget)
        if args.draft_noise is None and args.budget in w.budgets:
            # a swept budget runs at its own draft noise (the acceptance the pages
            # pair with that budget)
            w = w.with_(draft_noise=w.sweep_noise[list(w.budgets).index(args.budget)])
    if args.draft_noise is not None:
        w = w.with_(draft_noise=args.draft_noise)
    K, Wm = args.steps, args.warmup
    total_steps = K + Wm + 1
    G1, gamma, NL = w.block_len, w.gamma, w.num_layers
    B = w.num_seqs

    t_setup = time.perf_counter()
    log(f"workload {w.name}: B={B} layers={NL} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"ctx={w.ctx_range} gamma={gamma} budget={w.budget} V={w.vocab}")
    layers, table, ctx, x, max_pages, nb = build_inputs(w, args.seed, total_steps)
    torch.cuda.synchronize()
    kv_bytes = sum(l["k_cache"].numel() * l["k_cache"].element_size() * 2 for l in layers)
    log(f"inputs resident: KV {kv_bytes / 1e9:.2f} GB over {NL} layer(s), {nb} blocks per layer, "
        f"max_pages={max_pages}, setup {time.perf_counter() - t_setup:.1f}s")

    sweep = cache_flush(torch, args.flush)

    def flush():
        if not args.warm_cache:
            sweep()

    timer = OpTimer(torch, args.events)
    st = DecodeStep(layers, table, ctx, x, gamma, w.budget, w.temperature, before_attn=flush, run=timer.run,
                    fused_append=args.fused_append,
                    draft_rows=not (args.fused_append or args.draft_appends))
    st.seed_scores()
    torch.cuda.synchronize()
    hist_lens = torch.empty((total_steps + 1, B), dtype=torch.int32, device="cuda")
    hist_nsel = torch.empty((total_steps, NL, B), dtype=torch.int32, device="cuda")
    hist_acc = torch.empty((total_steps, B), dtype=torch.int32, device="cuda")

    def step(s):
        hist_lens[s].copy_(ctx)
        for l in range(NL):
            hist_nsel[s, l].copy_(st.nsel[l])
        st.run(s)
        hist_acc[s].copy_(st.num_accepted)

    for s in range(Wm):
        step(s)
    torch.cuda.synchronize()
    timer.reset()
    log(f"warmup done ({Wm} steps); timing {K} steps")
    t0 = time.perf_counter()
    for s in range(Wm, Wm + K):
        step(s)
    hist_lens[Wm + K].copy_(ctx)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    H = hist_lens.cpu().numpy()
    NS = hist_nsel.cpu().numpy()
    ver_ms = timer.ms("verify")
    dr_ms = {j: timer.ms(f"draft{j}") for j in range(1, gamma + 1)}
    vb, db = [], {j: [] for j in range(1, gamma + 1)}
    for s in range(Wm, Wm + K):
        for l in range(NL):
            vb.append(verify_bytes(H[s], G1, w, max_pages))
            for j in range(1, gamma + 1):
                db[j].append(draft_bytes(H[s], NS[s, l], j, w))
    v_bytes, v_time = float(np.sum(vb)), float(np.sum(ver_ms)) / 1e3
    d_bytes = float(sum(np.sum(db[j]) for j in db))
    d_time = float(sum(np.sum(dr_ms[j]) for j in dr_ms)) / 1e3
    attn_gbs = (v_bytes + d_bytes) / (v_time + d_time) / 1e9
    ops = ["append", "verify", "accept", "select"] + [f"draft{j}" for j in range(1, gamma + 1)]
    op_ms = {o: float(np.mean(timer.ms(o))) for o in ops if timer.ms(o)}
    path_s = sum(float(np.sum(timer.ms(o))) for o in ops) / 1e3
    emitted = int(np.sum(H[Wm + K] - H[Wm]))
    accepted = emitted - B * K
    A = hist_acc.cpu().numpy()[Wm:Wm + K].reshape(-1)
    assert int(A.sum()) == accepted
    # per draft position j: sequences that kept draft j among those whose test reached it
    alpha = [float((A >= j).sum()) / max(1, int((A >= j - 1).sum())) for j in range(1, gamma + 1)]

    # dense autoregressive reference on the same kernels: one query per sequence, layer 0
    q1 = layers[0]["q_verify"][:, :1].contiguous()
    out1 = torch.empty_like(q1)
    for _ in range(5):
        flush()
        timer.run("ar", lambda: s3r.s3r_dense_verify_attn(st.kv[0], q1, out=out1, want_scores=False,
                                                          workspace=st.verify_ws))
    torch.cuda.synchronize()
    ar_t = float(np.median(timer.ms("ar"))) / 1e3

    v_launch_bytes = v_bytes / (K * NL)
    v_launch_s = v_time / (K * NL)
    roof = {
        "kernel": "dense verify op (verify_main, then verify_unit_scores in whole-unit mode or verify_combine in "
                  "split mode; event-timed together)",
        "bound": "hbm",
        "achieved": v_launch_bytes / v_launch_s / 1e9,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": v_launch_bytes / v_launch_s / 1e9 / HBM_PEAK_GBS,
        "traffic": read_counter_traffic(os.path.join(ROOT, "rl_rollout_amd", "csrc", "verify_attn.hip"), w.name),
        "algorithmic_bytes_per_launch": v_launch_bytes,
        "avg_launch_us": v_launch_s * 1e6,
    }
    result = {
        "metric": METRIC,
        "value": round(attn_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(path_s / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "f32",
        "data": "synthetic (seeded on device; no weights or datasets)",
        "config": {"workload": w.name, "num_seqs": B, "layers": NL, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "ctx": list(w.ctx_range), "gamma": gamma, "budget": w.budget,
                   "vocab": w.vocab, "page_size": w.page_size, "draft_noise": w.draft_noise,
                   "cache": "warm" if args.warm_cache else f"cold (1 GiB {args.flush} sweep before each attention call)",
                   "kv_append": ("inside the attention launches" if args.fused_append else
                                 "separate launches" if args.draft_appends else
                                 "block rows appended before verify; drafts read their rows from the draft-row "
                                 "buffers"),
                   "timing_events": {"system": "torch events (system-scope fence at each record)",
                                     "nofence": "hipEventDisableSystemFence events",
                                     "device": "device-scope release events"}[args.events]},
        "attn_frac_of_peak": round(attn_gbs / HBM_PEAK_GBS, 4),
        "verify_gbps": round(v_bytes / v_time / 1e9, 1),
        "verify_frac": round(v_bytes / v_time / 1e9 / HBM_PEAK_GBS, 4),
        "draft_gbps": round(d_bytes / d_time / 1e9, 1),
        "draft_frac": round(d_bytes / d_time / 1e9 / HBM_PEAK_GBS, 4),
        "op_us": {o: round(v * 1e3, 2) for o, v in op_ms.items()},
        "emitted_tokens_per_s": round(emitted / path_s, 1),
        "accepted_tokens_per_s": round(accepted / path_s, 1),
        "accepted_drafts_per_step": round(accepted / (B * K), 4),
        "accepted_fraction_of_drafts": round(accepted / (B * K * gamma), 4),
        "per_position_acceptance": [round(x, 4) for x in alpha],
        "dense_ar_tokens_per_s": round(B / (ar_t * NL), 1),
        "dense_ar_verify_us": round(ar_t * 1e6, 2),
        "wall_ms_per_step": round(wall / K * 1e3, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample (cpu_baseline)")
        d0 = dict(layers[0], page_table=table, ctx_lens=ctx)
        try:
            result["cpu_baseline"] = cpu_baseline(mp_ctx, d0, x, w, max_pages, st.nsel[0], st.sel[0],
                                                  args.cpu_sample_seqs, args.cpu_workers)
        except Exception as e:  # the GPU line still goes out; the failure is named in it
            import traceback
            traceback.print_exc()
            result["cpu_baseline"] = {"value": None, "unit": "GB/s", "cores": 0, "kind": "oracle",
                                      "sample": "failed", "error": repr(e)}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
