"""Timing and byte accounting shared by bench.py and the budget sweep.

Algorithmic bytes are what the method has to move, not what a kernel happens to
move: the KV of every token an attention call attends, its queries and outputs,
and the index data it must read.
"""
from __future__ import annotations

import numpy as np

FLUSH_BYTES = 1 << 30
HBM_PEAK_GBS = 8000.0


def cache_flush(torch, mode: str = "read"):
    """A function that evicts L2 and the 256 MB Infinity Cache before a cold
    measurement by sweeping a 1 GiB buffer: reading it (default), or writing it
    ("write"), which also leaves dirty lines whose write-back lands in the next
    kernel (measured: ragged drafts then grow with the draft step)."""
    buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    if mode == "write":
        return lambda: buf.zero_()
    words = buf.view(torch.int64)
    return lambda: torch.amax(words)


class OpTimer:
    """Per-op HIP event pairs on the current stream; durations read after a sync."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return r

    def ms(self, name):
        return [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]

    def reset(self):
        self.pairs = {}


def verify_bytes(lens, G1, w, max_pages):
    """Dense verify of a block of G1 queries: KV of positions < L_b + G1, Q and O,
    page-table entries of the visible pages, and the page-score row."""
    kvb = w.kv_bytes_per_token()
    esz = 2 if w.kv_dtype == "bf16" else 4
    n = lens.shape[0]
    kv = int(np.sum(lens.astype(np.int64) + G1)) * kvb
    qo = n * G1 * w.num_q_heads * w.head_dim * esz * 2
    table = int(np.sum((lens.astype(np.int64) + G1 + 15) // 16)) * 4
    scores = n * max_pages * 4
    return kv + qo + table + scores


def dense_ar_bytes(lens, w):
    """Dense attention of one query per sequence over positions <= L_b (no scores)."""
    kvb = w.kv_bytes_per_token()
    esz = 2 if w.kv_dtype == "bf16" else 4
    n = lens.shape[0]
    kv = int(np.sum(lens.astype(np.int64) + 1)) * kvb
    qo = n * w.num_q_heads * w.head_dim * esz * 2
    table = int(np.sum((lens.astype(np.int64) + 16) // 16)) * 4
    return kv + qo + table


def draft_keys(lens, nsel, j):
    """Keys draft step j attends per sequence: the selected full pages plus the tail."""
    return nsel.astype(np.int64) * 16 + (lens.astype(np.int64) % 16) + j


def draft_bytes(lens, nsel, j, w):
    """Sparse draft step j: KV of the attended keys, Q and O, and for every selected
    page its index and its page-table entry."""
    kvb = w.kv_bytes_per_token()
    esz = 2 if w.kv_dtype == "bf16" else 4
    n = lens.shape[0]
    idx = 2 * int(np.sum(nsel)) * 4
    return int(np.sum(draft_keys(lens, nsel, j))) * kvb + n * w.num_q_heads * w.head_dim * esz * 2 + idx
