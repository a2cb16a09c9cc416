"""Timing and byte accounting shared by bench.py and the budget sweep.

Algorithmic bytes are what the method has to move, not what a kernel happens to
move: the KV of every token an attention call attends, its queries and outputs,
and the index data it must read.
"""
from __future__ import annotations

import ctypes

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


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000
EVENT_FLAGS = {"system": None, "nofence": HIP_EVENT_DISABLE_SYSTEM_FENCE, "device": HIP_EVENT_RELEASE_TO_DEVICE}


class HipEvents:
    """hipEventCreateWithFlags / hipEventRecord / hipEventElapsedTime of the HIP
    runtime this process has already loaded (torch's), so the events live in the
    same runtime instance as torch's streams and the library's launches."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split(None, 5)[-1].strip()
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded in this process")
        rt = ctypes.CDLL(path)
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for fn in (rt.hipEventCreateWithFlags, rt.hipEventRecord, rt.hipEventElapsedTime, rt.hipEventDestroy):
            fn.restype = ctypes.c_int
        self.rt = rt

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def create(self, flags):
        ev = ctypes.c_void_p()
        self._check(self.rt.hipEventCreateWithFlags(ctypes.byref(ev), flags), "hipEventCreateWithFlags")
        return ev

    def record(self, ev, stream):
        self._check(self.rt.hipEventRecord(ev, ctypes.c_void_p(stream)), "hipEventRecord")

    def elapsed_ms(self, s, e):
        out = ctypes.c_float()
        self._check(self.rt.hipEventElapsedTime(ctypes.byref(out), s, e), "hipEventElapsedTime")
        return float(out.value)

    def destroy(self, ev):
        self._check(self.rt.hipEventDestroy(ev), "hipEventDestroy")


class OpTimer:
    """Per-op HIP event pairs on the current stream; durations read after a sync.

    events: "system", torch's events (a system-scope fence when each is recorded:
    an L2 write-back and invalidate between the op and its neighbours); "nofence",
    events created with hipEventDisableSystemFence, which the HIP headers name for
    timing-only events (no fence, so the pair brackets the launches alone);
    "device", a device-scope release instead of the system-scope one."""

    def __init__(self, torch, events: str = "system"):
        if events not in EVENT_FLAGS:
            raise ValueError(f"events must be one of {sorted(EVENT_FLAGS)}")
        self.torch = torch
        self.flags = EVENT_FLAGS[events]
        self.hip = HipEvents() if self.flags is not None else None
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        if self.hip is None:
            s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            s.record()
            r = fn()
            e.record()
        else:
            stream = t.cuda.current_stream().cuda_stream
            s, e = self.hip.create(self.flags), self.hip.create(self.flags)
            self.hip.record(s, stream)
            r = fn()
            self.hip.record(e, stream)
        self.pairs.setdefault(name, []).append((s, e))
        return r

    def ms(self, name):
        if self.hip is None:
            return [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]
        return [self.hip.elapsed_ms(s, e) for s, e in self.pairs.get(name, [])]

    def reset(self):
        if self.hip is not None:
            for pairs in self.pairs.values():
                for s, e in pairs:
                    self.hip.destroy(s)
                    self.hip.destroy(e)
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
