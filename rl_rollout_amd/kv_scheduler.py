"""KV-aware admission of rollout requests: an AIMD concurrency limit over a paged
KV pool, with the pages of paused requests offloaded to host memory and restored.

What the pages describe (wispaper.ai, "Dense verification still pays the full
KV-cache bill"; rebasdaily.com, "真正难搬的，还是那叠完整笔记"):
  * dense verification reads the complete history of every running request, so
    when the GPU's KV pages run out, requests are paused and their pages either
    moved to host memory and back (offload) or dropped and rebuilt (recompute);
    repeated moves thrash;
  * the scheduler measures resident pressure as GPU KV utilisation and pending
    demand as a restoration backlog of the paused requests; with low utilisation
    the concurrency limit grows by a constant, with high utilisation or too large
    a backlog it is multiplied down;
  * paused requests keep their token and proposal state and finish under the same
    policy snapshot, so response groups keep their identity;
  * paused requests are restored before new ones are admitted.
Their baseline is a fixed concurrency cap of 256 with offload, and they report
pages moved per 1,000 generated tokens (18.0 with the fixed cap, 1.3 with AIMD).

Readings (the pages give the rule's shape but no constants):
  * utilisation = allocated blocks / pool blocks, sampled after each step's
    admissions; backlog = pages held by paused requests / pool blocks;
  * the limit moves once per step: x beta when utilisation > u_high or backlog >
    backlog_max, + alpha when utilisation < u_low, otherwise unchanged; it stays in
    [limit_min, limit_max]; after a backoff the next one waits `hold` steps, so that
    one congestion event backs off once (the backlog takes a while to drain);
  * under pressure the most recently admitted running request is paused first;
  * a request is admitted or restored only if the pool keeps room for every
    running request's next block (its pages up to L + block_len);
  * the limit governs admission of new requests (the scheduler "adapts request
    admission"); a paused request was admitted already and is restored as soon as
    memory allows, and new requests wait while any request is paused.
Everything here is host bookkeeping: the page moves themselves are
s3r_pack_pages / s3r_unpack_pages plus a host copy, priced by the study in
rl_rollout_amd/kv_sched_study.py.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

PAGE = 16


def pages_for(tokens: int) -> int:
    return (int(tokens) + PAGE - 1) // PAGE


@dataclass
class Request:
    rid: int
    prompt: int
    response: int
    generated: int = 0
    blocks: List[int] = field(default_factory=list)   # GPU blocks held
    host_pages: int = 0                               # pages offloaded to host memory
    state: str = "waiting"                            # waiting, running, paused, done
    admitted_at: int = -1

    @property
    def length(self) -> int:
        """Committed KV length: the prompt plus the tokens generated so far."""
        return self.prompt + self.generated

    @property
    def finished(self) -> bool:
        return self.generated >= self.response


class PagePool:
    """GPU KV blocks: a free stack; allocation and release keep every block owned once."""

    def __init__(self, num_blocks: int):
        self.num_blocks = int(num_blocks)
        self.free = list(range(self.num_blocks - 1, -1, -1))

    @property
    def used(self) -> int:
        return self.num_blocks - len(self.free)

    def alloc(self, n: int) -> Optional[List[int]]:
        if n > len(self.free):
            return None
        out = self.free[len(self.free) - n:]
        del self.free[len(self.free) - n:]
        return out[::-1]

    def release(self, blocks: List[int]) -> None:
        self.free.extend(reversed(blocks))


@dataclass
class AIMD:
    """Concurrency limit: + alpha under low utilisation, x beta under high
    utilisation or a large restoration backlog."""
    limit: float = 64
    alpha: float = 4
    beta: float = 0.5
    u_low: float = 0.85
    u_high: float = 0.95
    backlog_max: float = 0.05
    limit_min: int = 8
    limit_max: int = 256
    hold: int = 64        # steps after a backoff before another one
    _since: int = 1 << 30

    def update(self, utilisation: float, backlog: float) -> int:
        self._since += 1
        if utilisation > self.u_high or backlog > self.backlog_max:
            if self._since > self.hold:
                self.limit = max(self.limit_min, np.floor(self.limit * self.beta))
                self._since = 0
        elif utilisation < self.u_low:
            self.limit = min(self.limit_max, self.limit + self.alpha)
        return int(self.limit)


@dataclass
class FixedCap:
    """The baseline: a constant concurrency cap."""
    limit: int = 256

    def update(self, utilisation: float, backlog: float) -> int:
        return self.limit


class Scheduler:
    """One rollout batch of requests over a page pool. policy: "offload" (paused
    pages go to host memory and come back) or "recompute" (paused pages are
    dropped and rebuilt on restore). controller: AIMD or FixedCap."""

    def __init__(self, requests: List[Request], num_blocks: int, controller, policy: str = "offload",
                 block_len: int = 5, on_pause=None, on_restore=None):
        """on_pause(request, blocks) runs before a paused request's blocks are
        released; on_restore(request) after a restored one got its new blocks
        (an engine moves the pages there)."""
        if policy not in ("offload", "recompute"):
            raise ValueError(policy)
        self.reqs = requests
        self.pool = PagePool(num_blocks)
        self.ctl = controller
        self.policy = policy
        self.block_len = block_len
        self.waiting = [r for r in requests if r.state == "waiting"]
        self.waiting.reverse()                            # pop() takes the lowest id first
        self.paused: List[Request] = []                   # restore order: first paused, first restored
        self.running: List[Request] = []
        self.steps = 0
        self.pages_offloaded = 0
        self.pages_restored = 0
        self.pages_recomputed = 0
        self.prefill_tokens = 0
        self.limit = int(controller.limit)
        self.limit_trace: List[int] = []
        self.on_pause = on_pause
        self.on_restore = on_restore

    # -- bookkeeping ---------------------------------------------------------
    def _need(self, r: Request) -> int:
        """Blocks r needs for its next step: its history plus the verify block."""
        return pages_for(r.length + self.block_len)

    def _reserve(self) -> int:
        """Blocks the running requests still need for their next step."""
        return sum(max(0, self._need(r) - len(r.blocks)) for r in self.running)

    def _pause(self, r: Request) -> None:
        if self.on_pause is not None:
            self.on_pause(r, r.blocks)
        self.running.remove(r)
        held = len(r.blocks)
        if self.policy == "offload":
            self.pages_offloaded += held
            r.host_pages = held
        else:
            r.host_pages = 0
        self.pool.release(r.blocks)
        r.blocks = []
        r.state = "paused"
        self.paused.append(r)

    def _grow(self, r: Request) -> bool:
        extra = self._need(r) - len(r.blocks)
        if extra <= 0:
            return True
        got = self.pool.alloc(extra)
        if got is None:
            return False
        r.blocks.extend(got)
        return True

    def backlog(self) -> float:
        return sum(pages_for(r.length) for r in self.paused) / self.pool.num_blocks

    def utilisation(self) -> float:
        return self.pool.used / self.pool.num_blocks

    # -- one scheduling round ------------------------------------------------
    def admit(self) -> None:
        """Restore paused requests first, whenever the pool keeps room for every
        running request's next block; then admit new ones while nothing is paused,
        the running count is below the limit and the pool keeps that room. The
        limit governs admission: a paused request was admitted already."""
        while self.paused:
            r = self.paused[0]
            if self._need(r) + self._reserve() > len(self.pool.free):
                break
            self.paused.pop(0)
            r.blocks = self.pool.alloc(self._need(r))
            if self.policy == "offload":
                self.pages_restored += r.host_pages
            else:
                self.pages_recomputed += pages_for(r.length)
                self.prefill_tokens += r.length
            if self.on_restore is not None:
                self.on_restore(r)
            r.host_pages = 0
            r.state = "running"
            r.admitted_at = self.steps
            self.running.append(r)
        while self.waiting and not self.paused and len(self.running) < self.limit:
            r = self.waiting[-1]
            if self._need(r) + self._reserve() > len(self.pool.free):
                break
            self.waiting.pop()
            r.blocks = self.pool.alloc(self._need(r))
            self.prefill_tokens += r.prompt
            r.state = "running"
            r.admitted_at = self.steps
            self.running.append(r)

    def ensure_room(self) -> None:
        """Every running request gets the blocks of its next step, oldest first;
        under pressure the most recently admitted running request is paused (which
        may be the one that needs the blocks)."""
        for r in sorted(self.running, key=lambda x: (x.admitted_at, x.rid)):
            if r.state != "running":
                continue
            while not self._grow(r):
                if len(self.running) == 1:
                    raise RuntimeError("one request does not fit in the pool")
                victim = max(self.running, key=lambda x: (x.admitted_at, x.rid))
                self._pause(victim)
                if victim is r:
                    break

    def step(self, emitted: Dict[int, int]) -> int:
        """Advance the running requests by emitted[rid] tokens each (at least 1),
        retire the finished ones. Returns the tokens generated."""
        total = 0
        for r in list(self.running):
            e = min(int(emitted.get(r.rid, 1)), r.response - r.generated)
            r.generated += e
            total += e
            if r.finished:
                r.state = "done"
                self.running.remove(r)
                self.pool.release(r.blocks)
                r.blocks = []
        self.steps += 1
        self.limit = self.ctl.update(self.utilisation(), self.backlog())
        self.limit_trace.append(self.limit)
        return total

    @property
    def done(self) -> bool:
        return not (self.running or self.paused or self.waiting)

    def check(self) -> None:
        """Invariants: every block owned once, free + owned = pool, states consistent."""
        owned = [b for r in self.reqs for b in r.blocks]
        assert len(owned) == len(set(owned)), "a block owned twice"
        assert len(owned) + len(self.pool.free) == self.pool.num_blocks, "blocks lost"
        assert not set(owned) & set(self.pool.free), "a free block is owned"
        for r in self.reqs:
            assert (r.state == "running") == (r in self.running)
            assert (r.state == "paused") == (r in self.paused)
            assert r.state == "running" or not r.blocks


def rollout_batch(num_prompts: int, group: int, seed: int, prompt_range=(128, 1024), median_response=3000,
                  sigma=0.9, max_response=16384) -> List[Request]:
    """A batch of num_prompts x group requests: prompt lengths uniform in
    prompt_range (shared by a group), response lengths log-normal around
    median_response, clipped to [64, max_response] (long-tailed, as long-context
    reasoning responses are)."""
    rng = np.random.default_rng(seed)
    reqs = []
    for p in range(num_prompts):
        pl = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
        for g in range(group):
            rl = int(np.clip(rng.lognormal(np.log(median_response), sigma), 64, max_response))
            reqs.append(Request(rid=len(reqs), prompt=pl, response=rl))
    return reqs


def simulate(requests: List[Request], num_blocks: int, controller, policy: str, tokens_per_step, seed: int,
             block_len: int = 5, max_steps: int = 1_000_000, check_every: int = 0):
    """Run a batch to completion. tokens_per_step(rng, n) -> emitted tokens of n
    running requests in one step. Returns the scheduler and per-step records
    (running count, total committed KV length of the running requests)."""
    rng = np.random.default_rng(seed)
    s = Scheduler(requests, num_blocks, controller, policy, block_len)
    trace = []
    while not s.done:
        s.admit()
        s.ensure_room()
        if check_every and s.steps % check_every == 0:
            s.check()
        run = list(s.running)
        if not run:
            raise RuntimeError("nothing runs: the pool cannot hold a single request")
        em = tokens_per_step(rng, len(run))
        kv = sum(r.length for r in run)
        gen = s.step({r.rid: int(e) for r, e in zip(run, em)})
        trace.append((len(run), kv, gen))
        if s.steps >= max_steps:
            raise RuntimeError("batch did not finish")
    return s, np.array(trace, dtype=np.int64)
