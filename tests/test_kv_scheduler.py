"""Host checks of the KV-aware admission scheduler: the AIMD rule, the page
pool's bookkeeping, the scheduler's invariants at every step under memory
pressure (every block owned once, paused requests keep their tokens, restore
before admit), completion of every request, and fewer pages moved with AIMD than
with a fixed cap on a batch that over-commits the pool."""
import numpy as np
import pytest

from rl_rollout_amd.kv_scheduler import AIMD, FixedCap, PagePool, Request, Scheduler, pages_for, rollout_batch, \
    simulate


def _tps(rng, n):
    a = np.zeros(n, int)
    alive = np.ones(n, bool)
    for _ in range(4):
        alive &= rng.random(n) < 0.85
        a += alive
    return a + 1


def test_aimd_rule():
    c = AIMD(limit=64, alpha=4, beta=0.5, u_low=0.8, u_high=0.95, backlog_max=0.05, limit_min=8, limit_max=100,
             hold=2)
    assert c.update(0.5, 0.0) == 68            # low utilisation: + alpha
    assert c.update(0.9, 0.0) == 68            # between the thresholds: unchanged
    assert c.update(0.97, 0.0) == 34           # high utilisation: x beta
    assert c.update(0.97, 0.0) == 34           # held: no second backoff yet
    assert c.update(0.97, 0.0) == 34
    assert c.update(0.5, 0.10) == 17           # backlog: x beta once the hold has passed
    for _ in range(100):
        c.update(0.1, 0.0)
    assert c.limit == 100                      # capped above
    for _ in range(100):
        c.update(0.99, 0.0)
    assert c.limit == 8                        # floored below
    assert FixedCap(256).update(0.99, 0.5) == 256


def test_page_pool_conserves_blocks():
    p = PagePool(10)
    a = p.alloc(4)
    b = p.alloc(6)
    assert p.alloc(1) is None and p.used == 10
    assert sorted(a + b) == list(range(10))
    p.release(a)
    assert p.used == 6 and p.alloc(5) is None
    c = p.alloc(4)
    assert sorted(c) == sorted(a)


@pytest.mark.parametrize("policy", ["offload", "recompute"])
@pytest.mark.parametrize("ctl", ["fixed", "aimd"])
def test_batch_completes_with_invariants_under_pressure(policy, ctl):
    reqs = rollout_batch(16, 4, 7, prompt_range=(64, 256), median_response=600, max_response=3000)
    controller = FixedCap(64) if ctl == "fixed" else AIMD(limit=16, limit_max=64, hold=8)
    s = Scheduler(reqs, 800, controller, policy)   # 12.8K tokens of pool for 64 requests
    rng = np.random.default_rng(1)
    paused_tokens = {}
    while not s.done:
        s.admit()
        s.ensure_room()
        s.check()
        for r in s.paused:
            if r.rid in paused_tokens:
                assert r.generated == paused_tokens[r.rid]   # paused: keeps its state, makes no progress
            paused_tokens[r.rid] = r.generated
        for r in s.running:
            paused_tokens.pop(r.rid, None)
            assert len(r.blocks) >= pages_for(r.length + s.block_len)
        run = list(s.running)
        s.step({r.rid: int(e) for r, e in zip(run, _tps(rng, len(run)))})
    assert all(r.state == "done" and r.generated == r.response and not r.blocks for r in reqs)
    assert s.pool.used == 0
    if policy == "offload":
        assert s.pages_offloaded == s.pages_restored > 0
    else:
        assert s.pages_offloaded == s.pages_restored == 0 and s.pages_recomputed > 0


def test_restore_before_admission():
    """While a request is paused no new request is admitted."""
    reqs = rollout_batch(8, 4, 3, prompt_range=(64, 128), median_response=800, max_response=2000)
    s = Scheduler(reqs, 300, FixedCap(32), "offload")
    rng = np.random.default_rng(2)
    seen_pause = False
    while not s.done:
        waiting_before = len(s.waiting)
        s.admit()
        if s.paused:
            # a request still paused after the round: nothing new was admitted in it
            assert len(s.waiting) == waiting_before
            seen_pause = True
        s.ensure_room()
        run = list(s.running)
        s.step({r.rid: int(e) for r, e in zip(run, _tps(rng, len(run)))})
    assert seen_pause


def test_aimd_moves_fewer_pages_than_a_fixed_cap():
    out = {}
    for name, ctl in (("fixed", FixedCap(128)), ("aimd", AIMD(limit=32, limit_max=128))):
        reqs = rollout_batch(32, 8, 5, prompt_range=(64, 512), median_response=1500, max_response=8000)
        s, tr = simulate(reqs, 9000, ctl, "offload", _tps, seed=4, check_every=50)
        gen = int(tr[:, 2].sum())
        assert gen == sum(r.response for r in reqs)
        out[name] = (s.pages_offloaded + s.pages_restored) / gen * 1000
    assert out["fixed"] > 5 * max(out["aimd"], 0.1), out
