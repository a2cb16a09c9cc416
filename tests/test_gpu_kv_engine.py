"""The admission scheduler driving the real decode step: a small batch that
over-commits its page pool, so requests are paused (pages packed and copied to
pinned host memory) and restored (copied back and unpacked into new blocks).
Every restored page must equal the offloaded one byte for byte, and every request
must finish with exactly its response length."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("controller", ["fixed256", "aimd"])
def test_engine_moves_pages_exactly_and_finishes(controller):
    from rl_rollout_amd.kv_engine import run
    print(f"engine: {controller}, 32 requests over a 24K-token pool", flush=True)
    out = run(controller, pool_tokens=24_000, seed=3, slots=32, num_prompts=8, group=4, max_steps=20000,
              verify_moves=True, median_response=900)
    assert out["all_finished"]
    if controller == "fixed256":
        assert out["pages_moved_per_1k_tokens"] > 0 and out["pages_checked_after_restore"] > 0
