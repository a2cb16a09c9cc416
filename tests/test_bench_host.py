"""Host logic of bench.py that needs no GPU: the roofline's `traffic` comes from
the committed counter summary only while that summary was taken on the current
verify source and on the same workload."""
import os
import shutil

import pytest

import bench

VERIFY_SRC = os.path.join(bench.ROOT, "rl_rollout_amd", "csrc", "verify_attn.hip")
WORKLOAD = "qwen3_1.7b_like_gqa16x8_d128_ctx16k_b64"


def test_traffic_read_for_the_current_source_and_workload():
    text = open(os.path.join(bench.PROFILE_DIR, "verify_attn_qwen3_1.7b_ctx16k_counters.md")).read()
    if f"source_sha256_16: {bench.source_hash(VERIFY_SRC)}" not in text:
        pytest.skip("the verify source changed since the committed counters were taken")
    t = bench.read_counter_traffic(VERIFY_SRC, WORKLOAD)
    assert t is not None and 4.0e9 < t < 5.0e9


def test_traffic_is_null_once_the_kernel_source_changes(tmp_path):
    changed = tmp_path / "verify_attn.hip"
    shutil.copy(VERIFY_SRC, changed)
    with open(changed, "a") as f:
        f.write("\n// edited\n")
    assert bench.read_counter_traffic(str(changed), WORKLOAD) is None


def test_traffic_is_null_for_another_workload():
    assert bench.read_counter_traffic(VERIFY_SRC, "qwen3_8b_like_gqa32x8_d128_ctx24k_b128") is None


def test_oracle_pool_starts_every_worker_and_matches_the_oracle(tmp_path):
    """The CPU baseline's pool: the "ready" round holds one task in each worker at
    once (four distinct processes), and a chunked verify through the workers gives
    the oracle's page scores."""
    import numpy as np

    import oracle
    from rl_rollout_amd import synth
    from rl_rollout_amd import workloads as W

    w = W.TINY_FP32.with_(num_seqs=4)
    a = synth.make_attn_inputs(w, 5)
    arrays = {"k": a.k_cache, "v": a.v_cache, "qv": a.q_verify, "table": a.page_table, "lens": a.ctx_lens}
    for name, arr in arrays.items():
        np.save(tmp_path / f"{name}.npy", np.ascontiguousarray(arr))
    ctx = bench.oracle_pool_context()
    chunks = [np.array([0]), np.array([1]), np.array([2, 3])]
    barrier = ctx.Barrier(4)
    with ctx.Pool(4, initializer=bench._oracle_worker_init, initargs=(str(tmp_path), barrier)) as pool:
        ready = pool.map(bench._oracle_task, [("ready", None, 0, 1.0)] * 4, chunksize=1)
        assert len({pid for pid, _ in ready}) == 4
        out = pool.map(bench._oracle_task, [("verify", c, 0, 1.0) for c in chunks], chunksize=1)
    got = np.concatenate([r for _, r in out])
    want = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)[1]
    np.testing.assert_array_equal(got, want)


def test_bench_refuses_more_than_one_gpu():
    """`--gpus N` with N above 1 exits with a message before touching a GPU."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_op_timer_rejects_an_unknown_event_kind():
    import torch

    from rl_rollout_amd.measure import EVENT_FLAGS, OpTimer

    assert EVENT_FLAGS["nofence"] == 0x20000000 and EVENT_FLAGS["device"] == 0x40000000
    with pytest.raises(ValueError):
        OpTimer(torch, "fenceless")
