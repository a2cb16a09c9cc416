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
