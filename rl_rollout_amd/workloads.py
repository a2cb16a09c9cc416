"""Synthetic decode workloads for the S3R hot path.

Each workload mirrors a shape the pages run on (wispaper.ai, "Throughput gains
with comparable task performance": Qwen3-1.7B and Qwen3-8B, 256 prompts x 8
responses, responses up to 16K and 24K tokens, draft length 6, budget 0.05;
rebasdaily.com, "为什么值得关注": budget sweep 0.05 .. 0.50 with acceptance 80.4% ..
96.7%). The values are synthetic: no model weights or datasets are involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str                    # "f32" or "bf16"
    ctx_range: Tuple[int, int]       # committed length L_b, uniform in [lo, hi] (lo == hi: fixed)
    gamma: int
    budget: float
    vocab: int
    logits_dtype: str
    draft_noise: float               # draft logits = target + N(0, draft_noise)
    target_std: float = 2.0          # target logits ~ N(0, target_std)
    temperature: float = 1.0
    page_size: int = 16
    num_layers: int = 1
    budgets: Tuple[float, ...] = ()          # budget sweep (ragged workload)
    sweep_noise: Tuple[float, ...] = ()      # draft noise per swept budget
    position_noise: Tuple[float, ...] = ()   # draft noise per draft position (overrides draft_noise)
    late_position_noise: Tuple[float, ...] = ()  # a later-training profile of the same model
    spare_steps: int = 64            # page-table headroom, in decode steps of gamma + 1 tokens

    @property
    def block_len(self) -> int:
        return self.gamma + 1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def max_pages(self) -> int:
        top = self.ctx_range[1] + (self.spare_steps + 1) * self.block_len
        return math.ceil(top / self.page_size)

    def kv_bytes_per_token(self) -> int:
        return self.num_kv_heads * self.head_dim * 2 * (4 if self.kv_dtype == "f32" else 2)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


TINY_FP32 = Workload(
    name="tiny_fp32_ctx256", num_seqs=2, num_q_heads=2, num_kv_heads=1, head_dim=64,
    kv_dtype="f32", ctx_range=(256, 256), gamma=4, budget=0.25, vocab=512,
    logits_dtype="f32", draft_noise=0.5, spare_steps=4)

QWEN3_1P7B_16K = Workload(
    name="qwen3_1.7b_like_gqa16x8_d128_ctx16k_b64", num_seqs=64, num_q_heads=16, num_kv_heads=8,
    head_dim=128, kv_dtype="bf16", ctx_range=(16384, 16384), gamma=4, budget=0.05,
    vocab=151936, logits_dtype="bf16", draft_noise=0.3)

RAGGED_SWEEP = Workload(
    name="ragged_budget_sweep_b256_ctx1k_16k", num_seqs=256, num_q_heads=16, num_kv_heads=8,
    head_dim=128, kv_dtype="bf16", ctx_range=(1024, 16384), gamma=4, budget=0.05,
    vocab=151936, logits_dtype="bf16", draft_noise=0.4985,
    budgets=(0.05, 0.10, 0.25, 0.50), sweep_noise=(0.4985, 0.3718, 0.2066, 0.0829))

QWEN3_8B_24K = Workload(
    name="qwen3_8b_like_gqa32x8_d128_ctx24k_b128", num_seqs=128, num_q_heads=32, num_kv_heads=8,
    head_dim=128, kv_dtype="bf16", ctx_range=(24576, 24576), gamma=6, budget=0.05,
    vocab=151936, logits_dtype="bf16", draft_noise=0.3)

FULL_STEP_28L = Workload(
    name="full_step_1.7b_like_28layers_b128_ctx2k_16k", num_seqs=128, num_q_heads=16,
    num_kv_heads=8, head_dim=128, kv_dtype="bf16", ctx_range=(2048, 16384), gamma=4,
    budget=0.10, vocab=151936, logits_dtype="bf16", draft_noise=0.3718, num_layers=28,
    spare_steps=8)

# Position-dependent acceptance (wispaper.ai, "Acceptance falls at later draft
# positions"): six draft positions whose noise gives acceptance linear between
# the printed first- and sixth-position values (Qwen3-8B at training step 20:
# 95.8% -> 67.9%, at step 100: 94.2% -> 61.3%; Qwen3-1.7B: 95.0% -> 62.9%). The
# noise values come from rl_rollout_amd/calibrate.py.
QWEN3_8B_24K_POSITIONS = QWEN3_8B_24K.with_(
    name="qwen3_8b_like_gqa32x8_d128_ctx24k_b128_position_profile", gamma=6,
    position_noise=(0.1046, 0.2451, 0.3865, 0.5301, 0.6761, 0.8256),
    late_position_noise=(0.1447, 0.3110, 0.4788, 0.6501, 0.8261, 1.0091))

QWEN3_1P7B_16K_POSITIONS = QWEN3_1P7B_16K.with_(
    name="qwen3_1.7b_like_gqa16x8_d128_ctx16k_b64_position_profile", gamma=6,
    position_noise=(0.1248, 0.2866, 0.4502, 0.6165, 0.7872, 0.9636))

# The ragged lengths of the budget sweep with the 1.7B-like position profile and
# six draft positions: per-sequence draft costs differ sixteenfold, acceptance
# falls with the position.
RAGGED_POSITIONS = RAGGED_SWEEP.with_(
    name="ragged_b256_ctx1k_16k_position_profile", gamma=6, budgets=(), sweep_noise=(),
    position_noise=QWEN3_1P7B_16K_POSITIONS.position_noise)

ALL = (TINY_FP32, QWEN3_1P7B_16K, RAGGED_SWEEP, QWEN3_8B_24K, FULL_STEP_28L, QWEN3_8B_24K_POSITIONS,
       QWEN3_1P7B_16K_POSITIONS, RAGGED_POSITIONS)
BY_NAME = {w.name: w for w in ALL}
