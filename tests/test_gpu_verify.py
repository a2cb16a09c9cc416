"""GPU parity of s3r_dense_verify_attn against the fp64 oracle: outputs to the
per-row relative tolerance (1e-4 fp32 KV, 2e-2 bf16 KV) and page scores, over
ragged lengths that span several pages, splits and partial tails."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import TOL, check_page_scores, dev, host, max_row_rel_err, page_score_rtol, upload_cache

pytestmark = pytest.mark.gpu


class _env:
    """Set environment knobs of the library for the duration of a call."""

    def __init__(self, **kv):
        self.kv = {k: str(v) for k, v in kv.items() if v is not None}

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update(self.kv)

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


def _run(w, a, pps=None, mode=None, order=None):
    """pps forces split mode with that many pages per split; mode="split" forces
    split mode with the default split size; otherwise the library chooses (whole
    unit where the staging fits)."""
    from rl_rollout_amd import s3r
    with _env(S3R_VERIFY_PAGES_PER_SPLIT=pps, S3R_VERIFY_MODE=mode, S3R_VERIFY_ORDER=order):
        kv = upload_cache(a)
        out, scores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
        torch.cuda.synchronize()
    return host(out), host(scores)


def _check(w, a, pps=None, mode=None, order=None):
    print(f"verify {w.name} dtype={w.kv_dtype} lens={list(a.ctx_lens)} G1={w.block_len} pps={pps} mode={mode} "
          f"order={order}", flush=True)
    out, scores = _run(w, a, pps, mode, order)
    ref, ref_scores = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    err = max_row_rel_err(out, ref)
    assert err <= TOL[w.kv_dtype], err
    rtol = page_score_rtol(a.q_verify, a.k_cache, w.block_len * w.num_q_heads, w.kv_dtype)
    check_page_scores(scores, ref_scores, rtol, w.name)
    for b, L in enumerate(a.ctx_lens):
        n_pages = math.ceil((int(L) + w.block_len) / w.page_size)
        assert (scores[b, n_pages:] == 0).all()
    return out, scores


def test_verify_tiny_fp32_workload():
    w = W.TINY_FP32
    _check(w, synth.make_attn_inputs(w, 0))


@pytest.mark.parametrize("pps", [None, 3])
def test_verify_fp32_ragged_d128(pps):
    w = W.TINY_FP32.with_(num_seqs=4, num_q_heads=8, num_kv_heads=4, head_dim=128, gamma=3, spare_steps=2,
                          ctx_range=(0, 600))
    _check(w, synth.make_attn_inputs(w, 1, ctx_lens=np.array([0, 13, 200, 517])), pps)


@pytest.mark.parametrize("pps,mode", [(None, None), (5, None), (None, "split"), (None, "global")])
def test_verify_bf16_qwen3_1p7b_heads_ragged(pps, mode):
    """Whole-unit mode (the default for these shapes), small splits, split mode at
    the default split size, and whole-unit mode with the per-page staging in the
    workspace: all four against the oracle."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=4, ctx_range=(0, 2100), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 2, ctx_lens=np.array([5, 300, 1031, 2047])), pps, mode)


@pytest.mark.parametrize("mode", [None, "split", "global"])
def test_verify_bf16_more_than_1024_pages_per_sequence(mode):
    """Pages beyond the first 1024 of a sequence: whole-unit mode then reads block
    ids from its fifth lane register; split mode cuts five splits."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 16500), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 8, ctx_lens=np.array([16400, 4097])), None, mode)


@pytest.mark.parametrize("order", ["lpt", "natural"])
def test_verify_longest_first_order(order):
    """Whole-unit mode with units taken longest first (ties to the lower index) and
    in natural order: same results, against the oracle."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=7, ctx_range=(0, 1300), spare_steps=2)
    lens = np.array([40, 1290, 300, 300, 0, 777, 1290])
    _check(w, synth.make_attn_inputs(w, 9, ctx_lens=lens), None, None, order)


def test_verify_bf16_more_than_2048_pages_falls_back_to_split_mode():
    """Page tables longer than whole-unit mode's 2048 lane-held block ids: the plan
    picks split mode by itself (nine splits of the longest sequence)."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 33000), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 10, ctx_lens=np.array([32900, 700])))


@pytest.mark.parametrize("mode", [None, "split", "global"])
def test_verify_bf16_qwen3_8b_heads_two_column_tiles(mode):
    # 7 block queries x 4 query heads per kv head = 28 rows: two 16-column MFMA
    # tiles, in split mode (the plan's choice for three sequences) and in
    # whole-unit mode with the staging in the workspace (its choice from 256 units)
    w = W.QWEN3_8B_24K.with_(num_seqs=3, ctx_range=(0, 1600), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 3, ctx_lens=np.array([17, 700, 1500])), None, mode)


@pytest.mark.parametrize("order", ["lpt", "natural"])
def test_verify_two_column_tiles_whole_unit_many_units(order):
    """Two column tiles on 40 sequences x 8 kv heads = 320 units, more than the
    chip's CUs: the plan takes whole-unit mode with global staging by itself; the
    windows of 16 pages per wave end ragged (lengths 0 .. 2040), in both unit
    orders."""
    w = W.QWEN3_8B_24K.with_(num_seqs=40, ctx_range=(0, 2048), spare_steps=2)
    lens = np.random.default_rng(23).integers(0, 2041, 40)
    lens[:4] = [0, 1, 63, 1017]  # 1017 + 7 block rows: 64 pages, one full window per wave
    _check(w, synth.make_attn_inputs(w, 23, ctx_lens=lens), None, None, order)


def test_verify_global_staging_chunk_boundaries():
    """Whole-unit mode with global staging (two column tiles, M = 28) at page counts
    around the 512-page staging chunks: 512 and 1536 (the last chunk exactly full),
    513 and 1025 (the first chunk holds 4 pages), 515 and 1027 (the last chunk 3
    pages short of full), 1028 (both full), and 400 (nothing leaves LDS); tails
    full and partial."""
    w = W.QWEN3_8B_24K.with_(num_seqs=8, ctx_range=(0, 24600), spare_steps=2)
    pages = [512, 1536, 513, 1025, 515, 1027, 1028, 400]
    lens = np.array([16 * n - w.block_len - (3 if i % 2 else 0) for i, n in enumerate(pages)])
    assert [math.ceil((int(L) + w.block_len) / w.page_size) for L in lens] == pages
    _check(w, synth.make_attn_inputs(w, 31, ctx_lens=lens), None, "global")


def test_verify_bf16_head_dim_64():
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, head_dim=64, ctx_range=(0, 700), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 4, ctx_lens=np.array([64, 650])))


def test_verify_block_only_history():
    """L = 0: the queries see only the block's own rows (causal)."""
    w = W.TINY_FP32.with_(num_seqs=2, gamma=4, spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 5, ctx_lens=np.array([0, 0])))


def test_verify_deterministic():
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 1200), spare_steps=2)
    a = synth.make_attn_inputs(w, 6, ctx_lens=np.array([900, 1100]))
    o1, s1 = _run(w, a)
    o2, s2 = _run(w, a)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_verify_without_scores_matches_with_scores():
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 600), spare_steps=2)
    a = synth.make_attn_inputs(w, 7, ctx_lens=np.array([100, 555]))
    kv = upload_cache(a)
    q = dev(a.q_verify)
    o1, _ = s3r.s3r_dense_verify_attn(kv, q)
    o2, none = s3r.s3r_dense_verify_attn(kv, q, want_scores=False)
    assert none is None
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o1), host(o2))


@pytest.mark.parametrize("mode,pps,lens", [(None, None, [31, 700, 1023]), ("split", None, [31, 700, 1023]),
                                           (None, 3, [30, 46, 79])])
def test_verify_with_fused_append_equals_append_then_verify(mode, pps, lens):
    """s3r_dense_verify_attn_append gives the outputs, page scores and cache
    contents of s3r_append_kv followed by s3r_dense_verify_attn, bit for bit, and
    the oracle's. Lengths put the block across a page boundary; with 3-page
    splits also across a split boundary."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 1100), spare_steps=2)
    a = synth.make_attn_inputs(w, 17, ctx_lens=np.array(lens))
    print(f"verify append mode={mode} pps={pps} lens={lens}", flush=True)
    with _env(S3R_VERIFY_MODE=mode, S3R_VERIFY_PAGES_PER_SPLIT=pps):
        kv1, kv2 = upload_cache(a), upload_cache(a)
        q, kb, vb = dev(a.q_verify), dev(a.k_new), dev(a.v_new)
        s3r.s3r_append_kv(kv1, kb, vb, offset=0)
        o1, s1 = s3r.s3r_dense_verify_attn(kv1, q)
        o2, s2 = s3r.s3r_dense_verify_attn_append(kv2, q, kb, vb)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(s1), host(s2))
    assert torch.equal(kv1.k_cache, kv2.k_cache) and torch.equal(kv1.v_cache, kv2.v_cache)
    # oracle: the block rows written by definition
    k, v = a.k_cache.copy(), a.v_cache.copy()
    for b, L in enumerate(a.ctx_lens):
        for i in range(w.block_len):
            pos = int(L) + i
            blk = a.page_table[b, pos // 16]
            k[blk, :, pos % 16, :] = a.k_new[b, i]
            v[blk, :, :, pos % 16] = a.v_new[b, i]
    ref, ref_s = oracle.dense_verify_attn(a.q_verify, k, v, a.page_table, a.ctx_lens)
    assert max_row_rel_err(host(o2), ref) <= TOL[w.kv_dtype]
    check_page_scores(host(s2), ref_s, page_score_rtol(a.q_verify, np.concatenate([k.ravel(), a.k_new.ravel()]).reshape(-1, w.head_dim), w.block_len * w.num_q_heads, w.kv_dtype), "fused append")


@pytest.mark.parametrize("mode", [None, "split", "global"])
def test_verify_per_kv_head_scores(mode):
    """s3r_dense_verify_attn_head_scores: per-kv-head page scores against the
    oracle's, zero past the visible pages, summing to the shared scores; the same
    attention outputs."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 2100), spare_steps=2)
    a = synth.make_attn_inputs(w, 19, ctx_lens=np.array([7, 1500, 2047]))
    print(f"verify per-head scores mode={mode}", flush=True)
    with _env(S3R_VERIFY_MODE=mode):
        kv = upload_cache(a)
        q = dev(a.q_verify)
        o, hs = s3r.s3r_dense_verify_attn_head_scores(kv, q)
        o2, ss = s3r.s3r_dense_verify_attn(kv, q)
        torch.cuda.synchronize()
    ref, ref_h = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens, per_head=True)
    assert max_row_rel_err(host(o), ref) <= TOL[w.kv_dtype]
    np.testing.assert_array_equal(host(o), host(o2))
    h = host(hs)
    g = w.num_q_heads // w.num_kv_heads
    check_page_scores(h, ref_h, page_score_rtol(a.q_verify, a.k_cache, w.block_len * g, w.kv_dtype), "per kv head")
    # the per-head scores of the GPU add up to its shared scores: both within their bounds of the oracle's
    tot = page_score_rtol(a.q_verify, a.k_cache, w.block_len * w.num_q_heads, w.kv_dtype) + \
        page_score_rtol(a.q_verify, a.k_cache, w.block_len * g + w.num_kv_heads, w.kv_dtype)
    check_page_scores(h.sum(axis=1), host(ss), tot, "sum of per-kv-head scores against the shared ones")
    for b, L in enumerate(a.ctx_lens):
        n_pages = math.ceil((int(L) + w.block_len) / w.page_size)
        assert (h[b, :, n_pages:] == 0).all()


@pytest.mark.parametrize("hq,hkv,gamma,mode", [(4, 4, 4, None), (4, 4, 4, "split"), (16, 2, 3, None), (16, 2, 3, "split"),
                                               (8, 1, 3, None), (16, 2, 3, "global"), (4, 4, 4, "global")],
                         ids=["g1_unit", "g1_split", "g8_two_tiles", "g8_split", "g8_one_kv_head", "g8_global",
                              "g1_global"])
def test_verify_group_sizes_one_and_eight(hq, hkv, gamma, mode):
    """GQA groups of 1 and 8: with 8 query heads per kv head a block of 4 queries
    fills both 16-column tiles (M = 32, the largest block the kernel takes)."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, gamma=gamma, ctx_range=(0, 1500),
                               spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 14, ctx_lens=np.array([3, 700, 1499])), None, mode)


def test_verify_bf16_128k_context():
    """A 128K-token history: 8193 pages, 33 splits of the default 256 pages, so the
    combine merges split statistics over five load batches."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 131072), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 15, ctx_lens=np.array([131067, 2500])))


@pytest.mark.parametrize("hq,hkv,gamma,d,pps,mode", [(32, 8, 6, 128, None, None), (32, 8, 6, 128, 5, None),
                                                     (16, 2, 3, 64, None, None), (32, 8, 6, 128, None, "global"),
                                                     (16, 2, 3, 64, None, "global")],
                         ids=["m28_d128", "m28_d128_small_splits", "m32_d64", "m28_d128_global", "m32_d64_global"])
def test_verify_fp32_two_column_tiles(hq, hkv, gamma, d, pps, mode):
    """fp32 KV with blocks of 28 and 32 rows: two 16-column tiles on the fp32 MFMA
    path, in split mode and in whole-unit mode with global staging."""
    w = W.QWEN3_8B_24K.with_(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, gamma=gamma, head_dim=d, kv_dtype="f32",
                             ctx_range=(0, 1300), spare_steps=2)
    _check(w, synth.make_attn_inputs(w, 18, ctx_lens=np.array([9, 610, 1290])), pps, mode)
