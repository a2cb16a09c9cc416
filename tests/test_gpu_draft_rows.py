"""s3r_sparse_draft_attn_rows (the in-flight draft tokens' K/V rows read from the
caller's buffers, the cache read only below L_b) against the fp64 oracle, and the
attention kernels with large finite garbage in every cache slot past the positions
they attend (keys of 40 in every dim, values of 1000): a garbage key that got any
weight would dominate its row's softmax and show in the output."""
import math

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import TOL, check_page_scores, dev, host, max_row_rel_err, page_score_rtol

pytestmark = pytest.mark.gpu

GARBAGE_K, GARBAGE_V = 40.0, 1000.0  # exact in bf16


def _rows_from_cache(a, n):
    """[n][B][Hkv][D] K and V rows at positions L_b .. L_b + n - 1, read from the cache."""
    B = len(a.ctx_lens)
    _, Hkv, P, D = a.k_cache.shape
    kr = np.zeros((n, B, Hkv, D), dtype=a.k_cache.dtype)
    vr = np.zeros((n, B, Hkv, D), dtype=a.v_cache.dtype)
    for r in range(n):
        for b, L in enumerate(a.ctx_lens):
            t = int(L) + r
            blk = a.page_table[b, t // P]
            kr[r, b] = a.k_cache[blk, :, t % P, :]
            vr[r, b] = a.v_cache[blk, :, :, t % P]
    return kr, vr


def _garbage(a, first):
    """Copies of the caches with garbage at every position t >= first[b] of sequence
    b (each sequence owns its blocks)."""
    k, v = a.k_cache.copy(), a.v_cache.copy()
    if k.dtype == np.uint16:
        gk = synth.f32_to_bf16_bits(np.array([GARBAGE_K], dtype=np.float32))[0]
        gv = synth.f32_to_bf16_bits(np.array([GARBAGE_V], dtype=np.float32))[0]
    else:
        gk, gv = np.float32(GARBAGE_K), np.float32(GARBAGE_V)
    P = k.shape[2]
    for b in range(len(a.ctx_lens)):
        for t in range(int(first[b]), a.page_table.shape[1] * P):
            blk = a.page_table[b, t // P]
            k[blk, :, t % P, :] = gk
            v[blk, :, :, t % P] = gv
    return k, v


def _kv(a, k, v):
    from rl_rollout_amd import s3r
    lens = torch.from_numpy(a.ctx_lens.astype(np.int32)).cuda()
    return s3r.KVCache(dev(k), dev(v), dev(a.page_table.astype(np.int32)), lens)


def _random_sel(lens, P, frac, rng):
    out = []
    for L in lens:
        nf = int(L) // P
        k = oracle.num_selected(nf, frac) if nf else 0
        out.append(np.sort(rng.choice(nf, size=k, replace=False)) if k else np.array([], dtype=np.int64))
    return out


def _sel_arrays(sel):
    B = len(sel)
    k = max(1, max(len(s) for s in sel))
    arr = np.full((B, k), -1, dtype=np.int32)
    ns = np.zeros(B, dtype=np.int32)
    for b, s in enumerate(sel):
        arr[b, :len(s)] = s
        ns[b] = len(s)
    return arr, ns


CASES = {
    # name: (workload, lens, steps)
    "tiny_fp32_d64": (W.TINY_FP32, [256, 250], [1, 2, 4]),
    "qwen3_1p7b_heads": (W.QWEN3_1P7B_16K.with_(num_seqs=4, ctx_range=(0, 3000), spare_steps=2),
                         [15, 16, 1000, 2999], [1, 2, 4]),
    "qwen3_8b_heads": (W.QWEN3_8B_24K.with_(num_seqs=3, ctx_range=(0, 2000), spare_steps=2),
                       [9, 510, 1999], [1, 6]),
    # the smallest and largest GQA groups
    "group_1": (W.QWEN3_1P7B_16K.with_(num_seqs=3, num_q_heads=4, num_kv_heads=4, ctx_range=(0, 1200), spare_steps=2),
                [5, 300, 1199], [1, 4]),
    "group_8": (W.QWEN3_1P7B_16K.with_(num_seqs=3, num_q_heads=16, num_kv_heads=2, ctx_range=(0, 1200), spare_steps=2),
                [17, 640, 1100], [1, 4]),
    # fp32 KV at d = 128 (the eight-wave row-mode instance)
    "fp32_d128_group_4": (W.QWEN3_8B_24K.with_(num_seqs=3, kv_dtype="f32", ctx_range=(0, 1500), spare_steps=2),
                          [2, 777, 1490], [1, 3, 6]),
    # twenty draft steps: the rows span two 16-key pages; an empty history (L = 0)
    "twenty_rows": (W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 800), gamma=20, spare_steps=2),
                    [0, 33, 700], [1, 17, 20]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_draft_rows_against_oracle_with_garbage_from_L(case):
    """The rows mode equals the oracle's draft (rows appended to the cache) while the
    device cache holds garbage at every position >= L_b: the in-flight rows come from
    the row buffers only."""
    from rl_rollout_amd import s3r
    w, lens, steps = CASES[case]
    a = synth.make_attn_inputs(w, 31, ctx_lens=np.array(lens))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.2, np.random.default_rng(7))
    sel_arr, ns = _sel_arrays(sel)
    kr, vr = _rows_from_cache(a, w.gamma)
    kp, vp = _garbage(a, a.ctx_lens)
    kv = _kv(a, kp, vp)
    for j in steps:
        print(f"draft rows {case} lens={lens} step={j}", flush=True)
        out = s3r.s3r_sparse_draft_attn_rows(kv, dev(a.q_draft[j - 1]), dev(kr), dev(vr), dev(sel_arr), dev(ns), j)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
        o = host(out)
        assert np.isfinite(o).all()
        assert max_row_rel_err(o, ref) <= TOL[w.kv_dtype], j


@pytest.mark.parametrize("case", ["qwen3_1p7b_heads", "twenty_rows"])
def test_draft_rows_from_a_sequence_major_buffer(case):
    """Rows kept one sequence's rows adjacent ([B][rows][Hkv][D], passed as a permuted
    view: row stride Hkv * D, sequence stride rows * Hkv * D) give the same outputs as
    the [rows][B][Hkv][D] buffer."""
    from rl_rollout_amd import s3r
    w, lens, steps = CASES[case]
    a = synth.make_attn_inputs(w, 35, ctx_lens=np.array(lens))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.2, np.random.default_rng(10))
    sel_arr, ns = _sel_arrays(sel)
    kr, vr = _rows_from_cache(a, w.gamma)
    kp, vp = _garbage(a, a.ctx_lens)
    kv = _kv(a, kp, vp)
    kr_d, vr_d = dev(kr), dev(vr)
    kr_s = kr_d.permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    vr_s = vr_d.permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    assert kr_s.stride(0) == kr.shape[2] * kr.shape[3] and kr_s.stride(1) == w.gamma * kr.shape[2] * kr.shape[3]
    for j in steps:
        print(f"draft rows sequence-major {case} step={j}", flush=True)
        o1 = s3r.s3r_sparse_draft_attn_rows(kv, dev(a.q_draft[j - 1]), kr_d, vr_d, dev(sel_arr), dev(ns), j)
        o2 = s3r.s3r_sparse_draft_attn_rows(kv, dev(a.q_draft[j - 1]), kr_s, vr_s, dev(sel_arr), dev(ns), j)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(o1), host(o2))


def test_draft_rows_with_a_page_set_per_kv_head():
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 2100), spare_steps=2)
    a = synth.make_attn_inputs(w, 32, ctx_lens=np.array([40, 900, 2047]))
    rng = np.random.default_rng(8)
    Hkv = w.num_kv_heads
    per = [[_random_sel([L], w.page_size, 0.2, rng)[0] for _ in range(Hkv)] for L in a.ctx_lens]
    k = max(1, max(len(s) for row in per for s in row))
    sel = np.full((3, Hkv, k), -1, dtype=np.int32)
    ns = np.zeros((3, Hkv), dtype=np.int32)
    for b in range(3):
        for h in range(Hkv):
            sel[b, h, :len(per[b][h])] = per[b][h]
            ns[b, h] = len(per[b][h])
    kr, vr = _rows_from_cache(a, w.gamma)
    kp, vp = _garbage(a, a.ctx_lens)
    kv = _kv(a, kp, vp)
    for j in (1, 4):
        print(f"draft rows per-head selection step={j}", flush=True)
        out = s3r.s3r_sparse_draft_attn_rows(kv, dev(a.q_draft[j - 1]), dev(kr), dev(vr), dev(sel), dev(ns), j)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, per, j,
                                       per_head=True)
        assert max_row_rel_err(host(out), ref) <= TOL[w.kv_dtype]


@pytest.mark.parametrize("case", ["tiny_fp32_d64", "qwen3_1p7b_heads", "qwen3_8b_heads"])
def test_draft_ignores_garbage_past_its_query(case):
    """s3r_sparse_draft_attn with garbage at every position past pi = L_b + j - 1."""
    from rl_rollout_amd import s3r
    w, lens, steps = CASES[case]
    a = synth.make_attn_inputs(w, 33, ctx_lens=np.array(lens))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.2, np.random.default_rng(9))
    sel_arr, ns = _sel_arrays(sel)
    for j in steps:
        kp, vp = _garbage(a, a.ctx_lens + j)
        kv = _kv(a, kp, vp)
        print(f"draft garbage tail {case} step={j}", flush=True)
        out = s3r.s3r_sparse_draft_attn(kv, dev(a.q_draft[j - 1]), dev(sel_arr), dev(ns), j)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
        o = host(out)
        assert np.isfinite(o).all()
        assert max_row_rel_err(o, ref) <= TOL[w.kv_dtype], j


@pytest.mark.parametrize("case,mode", [("tiny_fp32_d64", None), ("qwen3_1p7b_heads", None),
                                       ("qwen3_1p7b_heads", "split"), ("qwen3_8b_heads", None),
                                       ("qwen3_8b_heads", "global"), ("qwen3_1p7b_heads", "global")])
def test_verify_ignores_garbage_past_the_block(case, mode, monkeypatch):
    """s3r_dense_verify_attn (whole-unit and split mode) with garbage at every
    position past the block, L_b + G1 and beyond: outputs and page scores as the
    oracle's."""
    from rl_rollout_amd import s3r
    if mode is not None:
        monkeypatch.setenv("S3R_VERIFY_MODE", mode)
    w, lens, _ = CASES[case]
    a = synth.make_attn_inputs(w, 34, ctx_lens=np.array(lens))
    kp, vp = _garbage(a, a.ctx_lens + w.block_len)
    kv = _kv(a, kp, vp)
    print(f"verify garbage tail {case} mode={mode}", flush=True)
    out, scores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
    torch.cuda.synchronize()
    ref, ref_scores = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    o = host(out)
    assert np.isfinite(o).all()
    assert max_row_rel_err(o, ref) <= TOL[w.kv_dtype]
    check_page_scores(host(scores), ref_scores,
                      page_score_rtol(a.q_verify, a.k_cache, w.block_len * w.num_q_heads, w.kv_dtype), case)
