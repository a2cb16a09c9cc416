"""GPU parity of s3r_sparse_draft_attn against the fp64 oracle, and the
budget-1.0 invariant on the GPU (all full pages selected equals dense attention
of the same query)."""
import os

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import TOL, dev, host, max_row_rel_err, upload_cache

pytestmark = pytest.mark.gpu


def _sel_arrays(sel, max_sel):
    B = len(sel)
    arr = np.full((B, max_sel), -1, dtype=np.int32)
    ns = np.zeros(B, dtype=np.int32)
    for b, s in enumerate(sel):
        arr[b, :len(s)] = s
        ns[b] = len(s)
    return arr, ns


def _random_sel(lens, P, frac, rng):
    out = []
    for L in lens:
        nf = int(L) // P
        k = oracle.num_selected(nf, frac) if nf else 0
        out.append(np.sort(rng.choice(nf, size=k, replace=False)) if k else np.array([], dtype=np.int64))
    return out


def _check(w, a, sel, steps):
    from rl_rollout_amd import s3r
    kv = upload_cache(a)
    max_sel = max(1, max(len(s) for s in sel))
    sel_arr, ns = _sel_arrays(sel, max_sel)
    for j in steps:
        print(f"draft {w.name} dtype={w.kv_dtype} lens={list(a.ctx_lens)} n_sel={list(ns)} step={j}", flush=True)
        out = s3r.s3r_sparse_draft_attn(kv, dev(a.q_draft[j - 1]), dev(sel_arr), dev(ns), j)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
        err = max_row_rel_err(host(out), ref)
        assert err <= TOL[w.kv_dtype], (j, err)


def test_draft_tiny_fp32_workload_oracle_selection():
    w = W.TINY_FP32
    a = synth.make_attn_inputs(w, 0)
    _, scores = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    sel = oracle.select_budget(scores, a.ctx_lens, w.page_size, w.budget)
    assert all(len(s) == 4 for s in sel)        # 4 of 16 pages
    _check(w, a, sel, range(1, w.gamma + 1))


@pytest.mark.parametrize("frac", [0.05, 0.3, 1.0])
def test_draft_bf16_qwen3_1p7b_heads(frac):
    w = W.QWEN3_1P7B_16K.with_(num_seqs=4, ctx_range=(0, 3000), spare_steps=2)
    a = synth.make_attn_inputs(w, 11, ctx_lens=np.array([15, 16, 1000, 2999]))
    sel = _random_sel(a.ctx_lens, w.page_size, frac, np.random.default_rng(1))
    _check(w, a, sel, [1, 2, 4])


def test_draft_bf16_qwen3_8b_heads_and_long_tail_step():
    w = W.QWEN3_8B_24K.with_(num_seqs=3, ctx_range=(0, 2000), spare_steps=2)
    a = synth.make_attn_inputs(w, 12, ctx_lens=np.array([9, 510, 1999]))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.1, np.random.default_rng(2))
    _check(w, a, sel, [1, 6])


@pytest.mark.parametrize("order", ["lpt", "natural"])
def test_draft_longest_first_order(order):
    """Units taken longest first (attended pages descending, index ascending) and in
    natural order give the oracle's outputs."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=6, ctx_range=(0, 2000), spare_steps=2)
    a = synth.make_attn_inputs(w, 16, ctx_lens=np.array([1900, 17, 600, 600, 1999, 250]))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.2, np.random.default_rng(3))
    old = os.environ.get("S3R_DRAFT_ORDER")
    os.environ["S3R_DRAFT_ORDER"] = order
    try:
        _check(w, a, sel, [1, 4])
    finally:
        if old is None:
            del os.environ["S3R_DRAFT_ORDER"]
        else:
            os.environ["S3R_DRAFT_ORDER"] = old


@pytest.mark.parametrize("order", ["lpt", "natural"])
def test_draft_order_covers_every_unit_once(order):
    """37 sequences (not a multiple of the ranking's four-entry reads, more than one
    unrolled pass of them) in groups of equal attended pages, empty histories among
    them, with the output filled with NaN first: in either order every (sequence,
    kv head) unit is written, with the oracle's values."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=37, ctx_range=(0, 1300), spare_steps=2)
    lens = np.array([1200, 0, 700, 700, 1200, 33, 0, 700] * 5)[:37]
    lens[36] = 1299
    a = synth.make_attn_inputs(w, 21, ctx_lens=lens)
    sel = _random_sel(a.ctx_lens, w.page_size, 0.1, np.random.default_rng(9))
    kv = upload_cache(a)
    sel_arr, ns = _sel_arrays(sel, max(1, max(len(x) for x in sel)))
    old = os.environ.get("S3R_DRAFT_ORDER")
    os.environ["S3R_DRAFT_ORDER"] = order
    try:
        for j in (1, 3):
            print(f"draft order {order} B=37 step {j}", flush=True)
            q = dev(a.q_draft[j - 1])
            out = torch.full_like(q, float("nan"))
            s3r.s3r_sparse_draft_attn(kv, q, dev(sel_arr), dev(ns), j, out=out)
            torch.cuda.synchronize()
            got = host(out)
            ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
            assert max_row_rel_err(got, ref) <= TOL[w.kv_dtype], j
    finally:
        if old is None:
            del os.environ["S3R_DRAFT_ORDER"]
        else:
            os.environ["S3R_DRAFT_ORDER"] = old


def test_draft_empty_selection_and_head_dim_64():
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, head_dim=64, ctx_range=(0, 800), spare_steps=2)
    a = synth.make_attn_inputs(w, 13, ctx_lens=np.array([40, 777]))
    _check(w, a, [np.array([], dtype=np.int64)] * 2, [1, 3])


def test_draft_fp32_more_entries_than_one_pass():
    """More than 8 waves x 64 entries: the entry loop wraps."""
    w = W.TINY_FP32.with_(num_seqs=1, num_q_heads=4, num_kv_heads=2, head_dim=64, spare_steps=2,
                          ctx_range=(0, 9000))
    a = synth.make_attn_inputs(w, 14, ctx_lens=np.array([8500]))
    sel = [np.arange(8500 // 16)]
    _check(w, a, sel, [2])


def test_draft_full_budget_equals_gpu_dense_attention():
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 1500), spare_steps=2)
    a = synth.make_attn_inputs(w, 15, ctx_lens=np.array([33, 600, 1400]))
    kv = upload_cache(a)
    sel = [np.arange(int(L) // 16) for L in a.ctx_lens]
    sel_arr, ns = _sel_arrays(sel, max(len(s) for s in sel))
    j = 3
    q = dev(a.q_draft[j - 1])
    d = host(s3r.s3r_sparse_draft_attn(kv, q, dev(sel_arr), dev(ns), j))
    lens2 = torch.from_numpy(a.ctx_lens + (j - 1)).cuda()
    kv2 = s3r.KVCache(kv.k_cache, kv.v_cache, kv.page_table, lens2)
    v, _ = s3r.s3r_dense_verify_attn(kv2, q[:, None].contiguous(), want_scores=False)
    torch.cuda.synchronize()
    assert max_row_rel_err(d, host(v)[:, 0]) <= 2e-2


@pytest.mark.parametrize("lens", [[15, 16, 1000], [0, 33, 2047]])
def test_draft_with_fused_append_equals_append_then_draft(lens):
    """s3r_sparse_draft_attn_append gives the outputs and cache contents of
    s3r_append_kv followed by s3r_sparse_draft_attn, bit for bit, and the oracle's."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 2100), spare_steps=2)
    a = synth.make_attn_inputs(w, 18, ctx_lens=np.array(lens))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.25, np.random.default_rng(4))
    sel_arr, ns = _sel_arrays(sel, max(1, max(len(s) for s in sel)))
    kv1, kv2 = upload_cache(a), upload_cache(a)
    k_cache, v_cache = a.k_cache.copy(), a.v_cache.copy()
    for j in (1, 2, 3):
        print(f"draft append lens={lens} step={j}", flush=True)
        q, kr, vr = dev(a.q_draft[j - 1]), dev(a.k_new[:, j - 1]), dev(a.v_new[:, j - 1])
        s3r.s3r_append_kv(kv1, kr[:, None].contiguous(), vr[:, None].contiguous(), offset=j - 1)
        o1 = s3r.s3r_sparse_draft_attn(kv1, q, dev(sel_arr), dev(ns), j)
        o2 = s3r.s3r_sparse_draft_attn_append(kv2, q, kr, vr, dev(sel_arr), dev(ns), j)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(o1), host(o2))
        assert torch.equal(kv1.k_cache, kv2.k_cache) and torch.equal(kv1.v_cache, kv2.v_cache)
        for b, L in enumerate(a.ctx_lens):
            pos = int(L) + j - 1
            blk = a.page_table[b, pos // 16]
            k_cache[blk, :, pos % 16, :] = a.k_new[b, j - 1]
            v_cache[blk, :, :, pos % 16] = a.v_new[b, j - 1]
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], k_cache, v_cache, a.page_table, a.ctx_lens, sel, j)
        assert max_row_rel_err(host(o2), ref) <= TOL[w.kv_dtype]


def test_draft_with_a_page_set_per_kv_head():
    """s3r_sparse_draft_attn_head_sel: each kv head's query heads attend that
    head's own selected pages plus the tail (oracle per_head=True); with the same
    set for every head it equals s3r_sparse_draft_attn."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 2100), spare_steps=2)
    a = synth.make_attn_inputs(w, 20, ctx_lens=np.array([40, 900, 2047]))
    rng = np.random.default_rng(5)
    Hkv = w.num_kv_heads
    per = [[_random_sel([L], w.page_size, 0.2, rng)[0] for _ in range(Hkv)] for L in a.ctx_lens]
    k = max(1, max(len(s) for row in per for s in row))
    sel = np.full((3, Hkv, k), -1, dtype=np.int32)
    ns = np.zeros((3, Hkv), dtype=np.int32)
    for b in range(3):
        for h in range(Hkv):
            sel[b, h, :len(per[b][h])] = per[b][h]
            ns[b, h] = len(per[b][h])
    kv = upload_cache(a)
    for j in (1, 3):
        print(f"draft per-head selection step={j}", flush=True)
        out = s3r.s3r_sparse_draft_attn_head_sel(kv, dev(a.q_draft[j - 1]), dev(sel), dev(ns), j)
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, per, j,
                                       per_head=True)
        assert max_row_rel_err(host(out), ref) <= TOL[w.kv_dtype]
    same = np.repeat(sel[:, :1], Hkv, axis=1)
    same_n = np.repeat(ns[:, :1], Hkv, axis=1)
    o1 = s3r.s3r_sparse_draft_attn_head_sel(kv, dev(a.q_draft[0]), dev(np.ascontiguousarray(same)),
                                            dev(np.ascontiguousarray(same_n)), 1)
    o2 = s3r.s3r_sparse_draft_attn(kv, dev(a.q_draft[0]), dev(np.ascontiguousarray(sel[:, 0])),
                                   dev(np.ascontiguousarray(ns[:, 0])), 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o1), host(o2))


@pytest.mark.parametrize("hq,hkv,dtype", [(4, 4, "bf16"), (16, 2, "bf16"), (8, 8, "f32"), (16, 2, "f32")],
                         ids=["g1_bf16", "g8_bf16", "g1_f32", "g8_f32"])
def test_draft_group_sizes_one_and_eight(hq, hkv, dtype):
    """The smallest and largest supported GQA groups (1 and 8 query heads per kv head)."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=dtype, ctx_range=(0, 1500),
                               spare_steps=2)
    a = synth.make_attn_inputs(w, 13, ctx_lens=np.array([7, 600, 1499]))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.2, np.random.default_rng(4))
    _check(w, a, sel, [1, 4])


def test_draft_bf16_128k_context():
    """A 128K-token history with 5 % of its pages selected: 410 pages, more than one
    pass of the workgroup's page loop."""
    w = W.QWEN3_1P7B_16K.with_(num_seqs=2, ctx_range=(0, 131072), spare_steps=2)
    a = synth.make_attn_inputs(w, 16, ctx_lens=np.array([131067, 2500]))
    sel = _random_sel(a.ctx_lens, w.page_size, 0.05, np.random.default_rng(5))
    _check(w, a, sel, [1, 4])
