"""GPU parity of s3r_select_budget (bit-exact page sets on identical fp32 scores,
ties included) and of s3r_append_kv (bit-exact scatter into the paged cache)."""
import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import dev, host, selection_mismatch_exempt, upload_cache

pytestmark = pytest.mark.gpu


def _select(scores, lens, budget, max_sel):
    from rl_rollout_amd import s3r
    sel, ns = s3r.s3r_select_budget(dev(scores), dev(lens.astype(np.int32)), budget, max_sel)
    torch.cuda.synchronize()
    return host(sel), host(ns)


@pytest.mark.parametrize("budget", [0.05, 0.10, 0.25, 0.5, 1.0])
def test_select_matches_oracle_with_ties(budget):
    rng = np.random.default_rng(int(budget * 100))
    B, MP = 9, 1100
    lens = np.array([0, 15, 16, 17, 1000, 4096, 9999, 16383, 16384 + 20], dtype=np.int32)
    lens = np.minimum(lens, MP * 16)
    S = (rng.random((B, MP)) * 0.2).astype(np.float32)
    S[5, 10:200] = np.float32(0.1)           # long runs of exact ties
    S[6, ::2] = S[6, 1]
    S[7] = np.float32(0.05)                  # every score equal
    S[8, :5] = 0.0                           # zeros
    max_sel = max(1, int(np.ceil(budget * MP)))
    print(f"select budget={budget} lens={list(lens)}", flush=True)
    sel, ns = _select(S, lens, budget, max_sel)
    ref = oracle.select_budget(S, lens, 16, budget)
    for b in range(B):
        assert ns[b] == len(ref[b])
        np.testing.assert_array_equal(sel[b, :ns[b]], ref[b])
        assert (sel[b, ns[b]:] == -1).all()


@pytest.mark.parametrize("budget", [0.05, 0.5])
def test_select_128k_context(budget):
    """Page tables of 8200 entries (128K-token histories): radix passes over rows
    eight times longer than the 16K workload's, with a run of exact ties."""
    rng = np.random.default_rng(17)
    B, MP = 3, 8200
    lens = np.array([131067, 70000, 2500], dtype=np.int32)
    S = (rng.random((B, MP)) * 0.2).astype(np.float32)
    S[0, 4000:6000] = np.float32(0.15)
    max_sel = int(np.ceil(budget * MP))
    print(f"select 128K budget={budget}", flush=True)
    sel, ns = _select(S, lens, budget, max_sel)
    ref = oracle.select_budget(S, lens, 16, budget)
    for b in range(B):
        assert ns[b] == len(ref[b])
        np.testing.assert_array_equal(sel[b, :ns[b]], ref[b])
        assert (sel[b, ns[b]:] == -1).all()


def test_select_with_a_budget_per_row():
    """s3r_select_budget_rows against the oracle with one budget per row (ties,
    empty rows, a budget of 1 and budgets rounding to one page)."""
    from rl_rollout_amd import s3r
    rng = np.random.default_rng(13)
    B, MP = 9, 1100
    lens = np.array([0, 15, 16, 17, 1000, 4096, 9999, 16383, 16384 + 20], dtype=np.int32)
    S = (rng.random((B, MP)) * 0.2).astype(np.float32)
    S[5, 10:200] = np.float32(0.1)
    S[7] = np.float32(0.05)
    budgets = np.array([0.5, 0.05, 1.0, 0.3, 0.1, 0.25, 0.05, 0.02, 0.5], dtype=np.float64)
    max_sel = int(np.ceil(budgets.max() * MP))
    print(f"select per-row budgets {list(budgets)}", flush=True)
    sel_t, ns_t = s3r.s3r_select_budget(dev(S), dev(lens), dev(budgets), max_sel)
    torch.cuda.synchronize()
    sel, ns = host(sel_t), host(ns_t)
    ref = oracle.select_budget(S, lens, 16, budgets)
    for b in range(B):
        assert ns[b] == len(ref[b]), b
        np.testing.assert_array_equal(sel[b, :ns[b]], ref[b])
        assert (sel[b, ns[b]:] == -1).all()


def test_select_on_gpu_verify_scores_tiny_workload():
    """4 of 16 pages: the GPU selection over the GPU's verify scores equals the
    oracle's selection over the oracle's scores of the same inputs (up to the
    near-tie window)."""
    from rl_rollout_amd import s3r
    w = W.TINY_FP32
    a = synth.make_attn_inputs(w, 0)
    kv = upload_cache(a)
    _, scores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
    torch.cuda.synchronize()
    sel, ns = _select(host(scores), a.ctx_lens, w.budget, 8)
    _, ref_s = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    ref = oracle.select_budget(ref_s, a.ctx_lens, 16, w.budget)
    assert list(ns) == [4, 4]
    for b in range(2):
        assert selection_mismatch_exempt(ref_s[b], int(a.ctx_lens[b]) // 16, 4, sel[b, :4], ref[b])


def test_select_per_kv_head_rows_from_gpu_head_scores():
    """A page set per kv head: select over num_seqs x num_kv_heads rows of the
    GPU's per-head scores (lengths repeated per head); against the oracle's
    per-head scores and selection of the same inputs."""
    from rl_rollout_amd import s3r
    w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 2100), spare_steps=2)
    a = synth.make_attn_inputs(w, 22, ctx_lens=np.array([100, 1200, 2047]))
    kv = upload_cache(a)
    _, hs = s3r.s3r_dense_verify_attn_head_scores(kv, dev(a.q_verify))
    torch.cuda.synchronize()
    H = w.num_kv_heads
    rows = host(hs).reshape(3 * H, -1)
    lens_rows = np.repeat(a.ctx_lens, H)
    max_sel = int(np.ceil(0.1 * rows.shape[1]))
    sel, ns = _select(np.ascontiguousarray(rows), lens_rows, 0.1, max_sel)
    _, ref_h = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens, per_head=True)
    ref_rows = ref_h.reshape(3 * H, -1)
    ref = oracle.select_budget(ref_rows, lens_rows, 16, 0.1)
    differ = 0
    for r in range(3 * H):
        assert ns[r] == len(ref[r])
        assert selection_mismatch_exempt(ref_rows[r], int(lens_rows[r]) // 16, len(ref[r]), sel[r, :ns[r]], ref[r])
        differ += int(list(sel[r, :ns[r]]) != list(ref[r]))
    assert differ <= 1
    # the kv heads do pick different pages
    assert any(list(ref[r]) != list(ref[r + 1]) for r in range(0, 3 * H - 1) if (r + 1) % H)


def test_select_max_sel_at_the_bound():
    """max_sel must hold the largest selection (0.5 of 64 pages: 32). At exactly
    32 every page is written; at 31 the host rejects the call before any launch
    and leaves the outputs untouched."""
    from rl_rollout_amd import s3r
    S = np.arange(64, dtype=np.float32)[None, :].copy()
    sel, ns = _select(S, np.array([1024], dtype=np.int32), 0.5, 32)
    assert ns[0] == 32
    np.testing.assert_array_equal(sel[0], np.arange(32, 64))
    out = torch.full((1, 31), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(s3r.S3RError):
        s3r.s3r_select_budget(dev(S), dev(np.array([1024], dtype=np.int32)), 0.5, 31, sel_pages=out)
    torch.cuda.synchronize()
    assert (host(out) == -7).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_kv_scatter_is_exact(dtype):
    from rl_rollout_amd import s3r
    w = W.TINY_FP32.with_(num_seqs=3, num_q_heads=8, num_kv_heads=4, head_dim=128, kv_dtype=dtype, gamma=4,
                          spare_steps=2)
    a = synth.make_attn_inputs(w, 21, ctx_lens=np.array([0, 30, 250]))
    kv = upload_cache(a)
    off = 1
    kv_rows = dev(a.k_new)
    vv_rows = dev(a.v_new)
    s3r.s3r_append_kv(kv, kv_rows, vv_rows, offset=off)
    torch.cuda.synchronize()
    k_ref, v_ref = a.k_cache.copy(), a.v_cache.copy()
    for b, L in enumerate(a.ctx_lens):
        for r in range(w.block_len):
            t = int(L) + off + r
            blk = a.page_table[b, t // 16]
            k_ref[blk, :, t % 16, :] = a.k_new[b, r]
            v_ref[blk, :, :, t % 16] = a.v_new[b, r]
    kk = kv.k_cache.cpu()
    vv = kv.v_cache.cpu()
    if dtype == "bf16":
        kk = kk.view(torch.int16).numpy().view(np.uint16)
        vv = vv.view(torch.int16).numpy().view(np.uint16)
    else:
        kk, vv = kk.numpy(), vv.numpy()
    np.testing.assert_array_equal(kk, k_ref)
    np.testing.assert_array_equal(vv, v_ref)


@pytest.mark.parametrize("dtype,hkv", [("f32", 8), ("bf16", 16)])
def test_append_kv_second_pass_and_skipped_rows(dtype, hkv):
    """Rows of hkv x 128 elements that need a second pass of the workgroup (1024
    fp32 or 2048 bf16 elements), rows past the end of the page table (dropped) and
    rows whose page-table entry is -1 (dropped); every other element of the cache
    is left as it was."""
    from rl_rollout_amd import s3r
    w = W.TINY_FP32.with_(num_seqs=3, num_q_heads=hkv, num_kv_heads=hkv, head_dim=128, kv_dtype=dtype, gamma=4,
                          spare_steps=2)
    mp = w.max_pages()
    lens = np.array([17, 100, mp * 16 - 2], dtype=np.int32)
    a = synth.make_attn_inputs(w, 23, ctx_lens=lens)
    table = a.page_table.copy()
    hole_page = (int(lens[1]) + 1) // 16  # sequence 1's rows start on this page
    table[1, hole_page] = -1
    lens_t = torch.from_numpy(lens).cuda()
    kv = s3r.KVCache(dev(a.k_cache), dev(a.v_cache), dev(table.astype(np.int32)), lens_t)
    off = 1
    s3r.s3r_append_kv(kv, dev(a.k_new), dev(a.v_new), offset=off)
    torch.cuda.synchronize()
    k_ref, v_ref = a.k_cache.copy(), a.v_cache.copy()
    written = 0
    for b, L in enumerate(lens):
        for r in range(w.block_len):
            t = int(L) + off + r
            if t >= mp * 16:
                continue
            blk = table[b, t // 16]
            if blk < 0:
                continue
            k_ref[blk, :, t % 16, :] = a.k_new[b, r]
            v_ref[blk, :, :, t % 16] = a.v_new[b, r]
            written += 1
    assert 0 < written < 3 * w.block_len
    kk = kv.k_cache.cpu()
    vv = kv.v_cache.cpu()
    if dtype == "bf16":
        kk = kk.view(torch.int16).numpy().view(np.uint16)
        vv = vv.view(torch.int16).numpy().view(np.uint16)
    else:
        kk, vv = kk.numpy(), vv.numpy()
    np.testing.assert_array_equal(kk, k_ref)
    np.testing.assert_array_equal(vv, v_ref)


def test_select_at_the_largest_page_table():
    """32768 candidate pages (512K-token histories), the most the selection stages
    in LDS (128 KB of its keys): full rows, a shorter row and ties, against the
    oracle; one page more is refused on the host."""
    from rl_rollout_amd import s3r
    rng = np.random.default_rng(31)
    B, MP = 2, 32768
    lens = np.array([MP * 16, 300000], dtype=np.int32)
    S = (rng.random((B, MP)) * 0.05).astype(np.float32)
    S[0, 20000:21000] = np.float32(0.04)
    budget = 0.05
    max_sel = int(np.ceil(budget * MP))
    print(f"select 32768 pages budget={budget}", flush=True)
    sel, ns = _select(S, lens, budget, max_sel)
    ref = oracle.select_budget(S, lens, 16, budget)
    for b in range(B):
        assert ns[b] == len(ref[b])
        np.testing.assert_array_equal(sel[b, :ns[b]], ref[b])
    with pytest.raises(s3r.S3RError):
        s3r.s3r_select_budget(dev(np.zeros((1, MP + 1), np.float32)), dev(np.array([16], dtype=np.int32)), 0.05,
                              max_sel + 1)
