"""Pins for the oracle's dense verify attention, page scores and sparse draft
attention: closed forms, an independent library routine (torch's
scaled_dot_product_attention in float64 on the CPU), mass conservation and brute
force over explicit key sets. No GPU."""
import math

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W


def _dense_seq(cache, table_row, n, P, transposed):
    """Explicit per-token gather written independently of the oracle: returns
    [Hkv][n][D] float64 for the first n tokens of one sequence."""
    rows = []
    for t in range(n):
        blk = table_row[t // P]
        if transposed:
            rows.append(cache[blk, :, :, t % P])
        else:
            rows.append(cache[blk, :, t % P, :])
    x = np.stack(rows, axis=1)
    if x.dtype == np.uint16:
        x = synth.bf16_bits_to_f32(x)
    return x.astype(np.float64)


def _small(kv_dtype="f32", B=3, Hq=4, Hkv=2, D=32, lens=(5, 16, 37), gamma=3, seed=3):
    w = W.TINY_FP32.with_(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                          kv_dtype=kv_dtype, gamma=gamma, spare_steps=2)
    return w, synth.make_attn_inputs(w, seed, ctx_lens=np.array(lens, dtype=np.int32))


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_verify_matches_torch_sdpa_fp64(kv_dtype):
    w, a = _small(kv_dtype)
    out, _ = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    q = a.q_verify if a.q_verify.dtype != np.uint16 else synth.bf16_bits_to_f32(a.q_verify)
    g = w.group
    for b, L in enumerate(a.ctx_lens):
        n = int(L) + w.block_len
        K = torch.from_numpy(_dense_seq(a.k_cache, a.page_table[b], n, w.page_size, False))
        V = torch.from_numpy(_dense_seq(a.v_cache, a.page_table[b], n, w.page_size, True))
        K = K.repeat_interleave(g, dim=0)   # [Hq][n][D]
        V = V.repeat_interleave(g, dim=0)
        Q = torch.from_numpy(q[b].astype(np.float64)).permute(1, 0, 2)   # [Hq][G1][D]
        # query i at position L + i sees keys t <= L + i
        mask = torch.arange(n)[None, :] <= (int(L) + torch.arange(w.block_len))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_verify_single_visible_key_returns_its_value():
    w, a = _small(lens=(0, 0, 0), gamma=0)
    out, scores = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    for b in range(3):
        blk = a.page_table[b, 0]
        for h in range(w.num_q_heads):
            np.testing.assert_array_equal(out[b, 0, h], a.v_cache[blk, h // w.group, :, 0].astype(np.float64))
        assert scores[b, 0] == pytest.approx(w.num_q_heads, abs=1e-12)


def test_verify_identical_keys_and_zero_query_give_mean_value():
    w, a = _small()
    a.k_cache[:] = a.k_cache[0, 0, 0]          # every key identical
    out, _ = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    w2, a2 = _small()
    a2.q_verify[:] = 0.0                       # zero query: uniform weights
    out2, _ = oracle.dense_verify_attn(a2.q_verify, a2.k_cache, a2.v_cache, a2.page_table, a2.ctx_lens)
    for b, L in enumerate(a.ctx_lens):
        for i in range(w.block_len):
            n = int(L) + i + 1
            for arr, o in ((a, out), (a2, out2)):
                Vd = _dense_seq(arr.v_cache, arr.page_table[b], n, w.page_size, True)
                for h in range(w.num_q_heads):
                    np.testing.assert_allclose(o[b, i, h], Vd[h // w.group].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_verify_ignores_keys_past_each_query():
    w, a = _small()
    out, sc = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    # overwrite every slot past L_b + G1 - 1 and the block rows after query 0
    for b, L in enumerate(a.ctx_lens):
        for t in range(int(L) + 1, a.page_table.shape[1] * w.page_size):
            blk = a.page_table[b, t // w.page_size]
            a.k_cache[blk, :, t % w.page_size, :] = 100.0
            a.v_cache[blk, :, :, t % w.page_size] = -100.0
    out2, _ = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    np.testing.assert_array_equal(out[:, 0], out2[:, 0])
    assert not np.allclose(out[:, 1:], out2[:, 1:])


def test_page_scores_conserve_mass_and_match_brute_force():
    w, a = _small(Hq=6, Hkv=2, lens=(31, 64, 100))
    _, S = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    assert (S >= 0).all()
    np.testing.assert_allclose(S.sum(axis=1), w.block_len * w.num_q_heads, rtol=0, atol=1e-12)
    q = a.q_verify.astype(np.float64)
    for b, L in enumerate(a.ctx_lens):
        n = int(L) + w.block_len
        n_pages = math.ceil(n / w.page_size)
        assert (S[b, n_pages:] == 0).all()
        K = torch.from_numpy(_dense_seq(a.k_cache, a.page_table[b], n, w.page_size, False))
        ref = torch.zeros(a.page_table.shape[1], dtype=torch.float64)
        for h in range(w.num_q_heads):
            for i in range(w.block_len):
                vis = int(L) + i + 1
                s = K[h // w.group, :vis] @ torch.from_numpy(q[b, i, h]) / math.sqrt(w.head_dim)
                p = torch.softmax(s, dim=0)
                for t in range(vis):
                    ref[t // w.page_size] += p[t]
        np.testing.assert_allclose(S[b], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_draft_full_budget_equals_dense_attention():
    """Selecting every full page makes the sparse draft the dense attention of the
    query at pi = L + j - 1."""
    w, a = _small(lens=(20, 48, 70), gamma=3)
    for j in range(1, w.gamma + 1):
        sel = [np.arange(int(L) // w.page_size) for L in a.ctx_lens]
        o = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
        dense, _ = oracle.dense_verify_attn(a.q_draft[j - 1][:, None], a.k_cache, a.v_cache, a.page_table,
                                            a.ctx_lens + (j - 1))
        np.testing.assert_allclose(o, dense[:, 0], rtol=1e-13, atol=1e-13)


def _attend_explicit(q_row, K, V, scale):
    s = torch.from_numpy(K) @ torch.from_numpy(q_row) * scale
    p = torch.softmax(s, dim=0)
    return (p @ torch.from_numpy(V)).numpy()


@pytest.mark.parametrize("pick", ["empty", "single", "scattered"])
def test_draft_selected_pages_plus_tail_brute_force(pick):
    w, a = _small(lens=(47, 80, 100), gamma=4)
    P = w.page_size
    rng = np.random.default_rng(7)
    sel = []
    for L in a.ctx_lens:
        nf = int(L) // P
        if pick == "empty":
            sel.append(np.array([], dtype=np.int64))
        elif pick == "single":
            sel.append(np.array([rng.integers(nf)]))
        else:
            sel.append(np.sort(rng.choice(nf, size=max(1, nf // 2), replace=False)))
    q = a.q_draft.astype(np.float64)
    for j in (1, 4):
        o = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, j)
        # the same result from the reversed page order (set semantics)
        o_rev = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens,
                                         [s[::-1] for s in sel], j)
        np.testing.assert_allclose(o, o_rev, rtol=1e-13, atol=1e-14)
        for b, L in enumerate(a.ctx_lens):
            n = int(L) + j
            Kd = _dense_seq(a.k_cache, a.page_table[b], n, P, False)
            Vd = _dense_seq(a.v_cache, a.page_table[b], n, P, True)
            keep = np.zeros(n, dtype=bool)
            for p in sel[b]:
                keep[int(p) * P:(int(p) + 1) * P] = True
            keep[(int(L) // P) * P:] = True
            for h in range(w.num_q_heads):
                ref = _attend_explicit(q[j - 1, b, h], Kd[h // w.group][keep], Vd[h // w.group][keep],
                                       1 / math.sqrt(w.head_dim))
                np.testing.assert_allclose(o[b, h], ref, rtol=1e-12, atol=1e-13)


def test_per_head_scores_add_up_to_shared_scores_and_brute_force():
    """Per-kv-head page scores: their sum over kv heads is the shared score, each
    is non-negative with mass G1 * g, and a brute-force recomputation of one head
    agrees."""
    w = W.TINY_FP32.with_(num_seqs=2, num_q_heads=4, num_kv_heads=2, ctx_range=(0, 120), spare_steps=2, gamma=2)
    a = synth.make_attn_inputs(w, 31, ctx_lens=np.array([37, 90]))
    _, shared = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    _, head = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens, per_head=True)
    assert head.shape == (2, 2, shared.shape[1])
    np.testing.assert_allclose(head.sum(axis=1), shared, rtol=0, atol=1e-12)
    assert (head >= 0).all()
    np.testing.assert_allclose(head.sum(axis=2), w.block_len * w.group, rtol=0, atol=1e-12)
    # brute force: sequence 1, kv head 1, token by token
    b, kvh, L = 1, 1, 90
    q = oracle.s3r_oracle._as_f64(a.q_verify)
    brute = np.zeros(shared.shape[1])
    for hh in range(w.group):
        h = kvh * w.group + hh
        for i in range(w.block_len):
            ts = np.arange(L + i + 1)
            K, V = oracle.s3r_oracle._gather_kv(a.k_cache, a.v_cache, a.page_table[b], kvh, ts)
            s = K @ q[b, i, h] / np.sqrt(w.head_dim)
            pr = np.exp(s - s.max())
            pr /= pr.sum()
            for t, x in zip(ts, pr):
                brute[t // 16] += x
    np.testing.assert_allclose(head[b, kvh], brute, rtol=0, atol=1e-12)


def test_per_head_draft_with_equal_selections_is_the_shared_draft():
    w = W.TINY_FP32.with_(num_seqs=2, num_q_heads=4, num_kv_heads=2, ctx_range=(0, 200), spare_steps=2)
    a = synth.make_attn_inputs(w, 32, ctx_lens=np.array([70, 181]))
    sel = [np.array([0, 2]), np.array([1, 3, 7])]
    shared = oracle.sparse_draft_attn(a.q_draft[1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, sel, 2)
    per = oracle.sparse_draft_attn(a.q_draft[1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens,
                                   [[s, s] for s in sel], 2, per_head=True)
    np.testing.assert_array_equal(per, shared)
    # different selections per head change only that head's query heads
    per2 = oracle.sparse_draft_attn(a.q_draft[1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens,
                                    [[sel[0], np.array([4])], [sel[1], sel[1]]], 2, per_head=True)
    np.testing.assert_array_equal(per2[0, :2], shared[0, :2])
    assert not np.allclose(per2[0, 2:], shared[0, 2:])
    np.testing.assert_array_equal(per2[1], shared[1])
