"""Parity over seeded random shapes: each case draws a kv dtype, head dim, GQA
group, block length, batch, ragged lengths, budget, draft step and accept
vocabulary, and checks verify (outputs and page scores), the selection over the
GPU's own scores (bit-exact: both sides read the same input), the draft over
that selection, and the accept, each against the fp64 oracle. The shapes cover
combinations the targeted tests do not list one by one."""

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import (TOL, accept_mismatch_exempt, check_page_scores, dev, host, max_row_rel_err, page_score_rtol,
                      upload_cache)

pytestmark = pytest.mark.gpu

N_CASES = 64


def _case(i):
    r = np.random.default_rng(1000 + i)
    dtype = ["bf16", "f32"][int(r.integers(0, 2))]
    d = [64, 128][int(r.integers(0, 2))]
    hkv = [1, 2, 4, 8][int(r.integers(0, 4))]
    g = [1, 2, 4, 8][int(r.integers(0, 4))]
    gamma = int(r.integers(1, 8))
    while (gamma + 1) * g > 32:  # the verify's largest block: two 16-column tiles
        gamma -= 1
    B = int(r.integers(1, 10))
    lens = r.integers(0, 2600, size=B)
    lens[r.integers(0, B)] = [0, 15, 16, 17, 4100][int(r.integers(0, 5))] if B > 1 else lens[0]
    budget = [0.05, 0.1, 0.25, 0.5, 1.0][int(r.integers(0, 5))]
    vocab = [64, 1000, 4096, 8200][int(r.integers(0, 4))]
    logits = ["bf16", "f32"][int(r.integers(0, 2))]
    base = W.TINY_FP32 if dtype == "f32" else W.QWEN3_1P7B_16K
    w = base.with_(name=f"random_{i}", num_seqs=B, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, kv_dtype=dtype,
                   gamma=gamma, ctx_range=(0, int(lens.max())), spare_steps=2, budget=budget, vocab=vocab,
                   logits_dtype=logits)
    return w, lens.astype(np.int64), int(r.integers(1, gamma + 1)), r


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    from rl_rollout_amd import s3r

    w, lens, j, r = _case(i)
    G1, Hq, P = w.block_len, w.num_q_heads, w.page_size
    print(f"random case {i}: {w.kv_dtype} d={w.head_dim} hkv={w.num_kv_heads} g={Hq // w.num_kv_heads} "
          f"gamma={w.gamma} B={w.num_seqs} lens={list(lens)} budget={w.budget} draft step {j} V={w.vocab} "
          f"logits={w.logits_dtype}", flush=True)
    a = synth.make_attn_inputs(w, 2000 + i, ctx_lens=lens)
    kv = upload_cache(a)

    out, scores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
    torch.cuda.synchronize()
    ref_o, ref_s = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    assert max_row_rel_err(host(out), ref_o) <= TOL[w.kv_dtype]
    gs = host(scores)
    check_page_scores(gs[:, : ref_s.shape[1]], ref_s, page_score_rtol(a.q_verify, a.k_cache, G1 * Hq, w.kv_dtype),
                      f"random case {i}")

    # selection over the GPU's scores on both sides: bit-exact
    max_pages = gs.shape[1]
    max_sel = max(1, oracle.num_selected(max_pages, w.budget))
    sel_t, ns_t = s3r.s3r_select_budget(scores, kv.ctx_lens, w.budget, max_sel)
    torch.cuda.synchronize()
    ref_sel = oracle.select_budget(gs.astype(np.float64), lens, P, w.budget)
    ns, sel = host(ns_t), host(sel_t)
    for b in range(w.num_seqs):
        assert ns[b] == len(ref_sel[b]), (b, ns[b], len(ref_sel[b]))
        assert list(sel[b, : ns[b]]) == list(ref_sel[b]), b
        assert (sel[b, ns[b]:] == -1).all()

    # draft step j over that selection (cache mode: the cache already holds the rows up to the query)
    dout = s3r.s3r_sparse_draft_attn(kv, dev(a.q_draft[j - 1]), sel_t, ns_t, j)
    torch.cuda.synchronize()
    ref_d = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, ref_sel, j)
    assert max_row_rel_err(host(dout), ref_d) <= TOL[w.kv_dtype]

    # accept over a vocabulary of the case's size
    x = synth.make_accept_inputs(w, 3000 + i)
    T = [1.0, 0.7][int(r.integers(0, 2))]
    na, toks = s3r.s3r_spec_accept(dev(x.target_logits), dev(x.draft_logits), dev(x.draft_tokens.astype(np.int32)),
                                   dev(x.u_accept), dev(x.u_sample), T)
    torch.cuda.synchronize()
    a_ref, out_ref = oracle.spec_accept(x.target_logits, x.draft_logits, x.draft_tokens, x.u_accept, x.u_sample, T)
    a_gpu, out_gpu = host(na), host(toks)
    for b in range(w.num_seqs):
        ok, _ = accept_mismatch_exempt(x.target_logits[b], x.draft_logits[b], x.draft_tokens[b], x.u_accept[b],
                                       x.u_sample[b], T, a_gpu[b], out_gpu[b], a_ref[b], out_ref[b])
        assert ok, (b, a_gpu[b], out_gpu[b], a_ref[b], out_ref[b])


N_STAGED = 16


def _staged_case(i):
    r = np.random.default_rng(5000 + i)
    dtype = ["bf16", "bf16", "f32"][int(r.integers(0, 3))]
    d = [64, 128][int(r.integers(0, 2))]
    hkv = [1, 2, 4][int(r.integers(0, 3))]
    g = [1, 2, 4, 8][int(r.integers(0, 4))]
    gamma = int(r.integers(1, 8))
    while (gamma + 1) * g > 32:
        gamma -= 1
    B = int(r.integers(1, 5))
    lens = r.integers(4000, 30000, size=B)
    base = W.TINY_FP32 if dtype == "f32" else W.QWEN3_1P7B_16K
    w = base.with_(name=f"random_staged_{i}", num_seqs=B, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                   kv_dtype=dtype, gamma=gamma, ctx_range=(0, int(lens.max())), spare_steps=2)
    return w, lens.astype(np.int64)


@pytest.mark.parametrize("i", range(N_STAGED))
def test_random_shape_staged_verify(i):
    """Whole-unit verify with the per-page staging in the workspace (forced), over
    histories of 4K-30K tokens: 250-1875 pages, so zero to three 512-page chunks
    leave the chip and, with bf16 KV, the chunk before the last is kept in the
    waves' registers. Outputs and page scores against the oracle, and the scores
    of every sequence sum to G1 * Hq."""
    import os

    from rl_rollout_amd import s3r

    w, lens = _staged_case(i)
    G1, Hq, P = w.block_len, w.num_q_heads, w.page_size
    pages = [int(-(-(int(L) + G1) // P)) for L in lens]
    print(f"staged random case {i}: {w.kv_dtype} d={w.head_dim} hkv={w.num_kv_heads} g={Hq // w.num_kv_heads} "
          f"gamma={w.gamma} lens={list(lens)} pages={pages}", flush=True)
    a = synth.make_attn_inputs(w, 6000 + i, ctx_lens=lens)
    kv = upload_cache(a)
    old = os.environ.get("S3R_VERIFY_MODE")
    os.environ["S3R_VERIFY_MODE"] = "global"
    try:
        out, scores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["S3R_VERIFY_MODE"]
        else:
            os.environ["S3R_VERIFY_MODE"] = old
    ref_o, ref_s = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    assert max_row_rel_err(host(out), ref_o) <= TOL[w.kv_dtype]
    gs = host(scores)
    check_page_scores(gs[:, : ref_s.shape[1]], ref_s, page_score_rtol(a.q_verify, a.k_cache, G1 * Hq, w.kv_dtype),
                      f"staged random case {i}")
    for b, n in enumerate(pages):
        assert (gs[b, n:] == 0).all()
        assert abs(float(gs[b].astype(np.float64).sum()) - G1 * Hq) <= 1e-4 * G1 * Hq, b
