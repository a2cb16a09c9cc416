"""Parity of a rollout of several decode steps (rl_rollout_amd.step.DecodeStep,
the benchmark's launch configuration) against the fp64 oracle, which carries the
same state from step to step: the committed lengths ctx_lens, the cache rows
(each step's block rows overwrite the rows past the new length), the page scores
of the previous verify and the selection made from them.

Every sequence of every layer is checked at every step: the drafts (over the
oracle's own selection), the verify outputs and page scores, the accept counts
and emitted tokens, the commit, and the next selection. Where the GPU's selection
or accept differs from the oracle's inside the near-tie windows, the oracle
continues from the GPU's choice, which is as valid.
"""

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import workloads as W

from gpu_util import (TOL, accept_mismatch_exempt, check_page_scores, host, max_row_rel_err, page_score_rtol,
                      selection_mismatch_exempt)

pytestmark = pytest.mark.gpu

P = 16


def _np(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


class HostCache:
    """One sequence's pages of one layer on the host, compacted to blocks 0..n-1."""

    def __init__(self, layer, table_row, n_pages):
        idx = torch.from_numpy(table_row[:n_pages].astype(np.int64)).cuda()
        self.k = _np(layer["k_cache"].index_select(0, idx)).copy()
        self.v = _np(layer["v_cache"].index_select(0, idx)).copy()
        self.table = np.arange(n_pages, dtype=np.int32)[None]

    def write_row(self, pos, k_row, v_row):
        self.k[pos // P, :, pos % P, :] = k_row
        self.v[pos // P, :, :, pos % P] = v_row


def _select(scores_row, L, budget, gpu_sel):
    """The oracle's selection at length L, or the GPU's where they differ only
    inside the near-tie window. Returns (pages, exempted)."""
    pad = np.zeros(max(scores_row.shape[0], L // P + 1))
    pad[: scores_row.shape[0]] = scores_row
    ref = oracle.select_budget(pad[None], np.array([L]), P, budget)[0]
    assert len(gpu_sel) == len(ref), (len(gpu_sel), len(ref))
    if list(gpu_sel) == list(ref):
        return list(ref), False
    assert selection_mismatch_exempt(pad, L // P, len(ref), gpu_sel, ref)
    return list(gpu_sel), True


def _rollout(w, steps, seed, horizons=None, budgets=None):
    """horizons: int [B], sequence b drafts horizons[b] tokens each step; budgets:
    float64 [B], one sparse budget per sequence."""
    from rl_rollout_amd.step import DecodeStep, build_inputs

    G1, gamma, Hq = w.block_len, w.gamma, w.num_q_heads
    print(f"rollout {w.name} B={w.num_seqs} layers={w.num_layers} steps={steps} horizons={horizons} "
          f"budgets={budgets}", flush=True)
    layers, table, ctx, acc, max_pages, _ = build_inputs(w, seed, steps=steps)
    budget_arg = w.budget if budgets is None else torch.from_numpy(np.asarray(budgets, dtype=np.float64))
    st = DecodeStep(layers, table, ctx, acc, gamma, budget_arg, w.temperature)
    hz = None if horizons is None else np.asarray(horizons, dtype=np.int64)
    hz_dev = None if hz is None else torch.from_numpy(hz.astype(np.int32)).cuda()
    budget_of = (lambda b: w.budget) if budgets is None else (lambda b: float(budgets[b]))
    table_np = table.cpu().numpy()
    B = w.num_seqs
    lens = host(ctx).astype(np.int64)
    n_alloc = [int((table_np[b] >= 0).sum()) for b in range(B)]
    caches = {(l, b): HostCache(layers[l], table_np[b], n_alloc[b]) for l in range(w.num_layers) for b in range(B)}
    inputs = [{k: _np(layers[l][k]) for k in ("q_verify", "q_draft", "k_draft", "v_draft", "k_block", "v_block")}
              for l in range(w.num_layers)]
    tl, dl = _np(acc["target_logits"]), _np(acc["draft_logits"])
    dt = host(acc["draft_tokens"])

    st.seed_scores()
    torch.cuda.synchronize()
    sel = {}
    exempt = {"select": 0, "accept": 0}
    for l in range(w.num_layers):
        qv = inputs[l]["q_verify"]
        for b in range(B):
            hc = caches[(l, b)]
            prev = max(int(lens[b]) - G1, 0)
            _, ref_s = oracle.dense_verify_attn(qv[b:b + 1], hc.k, hc.v, hc.table, np.array([prev]))
            ns = int(host(st.nsel[l][b]))
            sel[(l, b)], ex = _select(ref_s[0], int(lens[b]), budget_of(b), host(st.sel[l][b])[:ns])
            exempt["select"] += int(ex)

    for s in range(steps):
        print(f"rollout {w.name}: step {s}, lengths {lens.min()}..{lens.max()}", flush=True)
        for j in range(1, gamma + 1):
            st.draft_phase(j, hz_dev)
            torch.cuda.synchronize()
            for l in range(w.num_layers):
                x = inputs[l]
                for b in range(B):
                    if hz is not None and j > hz[b]:
                        continue  # this sequence drafts fewer tokens: skipped
                    hc = caches[(l, b)]
                    L = int(lens[b])
                    hc.write_row(L + j - 1, x["k_draft"][j - 1, b, 0], x["v_draft"][j - 1, b, 0])
                    ref = oracle.sparse_draft_attn(x["q_draft"][j - 1][b:b + 1], hc.k, hc.v, hc.table,
                                                   np.array([L]), [np.array(sel[(l, b)], dtype=np.int64)], j)
                    e = max_row_rel_err(host(st.out_draft[l][b:b + 1]), ref)
                    assert e <= TOL[w.kv_dtype], ("draft", s, j, l, b, e)
        st.verify_phase(None, hz_dev)
        torch.cuda.synchronize()
        scores = {}
        for l in range(w.num_layers):
            x = inputs[l]
            for b in range(B):
                hc = caches[(l, b)]
                L = int(lens[b])
                for i in range(G1):
                    hc.write_row(L + i, x["k_block"][b, i], x["v_block"][b, i])
                hb = None if hz is None else hz[b:b + 1]
                ref_o, ref_s = oracle.dense_verify_attn(x["q_verify"][b:b + 1], hc.k, hc.v, hc.table, np.array([L]),
                                                        horizons=hb)
                e = max_row_rel_err(host(st.out_verify[l][b:b + 1]), ref_o)
                assert e <= TOL[w.kv_dtype], ("verify", s, l, b, e)
                gs = host(st.scores[l][b])
                n_terms = (G1 if hz is None else int(hz[b]) + 1) * Hq
                check_page_scores(gs[: ref_s.shape[1]], ref_s[0],
                                  page_score_rtol(x["q_verify"][b], hc.k, n_terms, w.kv_dtype),
                                  f"step {s} layer {l} seq {b}")
                assert (gs[ref_s.shape[1]:] == 0).all()
                scores[(l, b)] = ref_s[0]
        st.accept_phase(s, None, hz_dev)
        torch.cuda.synchronize()
        a_gpu = host(st.num_accepted).astype(np.int64)
        out_gpu = host(st.out_tokens)
        ua, us = host(acc["u_accept"][s]), host(acc["u_sample"][s])
        a_ref, out_ref = oracle.spec_accept(tl, dl, dt, ua, us, w.temperature, horizons=hz)
        if hz is not None:
            assert (a_gpu <= hz).all()
        for b in range(B):
            if hz is not None:
                # one sequence at its own horizon: its first hz[b] drafts and target rows 0 .. hz[b]
                g = int(hz[b])
                ok, ex = accept_mismatch_exempt(tl[b, : g + 1], dl[b, :g], dt[b, :g], ua[b, :g], us[b],
                                                w.temperature, a_gpu[b], out_gpu[b, : g + 1], a_ref[b],
                                                out_ref[b, : g + 1])
                assert (out_gpu[b, g + 1:] == -1).all()
            else:
                ok, ex = accept_mismatch_exempt(tl[b], dl[b], dt[b], ua[b], us[b], w.temperature, a_gpu[b],
                                                out_gpu[b], a_ref[b], out_ref[b])
            assert ok, ("accept", s, b, a_gpu[b], out_gpu[b], a_ref[b], out_ref[b])
            exempt["accept"] += int(ex)
        # the oracle commits the GPU's count (equal to its own outside the windows)
        new_lens = oracle.commit(lens, a_gpu)
        np.testing.assert_array_equal(host(ctx).astype(np.int64), new_lens)
        lens = new_lens
        st.select_phase()
        torch.cuda.synchronize()
        for l in range(w.num_layers):
            for b in range(B):
                ns = int(host(st.nsel[l][b]))
                sel[(l, b)], ex = _select(scores[(l, b)], int(lens[b]), budget_of(b), host(st.sel[l][b])[:ns])
                exempt["select"] += int(ex)
    print(f"rollout {w.name}: exemptions {exempt}, final lengths {lens.min()}..{lens.max()}", flush=True)
    return lens


@pytest.mark.parametrize("name", ["1.7b_two_layers", "8b_staged", "fp32_g4_d128", "ragged_horizons_and_budgets"])
def test_rollout_of_several_steps(name):
    """Four steps of two 1.7B-like layers (whole-unit verify with LDS staging);
    three steps of the 8B-like heads on 40 sequences of 494..563 pages (320 units:
    whole-unit verify with the staging in the workspace, some units writing one
    512-page chunk out); five steps of fp32 KV and logits with four query heads per
    kv head, d = 128, budget 0.25. Each against the oracle carrying the state."""
    if name == "ragged_horizons_and_budgets":
        w = W.QWEN3_1P7B_16K.with_(num_seqs=8, ctx_range=(200, 2500), spare_steps=5)
        hz = np.array([0, 1, 2, 3, 4, 4, 2, 1])
        budgets = np.array([0.05, 0.1, 0.25, 0.5, 0.05, 0.3, 0.15, 0.5])
        lens = _rollout(w, 4, seed=6, horizons=hz, budgets=budgets)
        assert lens.min() >= w.ctx_range[0] + 4
        return
    if name == "fp32_g4_d128":
        w = W.TINY_FP32.with_(num_seqs=8, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(20, 700),
                              spare_steps=7)
        steps = 5
    elif name == "1.7b_two_layers":
        w = W.QWEN3_1P7B_16K.with_(num_seqs=6, num_layers=2, ctx_range=(40, 1200), spare_steps=6)
        steps = 4
    else:
        w = W.QWEN3_8B_24K.with_(num_seqs=40, ctx_range=(7900, 9000), spare_steps=5)
        steps = 3
    lens = _rollout(w, steps, seed=5)
    assert lens.min() >= w.ctx_range[0] + steps
