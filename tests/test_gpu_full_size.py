"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (rl_rollout_amd.step.DecodeStep over device-generated inputs).

The oracle cannot run a whole 16K-24K context batch in seconds, so it checks
sampled outputs one sequence at a time: for sampled (layer, sequence) pairs the
sequence's pages are copied to the host and the oracle recomputes, from the
inputs alone,
  * the seeding verify (block at L - G1 .. L - 1): outputs and page scores;
  * the budget selection over those scores (exact, up to near-ties);
  * each of the gamma draft steps, with the oracle's own selection and the draft
    rows the step appended;
  * the step's verify (after the block rows are appended): outputs and scores;
  * the selection for the next step, over the oracle's scores and the oracle's
    committed length;
and, for up to 64 sequences, the accept counts and emitted tokens over the full
vocabulary, plus the commit of ctx_lens for every sequence.

Every sequence (not only the sampled ones) is also held to what must hold at any
size:
  * its page scores add up to G1 * Hq (each of the block's softmax rows sums to
    one), are finite and non-negative, and are zero past its visible pages
    (every layer);
  * its selection is the top n_sel pages of those scores by (score desc, page
    asc), emitted ascending, with n_sel the budget's count (every layer); the
    selection is unique, so this is the oracle's selection over the same scores;
  * every draft and verify output element lies between the smallest and largest
    value its kv head's attended V rows hold in that dim, since attention
    averages them with non-negative weights (the checked layers);
  * its accept keeps a prefix of its drafts, emits one token in the vocabulary
    after them and -1 past it.
"""
import math

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
    """Device tensor -> numpy input array (bf16 as uint16 bit patterns)."""
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


class HostSeq:
    """One sequence of one layer on the host: its pages, compacted to blocks 0..n-1."""

    def __init__(self, layer, table_row, n_pages):
        idx = torch.from_numpy(table_row[:n_pages].astype(np.int64)).cuda()
        self.k = _np(layer["k_cache"].index_select(0, idx)).copy()
        self.v = _np(layer["v_cache"].index_select(0, idx)).copy()
        self.table = np.arange(n_pages, dtype=np.int32)[None]

    def write_row(self, pos, k_row, v_row):
        """The append's effect by definition: token pos gets K/V rows [Hkv][D]."""
        self.k[pos // P, :, pos % P, :] = k_row
        self.v[pos // P, :, :, pos % P] = v_row


def _sample_seqs(lens):
    """First, middle and last sequence, the shortest and the longest, and four more
    drawn with a fixed seed."""
    B = len(lens)
    drawn = np.random.default_rng(B).choice(B, size=min(4, B), replace=False)
    return sorted({0, B // 2, B - 1, int(np.argmin(lens)), int(np.argmax(lens))} | {int(x) for x in drawn})


def _check_scores_all(st, lens_vis, G1, Hq, what):
    """Page scores of every sequence of every layer: sum G1 * Hq, finite, >= 0,
    zero from page ceil((L + G1) / P) on (L = lens_vis, the verify's length)."""
    n_vis = torch.from_numpy((lens_vis.astype(np.int64) + G1 + P - 1) // P).cuda()
    for l, S in enumerate(st.scores):
        assert torch.isfinite(S).all() and (S >= 0).all(), (what, l)
        past = torch.arange(S.shape[1], device=S.device)[None, :] >= n_vis[:, None]
        assert (S[past] == 0).all(), (what, l)
        mass = S.double().sum(dim=1).cpu().numpy()
        bad = np.flatnonzero(np.abs(mass - G1 * Hq) > 1e-4 * G1 * Hq)
        assert bad.size == 0, (what, l, bad[:8], mass[bad[:8]])


def _check_selection_all(st, lens, budgets, what):
    """Selection of every sequence of every layer against its own page scores:
    the count the budget gives, pages ascending and below n_full, -1 past them,
    and the top-n_sel set by (score desc, page asc)."""
    for l in range(len(st.scores)):
        S = host(st.scores[l])
        sel, ns = host(st.sel[l]), host(st.nsel[l])
        for b in range(len(lens)):
            n_full = int(lens[b]) // P
            k = oracle.num_selected(n_full, budgets[b])
            assert ns[b] == k, (what, l, b, ns[b], k)
            pages = sel[b, :k].astype(np.int64)
            assert (sel[b, k:] == -1).all(), (what, l, b)
            assert ((pages >= 0) & (pages < n_full)).all() and (np.diff(pages) > 0).all(), (what, l, b)
            if 0 < k < n_full:
                sc = S[b, :n_full]
                chosen = np.zeros(n_full, dtype=bool)
                chosen[pages] = True
                thr = sc[chosen].min()
                assert sc[~chosen].max() <= thr, (what, l, b)
                tie_in, tie_out = np.flatnonzero(chosen & (sc == thr)), np.flatnonzero(~chosen & (sc == thr))
                if tie_out.size:
                    assert tie_in.max() < tie_out.min(), (what, l, b)


def _v_range(layer, table, n_pages, chunk=16):
    """Per (sequence, kv head, dim): the smallest and largest V value over every
    slot of the sequence's pages below n_pages[b] (a superset of the keys any of
    its attention calls sees there)."""
    vc = layer["v_cache"]  # [blocks][Hkv][D][P]
    n_max = int(n_pages.max())
    npg = torch.from_numpy(n_pages.astype(np.int64)).cuda()
    lo, hi = [], []
    for b0 in range(0, table.shape[0], chunk):
        t = table[b0:b0 + chunk, :n_max].long().clamp(min=0)
        v = vc[t].float()  # [c][n_max][Hkv][D][P]
        ok = (torch.arange(n_max, device=v.device)[None, :] < npg[b0:b0 + chunk, None])[:, :, None, None, None]
        lo.append(torch.where(ok, v, torch.inf).amin(dim=(1, 4)))
        hi.append(torch.where(ok, v, -torch.inf).amax(dim=(1, 4)))
        del v, ok
    return torch.cat(lo), torch.cat(hi)  # [B][Hkv][D]


def _check_within(out, lo, hi, what):
    """out [B][..][Hq][D] against per-(sequence, kv head, dim) bounds [B][Hkv][D].
    With bf16 KV the kernels round the softmax weights to bf16 before the PV
    product while the normaliser sums them unrounded, so the weights add up to
    1 +- 2^-9 and the output may pass the range by 2^-9 of its largest |V|."""
    B, Hkv, D = lo.shape
    o = out.float().reshape(B, -1, Hkv, out.shape[-2] // Hkv, D)
    lo_, hi_ = lo[:, None, :, None, :], hi[:, None, :, None, :]
    rel = 2.0 ** -8 if out.dtype == torch.bfloat16 else 1e-5
    tol = rel * torch.maximum(lo_.abs(), hi_.abs())
    bad = ~torch.isfinite(o) | (o < lo_ - tol) | (o > hi_ + tol)
    assert not bad.any(), (what, int(bad.sum()), torch.nonzero(bad)[:4].tolist())


def _check_accept_all(st, dt, a, out, V, gamma):
    """Every sequence: 0 <= a <= gamma, its first a drafts kept, one token of the
    vocabulary after them, -1 past it."""
    assert ((a >= 0) & (a <= gamma)).all()
    for b in range(len(a)):
        k = int(a[b])
        assert (out[b, :k] == dt[b, :k]).all(), b
        assert 0 <= out[b, k] < V, (b, out[b, k])
        assert (out[b, k + 1:] == -1).all(), b


def _run_full_size(w, layers_to_check, seed=11, accept_check=64, draft_rows=None, budget_of_len=None):
    """budget_of_len: lens [B] -> float64 budgets [B], one sparse budget per sequence."""
    from rl_rollout_amd.step import DecodeStep, build_inputs

    G1, gamma = w.block_len, w.gamma
    print(f"full-size {w.name} layers={w.num_layers} budget={w.budget} draft_rows={draft_rows} "
          f"per-sequence budgets={budget_of_len is not None}: generating inputs", flush=True)
    layers, table, ctx, acc, max_pages, nb = build_inputs(w, seed, steps=2)
    lens = ctx.cpu().numpy().astype(np.int64)
    if budget_of_len is None:
        budgets = np.full(len(lens), w.budget)
        st = DecodeStep(layers, table, ctx, acc, gamma, w.budget, w.temperature, draft_rows=draft_rows)
    else:
        budgets = np.asarray(budget_of_len(lens), dtype=np.float64)
        st = DecodeStep(layers, table, ctx, acc, gamma, torch.from_numpy(budgets), w.temperature,
                        draft_rows=draft_rows)
    table_np = table.cpu().numpy()
    seqs = _sample_seqs(lens)
    print(f"full-size {w.name}: seeding verify + select, sampled seqs {seqs}, layers {layers_to_check}", flush=True)
    st.seed_scores()
    torch.cuda.synchronize()
    _check_scores_all(st, np.maximum(lens - G1, 0), G1, w.num_q_heads, "seed scores")
    _check_selection_all(st, lens, budgets, "seed select")
    # V bounds over every page the step reads before its block rows land (the
    # drafts' and the verify's rows are added below)
    n_read = (lens + G1 + P - 1) // P
    vr = {l: _v_range(layers[l], table, n_read) for l in layers_to_check}

    err = {"seed_verify": 0.0, "draft": 0.0, "verify": 0.0, "score_rel": 0.0}
    exempt = {"select": 0, "accept": 0, "draft_skipped": 0}
    state = {}
    for l in layers_to_check:
        lay = layers[l]
        qv, qd = _np(lay["q_verify"]), _np(lay["q_draft"])
        for b in seqs:
            L = int(lens[b])
            hs = HostSeq(lay, table_np[b], math.ceil((L + G1) / P))
            prev = max(L - G1, 0)
            ref_o, ref_s = oracle.dense_verify_attn(qv[b:b + 1], hs.k, hs.v, hs.table, np.array([prev]))
            e = max_row_rel_err(host(st.out_verify[l][b:b + 1]), ref_o)
            assert e <= TOL[w.kv_dtype], ("seed verify", l, b, e)
            err["seed_verify"] = max(err["seed_verify"], e)
            gs = host(st.scores[l][b])
            err["score_rel"] = max(err["score_rel"], check_page_scores(
                gs[: ref_s.shape[1]], ref_s[0], page_score_rtol(qv[b], hs.k, G1 * w.num_q_heads, w.kv_dtype),
                f"seed verify layer {l} seq {b}"))
            ref_sel = oracle.select_budget(ref_s, np.array([L]), P, budgets[b])[0]
            ns = int(host(st.nsel[l][b]))
            gsel = host(st.sel[l][b])[:ns]
            n_full = L // P
            ok = selection_mismatch_exempt(ref_s[0], n_full, len(ref_sel), gsel, ref_sel)
            assert ok and ns == len(ref_sel), ("seed select", l, b, ns, len(ref_sel))
            same = list(gsel) == list(ref_sel)
            exempt["select"] += int(not same)
            state[(l, b)] = (hs, ref_sel if same else None)

    for j in range(1, gamma + 1):
        print(f"full-size {w.name}: draft step {j}", flush=True)
        st.draft_phase(j)
        torch.cuda.synchronize()
        for l in layers_to_check:
            lay = layers[l]
            vd_t = lay["v_draft"][:j, :, 0].float()  # the draft rows up to this step [j][B][Hkv][D]
            _check_within(st.out_draft[l], torch.minimum(vr[l][0], vd_t.amin(0)),
                          torch.maximum(vr[l][1], vd_t.amax(0)), f"draft {j} layer {l} (all sequences)")
            qd = _np(lay["q_draft"][j - 1])
            kd, vd = _np(lay["k_draft"][j - 1]), _np(lay["v_draft"][j - 1])
            for b in seqs:
                hs, sel = state[(l, b)]
                L = int(lens[b])
                hs.write_row(L + j - 1, kd[b, 0], vd[b, 0])
                if sel is None:
                    exempt["draft_skipped"] += 1
                    continue
                ref = oracle.sparse_draft_attn(qd[b:b + 1], hs.k, hs.v, hs.table, np.array([L]), [sel], j)
                e = max_row_rel_err(host(st.out_draft[l][b:b + 1]), ref)
                assert e <= TOL[w.kv_dtype], ("draft", j, l, b, e)
                err["draft"] = max(err["draft"], e)

    print(f"full-size {w.name}: verify", flush=True)
    st.verify_phase()
    torch.cuda.synchronize()
    _check_scores_all(st, lens, G1, w.num_q_heads, "step scores")
    for l in layers_to_check:
        vb_t = layers[l]["v_block"][:, :G1].float()  # [B][G1][Hkv][D]
        _check_within(st.out_verify[l], torch.minimum(vr[l][0], vb_t.amin(1)), torch.maximum(vr[l][1], vb_t.amax(1)),
                      f"verify layer {l} (all sequences)")
    ref_scores = {}
    for l in layers_to_check:
        lay = layers[l]
        qv = _np(lay["q_verify"])
        kb, vb = _np(lay["k_block"]), _np(lay["v_block"])
        for b in seqs:
            hs, _ = state[(l, b)]
            L = int(lens[b])
            for i in range(G1):
                hs.write_row(L + i, kb[b, i], vb[b, i])
            ref_o, ref_s = oracle.dense_verify_attn(qv[b:b + 1], hs.k, hs.v, hs.table, np.array([L]))
            e = max_row_rel_err(host(st.out_verify[l][b:b + 1]), ref_o)
            assert e <= TOL[w.kv_dtype], ("verify", l, b, e)
            err["verify"] = max(err["verify"], e)
            gs = host(st.scores[l][b])
            err["score_rel"] = max(err["score_rel"], check_page_scores(
                gs[: ref_s.shape[1]], ref_s[0], page_score_rtol(qv[b], hs.k, G1 * w.num_q_heads, w.kv_dtype),
                f"verify layer {l} seq {b}"))
            assert (gs[ref_s.shape[1]:] == 0).all()
            ref_scores[(l, b)] = ref_s[0]

    print(f"full-size {w.name}: accept (B={w.num_seqs}, V={w.vocab})", flush=True)
    st.accept_phase(0)
    torch.cuda.synchronize()
    a_gpu = host(st.num_accepted).astype(np.int64)
    out_gpu = host(st.out_tokens)
    new_lens = host(ctx).astype(np.int64)
    np.testing.assert_array_equal(new_lens, lens + a_gpu + 1)
    _check_accept_all(st, host(acc["draft_tokens"]), a_gpu, out_gpu, w.vocab, gamma)
    chk = sorted(set(range(min(accept_check, w.num_seqs))) | set(seqs))
    tl, dl = _np(acc["target_logits"][chk]), _np(acc["draft_logits"][chk])
    dt = host(acc["draft_tokens"][chk])
    ua, us = host(acc["u_accept"][0][chk]), host(acc["u_sample"][0][chk])
    a_ref, out_ref = oracle.spec_accept(tl, dl, dt, ua, us, w.temperature)
    a_ref_of = {}
    for i, b in enumerate(chk):
        ok, ex = accept_mismatch_exempt(tl[i], dl[i], dt[i], ua[i], us[i], w.temperature, a_gpu[b], out_gpu[b],
                                        a_ref[i], out_ref[i])
        assert ok, ("accept", b, a_gpu[b], out_gpu[b], a_ref[i], out_ref[i])
        exempt["accept"] += int(ex)
        a_ref_of[b] = None if ex else int(a_ref[i])

    print(f"full-size {w.name}: select for the next step", flush=True)
    st.select_phase()
    torch.cuda.synchronize()
    _check_selection_all(st, new_lens, budgets, "next select")
    for l in layers_to_check:
        for b in seqs:
            if a_ref_of.get(b) is None:
                continue
            L_new = int(oracle.commit(np.array([lens[b]]), np.array([a_ref_of[b]]))[0])
            s_ref = ref_scores[(l, b)]
            pad = np.zeros(max(s_ref.shape[0], L_new // P + 1))
            pad[: s_ref.shape[0]] = s_ref
            ref_sel = oracle.select_budget(pad[None], np.array([L_new]), P, budgets[b])[0]
            ns = int(host(st.nsel[l][b]))
            gsel = host(st.sel[l][b])[:ns]
            assert ns == len(ref_sel), ("select", l, b, ns, len(ref_sel))
            assert selection_mismatch_exempt(pad, L_new // P, len(ref_sel), gsel, ref_sel), ("select", l, b)
            exempt["select"] += int(list(gsel) != list(ref_sel))
    print(f"full-size {w.name}: max row errors {err}, exemptions {exempt}", flush=True)
    del layers, table, ctx, acc, st, vr
    torch.cuda.empty_cache()
    return err, exempt


@pytest.mark.parametrize("draft_rows", [True, False], ids=["draft_rows", "draft_appends"])
def test_full_size_qwen3_1p7b_ctx16k(draft_rows):
    """The chained step with the drafts reading the in-flight rows from the draft-row
    buffers (the default) and with an append launch before each draft."""
    err, ex = _run_full_size(W.QWEN3_1P7B_16K, [0], draft_rows=draft_rows)
    assert ex["draft_skipped"] == 0


def test_full_size_qwen3_8b_ctx24k_two_column_tiles():
    _run_full_size(W.QWEN3_8B_24K, [0])


@pytest.mark.parametrize("k", [0, 1, 2, 3], ids=["s0.05", "s0.10", "s0.25", "s0.50"])
def test_full_size_ragged_budget_sweep(k):
    w = W.RAGGED_SWEEP
    _run_full_size(w.with_(budget=w.budgets[k], draft_noise=w.sweep_noise[k]), [0], accept_check=32)


def test_full_size_ragged_budget_per_sequence():
    """One budget per sequence, larger for shorter sequences (the shape of the
    per-sequence allocation): the step's selections hold each sequence's own
    budget, and the drafts read them."""
    w = W.RAGGED_SWEEP

    def budget_of_len(lens):
        return np.select([lens < 4096, lens < 8192, lens < 12288], [0.5, 0.25, 0.1], 0.05)

    _run_full_size(w, [0], accept_check=32, budget_of_len=budget_of_len)


def test_full_size_28_layer_step():
    w = W.FULL_STEP_28L
    _run_full_size(w, [0, w.num_layers - 1], accept_check=32)


def test_step_at_a_shorter_horizon():
    """A step run at draft horizon 3 of a horizon-6 workload (the adaptive
    controller's case): the verify block is the first 4 queries and rows, the
    accept reads the first 4 target rows, 3 draft rows and uniforms."""
    from rl_rollout_amd.step import DecodeStep, build_inputs

    w = W.QWEN3_1P7B_16K_POSITIONS.with_(num_seqs=8, ctx_range=(1000, 3000))
    g = 3
    layers, table, ctx, acc, max_pages, nb = build_inputs(w, 21, steps=2)
    st = DecodeStep(layers, table, ctx, acc, w.gamma, w.budget, w.temperature)
    lens = ctx.cpu().numpy().astype(np.int64)
    table_np = table.cpu().numpy()
    print(f"horizon {g} of {w.gamma}: lens {list(lens)}", flush=True)
    st.seed_scores()
    for j in range(1, g + 1):
        st.draft_phase(j)
    st.verify_phase(g)
    st.accept_phase(0, g)
    torch.cuda.synchronize()
    lay = layers[0]
    h = st.horizon(g)
    qv = _np(lay["q_verify"])[:, : g + 1]
    kb, vb = _np(lay["k_block"]), _np(lay["v_block"])
    for b in (0, 5):
        L = int(lens[b])
        hs = HostSeq(lay, table_np[b], math.ceil((L + g + 1) / P))
        for i in range(g + 1):
            hs.write_row(L + i, kb[b, i], vb[b, i])
        ref_o, ref_s = oracle.dense_verify_attn(qv[b:b + 1], hs.k, hs.v, hs.table, np.array([L]))
        assert max_row_rel_err(host(h["out_verify"][0][b:b + 1]), ref_o) <= TOL[w.kv_dtype]
        check_page_scores(host(st.scores[0][b])[: ref_s.shape[1]], ref_s[0],
                          page_score_rtol(qv[b], hs.k, (g + 1) * w.num_q_heads, w.kv_dtype), f"horizon {g} seq {b}")
    tl = _np(acc["target_logits"])[:, : g + 1]
    dl = _np(acc["draft_logits"])[:, :g]
    dt = host(acc["draft_tokens"])[:, :g]
    ua, us = host(acc["u_accept"][0])[:, :g], host(acc["u_sample"][0])
    a_ref, out_ref = oracle.spec_accept(tl, dl, dt, ua, us, w.temperature)
    a_gpu, out_gpu = host(st.num_accepted), host(h["out_tokens"])
    for b in range(w.num_seqs):
        ok, _ = accept_mismatch_exempt(tl[b], dl[b], dt[b], ua[b], us[b], w.temperature, a_gpu[b], out_gpu[b],
                                       a_ref[b], out_ref[b])
        assert ok, (b, a_gpu[b], out_gpu[b], a_ref[b], out_ref[b])
    np.testing.assert_array_equal(host(ctx).astype(np.int64), lens + a_gpu + 1)


def test_step_with_page_sets_per_kv_head():
    """The step runtime in per-kv-head selection mode: seeding verify with
    per-head scores, selection over sequence x kv-head rows, and a draft step with
    each head's own pages, against the oracle's per-head scores, selections and
    draft."""
    from rl_rollout_amd.step import DecodeStep, build_inputs

    w = W.QWEN3_1P7B_16K.with_(num_seqs=4, ctx_range=(1000, 3000), budget=0.1)
    layers, table, ctx, acc, max_pages, nb = build_inputs(w, 23, steps=2)
    st = DecodeStep(layers, table, ctx, acc, w.gamma, w.budget, w.temperature, per_head_selection=True)
    lens = ctx.cpu().numpy().astype(np.int64)
    table_np = table.cpu().numpy()
    print(f"per-head selection step: lens {list(lens)}", flush=True)
    st.seed_scores()
    st.draft_phase(1)
    torch.cuda.synchronize()
    lay = layers[0]
    G1, H = w.block_len, w.num_kv_heads
    qv, qd = _np(lay["q_verify"]), _np(lay["q_draft"][0])
    kd, vd = _np(lay["k_draft"][0]), _np(lay["v_draft"][0])
    for b in range(w.num_seqs):
        L = int(lens[b])
        hs = HostSeq(lay, table_np[b], math.ceil((L + G1) / P))
        _, ref_h = oracle.dense_verify_attn(qv[b:b + 1], hs.k, hs.v, hs.table, np.array([max(L - G1, 0)]),
                                            per_head=True)
        gh = host(st.scores[0][b])
        check_page_scores(gh[:, : ref_h.shape[2]], ref_h[0],
                          page_score_rtol(qv[b], hs.k, G1 * (w.num_q_heads // H), w.kv_dtype), f"per-head seq {b}")
        ref_sel = oracle.select_budget(ref_h[0], np.full(H, L), P, w.budget)
        sels = []
        for h in range(H):
            ns = int(host(st.nsel[0][b, h]))
            g = host(st.sel[0][b, h])[:ns]
            assert ns == len(ref_sel[h])
            assert selection_mismatch_exempt(ref_h[0, h], L // P, len(ref_sel[h]), g, ref_sel[h])
            sels.append(ref_sel[h] if list(g) == list(ref_sel[h]) else None)
        if any(x is None for x in sels):
            continue
        hs.write_row(L, kd[b, 0], vd[b, 0])
        ref = oracle.sparse_draft_attn(qd[b:b + 1], hs.k, hs.v, hs.table, np.array([L]), [sels], 1, per_head=True)
        assert max_row_rel_err(host(st.out_draft[0][b:b + 1]), ref) <= TOL[w.kv_dtype]
