"""Plain float64 CPU oracle for the S3R decode hot path.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark import this module. The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path: it
reads the same input arrays and nothing else.

Sources. The method is Self-Sparse Speculative Rollouts (S3R), arXiv 2610.13202,
as described on five web pages:
  * the abstract ("S^3R: Fast and Faithful RL Rollouts via Self-Sparse
    Speculative Decoding", paperdot.bitmofang.com and space-kitty.com);
  * wispaper.ai, sections "S3R drafts sparsely and verifies densely",
    "Dense verification still pays the full KV-cache bill" and
    "Where the speedup claim holds";
  * rebasdaily.com, sections "草稿可以稀疏，交卷必须完整" (the draft may be sparse,
    the submission must be complete) and "真正难搬的，还是那叠完整笔记";
  * rit.work, section "Как разреженный черновик сохраняет ответы плотной модели".
The pages state the method in prose only. Where they leave a step open, the
reading taken is written next to the function that takes it.

Everything is computed in float64 from the exact input values (bf16 and fp32
inputs are exactly representable in float64). Loops are per sequence and per
head, with explicit masks, so that each function can be checked by eye.

Data layout of the paged KV cache (the layout the library also uses):
  k_cache[num_blocks][num_kv_heads][page_size][head_dim]
  v_cache[num_blocks][num_kv_heads][head_dim][page_size]   (page-transposed V)
  page_table[num_seqs][max_pages]   logical page -> physical block
Token t of sequence b lives in block page_table[b][t // P], slot t % P.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 values stored as uint16 bit patterns into float64 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(F64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(F64)


def _gather_kv(k_cache, v_cache, table_row, kvh, positions):
    """K[t], V[t] (float64 rows of length head_dim) for the given token positions."""
    P = k_cache.shape[2]
    pos = np.asarray(positions, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[pos // P]
    slots = pos % P
    K = _as_f64(k_cache[blocks, kvh, slots, :])
    V = _as_f64(v_cache[blocks, kvh, :, slots])
    return K, V


def _softmax_attend(q_row, K, V, scale):
    """Softmax attention of one query over the rows of K/V, all in float64.

    Returns (output, probabilities). s_t = scale * <q, K[t]>, P(t) = exp(s_t - m) / Z.
    """
    s = scale * (K @ q_row)
    m = s.max()
    w = np.exp(s - m)
    p = w / w.sum()
    return p @ V, p


def dense_verify_attn(q, k_cache, v_cache, page_table, ctx_lens, scale=None, per_head=False, horizons=None):
    """Dense verification attention for a block of G1 = gamma + 1 queries, and the
    attention-score summary used for the next draft's selection.

    Dense verification attends the whole committed history (abstract; wispaper.ai,
    "Dense verification still pays the full KV-cache bill"; rebasdaily.com,
    "真正难搬的，还是那叠完整笔记"), for the whole block in one pass (rit.work,
    "Как разреженный черновик ...").

    q:          [B][G1][Hq][D]  query i of sequence b sits at position L_b + i;
                the block's own K/V rows are already written at L_b .. L_b + G1 - 1.
    ctx_lens:   [B] committed length L_b.
    Query i attends every t <= L_b + i (causal). GQA: query head h reads kv head
    h // (Hq / Hkv). No bias, soft-cap or window; RoPE is assumed applied upstream.

    Returns (out [B][G1][Hq][D] float64, page_scores [B][max_pages] float64), where
    page_scores[b][p] = sum over i, h and tokens t of page p of softmax_{b,i,h}(t):
    the "summed softmax scores" reading of the pages' attention-score selection
    (rit.work, "Как разреженный черновик ..."). Every query of the block and every
    query head counts; the sum is shared by all kv heads of the sequence. Pages at
    or beyond ceil((L_b + G1) / P) score 0.

    per_head=True returns page_scores [B][Hkv][max_pages] instead: the same sum
    restricted to the query heads of each kv head (for a page selection per kv
    head; the pages name context selection as future work, wispaper.ai, "What to
    watch before adopting S3R"). The per-head scores add up to the shared ones.

    horizons ([B] ints, optional): a draft horizon gamma_b per sequence, for the
    adaptive horizon the pages leave as future work (wispaper.ai, "Acceptance falls
    at later draft positions"). Sequence b's block is then its queries
    i <= gamma_b (clamped to 0 .. G1 - 1); later rows of out are zero and add
    nothing to the page scores. Reading: only the block's drafted positions and
    the one after them are verified, so only their queries summarise attention.
    """
    q = _as_f64(q)
    B, G1, Hq, D = q.shape
    Hkv, P = k_cache.shape[1], k_cache.shape[2]
    g = Hq // Hkv
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = F64(scale)
    out = np.zeros((B, G1, Hq, D), dtype=F64)
    scores = np.zeros((B, Hkv, max_pages), dtype=F64)
    for b in range(B):
        L = int(ctx_lens[b])
        assert L + G1 <= max_pages * P, "block does not fit in the page table"
        block = G1 if horizons is None else min(max(int(horizons[b]), 0), G1 - 1) + 1
        for kvh in range(Hkv):
            K, V = _gather_kv(k_cache, v_cache, page_table[b], kvh, np.arange(L + G1))
            for hh in range(g):
                h = kvh * g + hh
                for i in range(block):
                    visible = L + i + 1
                    o, p = _softmax_attend(q[b, i, h], K[:visible], V[:visible], scale)
                    out[b, i, h] = o
                    pages_of_t = np.arange(visible) // P
                    scores[b, kvh] += np.bincount(pages_of_t, weights=p, minlength=max_pages)
    if per_head:
        return out, scores
    return out, scores.sum(axis=1)


def num_selected(n_full: int, budget) -> int:
    """Pages kept by the sparse budget s over n_full candidate pages.

    The pages give the budget as a ratio s of the history (wispaper.ai,
    "Throughput gains with comparable task performance": s = 0.05; rebasdaily.com,
    "为什么值得关注": sweep 0.05 .. 0.50) without a rounding rule. Reading: round up,
    with a 1e-9 guard against products like 0.1 * 1000 landing just above an
    integer, computed in float64 (s is a float64 value); at least one page when
    any full page exists, never more than n_full.
    """
    if n_full <= 0:
        return 0
    s = F64(budget)
    k = math.ceil(s * F64(n_full) - 1e-9)
    return int(min(n_full, max(1, k)))


def select_budget(page_scores, ctx_lens, page_size, budget):
    """Score-selected budget of history pages for the next draft.

    After verification the attention scores pick the history the next draft reads
    (rit.work, "Как разреженный черновик ..."), at a small selection cost
    (wispaper.ai, "Where the speedup claim holds").

    Candidates are the full pages of the committed history, p < floor(L_b / P); the
    partial last page is always read by the draft (as its tail) and is never a
    candidate. The top num_selected(n_full, s) candidates by (score descending,
    page index ascending) are kept and returned in ascending page order.
    budget: one ratio s for every row, or a sequence of one ratio per row (the
    adaptive per-sequence budgets the pages leave as future work; wispaper.ai,
    "What to watch before adopting S3R"), each a float64 value rounded by the
    same rule as the scalar budget.
    Returns a list of int64 arrays, one per sequence.
    """
    S = _as_f64(page_scores)
    per_row = np.ndim(budget) > 0
    out = []
    for b in range(S.shape[0]):
        n_full = int(ctx_lens[b]) // int(page_size)
        k = num_selected(n_full, budget[b] if per_row else budget)
        order = sorted(range(n_full), key=lambda p: (-S[b, p], p))
        out.append(np.array(sorted(order[:k]), dtype=np.int64))
    return out


def sparse_draft_attn(q, k_cache, v_cache, page_table, ctx_lens, selected, draft_step, scale=None,
                      per_head=False):
    """Sparse self-draft attention for draft step j (1-based).

    The policy itself drafts, with the same parameters as the verifier, reading
    only part of its KV history (abstract; wispaper.ai, "S3R drafts sparsely and
    verifies densely"; rebasdaily.com, "草稿可以稀疏，交卷必须完整").

    q: [B][Hq][D], the query of the token at position pi = L_b + j - 1 (its K/V row
    already written). The attended set is the selected full pages plus the tail
    {P*floor(L_b/P) <= t <= pi}; the softmax is renormalised over that set.
    per_head=True: selected[b][kvh] is the page list of kv head kvh (its query
    heads attend those pages plus the tail).
    Returns out [B][Hq][D] float64.
    """
    q = _as_f64(q)
    B, Hq, D = q.shape
    Hkv, P = k_cache.shape[1], k_cache.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = F64(scale)
    j = int(draft_step)
    out = np.zeros((B, Hq, D), dtype=F64)
    for b in range(B):
        L = int(ctx_lens[b])
        pi = L + j - 1
        tau = P * (L // P)
        for kvh in range(Hkv):
            pages = selected[b][kvh] if per_head else selected[b]
            attended = [t for p in pages for t in range(int(p) * P, int(p) * P + P)]
            attended += list(range(tau, pi + 1))
            K, V = _gather_kv(k_cache, v_cache, page_table[b], kvh, attended)
            for hh in range(g):
                h = kvh * g + hh
                out[b, h], _ = _softmax_attend(q[b, h], K, V, scale)
    return out


def softmax_row(logits_row, temperature) -> np.ndarray:
    """softmax(logits / T) in float64."""
    x = _as_f64(logits_row) / F64(np.float32(temperature))
    w = np.exp(x - x.max())
    return w / w.sum()


def inverse_cdf(w: np.ndarray, u) -> int:
    """Smallest index x with sum_{y <= x} w_y > u * sum(w), in vocabulary order.

    If rounding leaves no such index, the largest index with w_x > 0.
    """
    W = w.sum()
    c = np.cumsum(w)
    hit = np.nonzero(c > F64(u) * W)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def spec_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature=1.0, horizons=None):
    """Exact speculative sampling over one drafted block per sequence.

    Each draft token is accepted with probability min(1, p/q); at the first
    rejection one corrected token is drawn from the normalised residual
    max(0, p - q) and the block ends (rebasdaily.com, "草稿可以稀疏，交卷必须完整";
    rit.work, "Как разреженный черновик ..."). The emitted tokens then follow the
    dense policy (abstract).

    target_logits: [B][G1][V]   row i gives p_i, the dense distribution of the token
                                after block position i.
    draft_logits:  [B][gamma][V] row j gives q_j, the draft distribution d_j came from.
    draft_tokens:  [B][gamma]
    u_accept:      [B][gamma] uniforms in [0, 1), one per acceptance test
    u_sample:      [B] uniform in [0, 1), the one final (residual or bonus) draw
    Readings: accept iff u * q(x) < p(x), the same test as u < p(x)/q(x) for q(x) > 0;
    with q(x) = 0 (the draft row masks its own token) the draft is kept exactly when
    p(x) > 0, so no token the target gives no mass is ever emitted; when every draft
    is accepted, the extra token is drawn from p_gamma (the bonus); the residual
    draw uses inverse_cdf in vocabulary order; a residual with zero mass (possible
    only through rounding) falls back to p_j.

    horizons ([B] ints, optional): a draft horizon gamma_b per sequence (the
    adaptive horizon the pages leave as future work; wispaper.ai, "Acceptance
    falls at later draft positions"), clamped to 0 .. gamma. Sequence b's block is
    then speculative sampling with its first gamma_b drafts: rows past them are not
    read, and the bonus comes from p_{gamma_b}.

    Returns (num_accepted [B] int64, out_tokens [B][G1] int64 padded with -1).
    """
    T = np.asarray(target_logits)
    Dl = np.asarray(draft_logits)
    B, G1, V = T.shape
    num_acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, G1), -1, dtype=np.int64)
    for b in range(B):
        gamma = G1 - 1 if horizons is None else min(max(int(horizons[b]), 0), G1 - 1)
        p = [softmax_row(T[b, i], temperature) for i in range(gamma + 1)]
        q = [softmax_row(Dl[b, j], temperature) for j in range(gamma)]
        a = 0
        final = None
        for j in range(gamma):
            x = int(draft_tokens[b, j])
            u = F64(np.float32(u_accept[b, j]))
            if u * q[j][x] < p[j][x]:
                out[b, a] = x
                a += 1
                continue
            r = np.maximum(0.0, p[j] - q[j])
            if r.sum() <= 0.0:
                r = p[j]
            final = inverse_cdf(r, np.float32(u_sample[b]))
            break
        if final is None:
            final = inverse_cdf(p[gamma], np.float32(u_sample[b]))
        out[b, a] = final
        num_acc[b] = a
    return num_acc, out


def commit(ctx_lens, num_accepted):
    """Committed length after a step: L_b + a_b + 1 (the accepted drafts plus the
    corrected or bonus token, whose K/V the next step writes)."""
    return np.asarray(ctx_lens, dtype=np.int64) + np.asarray(num_accepted, dtype=np.int64) + 1
