"""Helpers shared by the GPU tests: upload synthetic inputs, read results back,
and the parity rules (per-row relative error for attention outputs; exemption
windows for near-ties in selection, acceptance and sampling)."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def dev(arr: np.ndarray) -> torch.Tensor:
    """numpy -> GPU tensor; uint16 arrays are bf16 bit patterns."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> numpy; bf16 comes back as float64 (exact)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy()


def upload_cache(a):
    from rl_rollout_amd import s3r
    lens = torch.from_numpy(a.ctx_lens.astype(np.int32)).cuda()
    return s3r.KVCache(dev(a.k_cache), dev(a.v_cache), dev(a.page_table.astype(np.int32)), lens)


def max_row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis = head_dim) of ||out - ref||_2 / ||ref||_2."""
    o = out.reshape(-1, out.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.linalg.norm(o - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    return float((num / den).max())


TOL = {"f32": 1e-4, "bf16": 2e-2}


def selection_mismatch_exempt(scores_ref: np.ndarray, n_full: int, k: int, sel_gpu, sel_ref, window=1e-6) -> bool:
    """A selection mismatch is allowed only among pages whose reference score lies
    within `window` of the k-th largest reference score."""
    a, b = set(int(x) for x in sel_gpu), set(int(x) for x in sel_ref)
    if a == b:
        return True
    if len(a) != len(b):
        return False
    s = scores_ref[:n_full]
    kth = np.sort(s)[::-1][k - 1]
    return all(abs(s[p] - kth) < window for p in a.symmetric_difference(b))


def accept_mismatch_exempt(tl, dl, d, ua, us, T, a_gpu, out_gpu, a_ref, out_ref, window=1e-6):
    """Accept parity for one sequence: exact, or the first difference is a near-tie
    (|u - p/q| < window) or a sampled token whose boundary lies within window * R
    of u * R. Returns (ok, exempted)."""
    if a_gpu == a_ref and list(out_gpu) == list(out_ref):
        return True, False
    G1 = tl.shape[0]
    gamma = G1 - 1
    p = [oracle.softmax_row(tl[i], T) for i in range(G1)]
    q = [oracle.softmax_row(dl[j], T) for j in range(gamma)]
    first = min(a_gpu, a_ref)
    if a_gpu != a_ref:
        j = first
        ratio = p[j][d[j]] / q[j][d[j]]
        return abs(float(np.float32(ua[j])) - ratio) < window, True
    # same count: compare the final draw
    j = a_ref
    r = np.maximum(0.0, p[j] - q[j]) if j < gamma else p[gamma]
    R = r.sum()
    c = np.cumsum(r)
    thr = float(np.float32(us)) * R
    x_g, x_o = int(out_gpu[j]), int(out_ref[j])
    lo, hi = min(x_g, x_o), max(x_g, x_o)
    ok = all(abs(c[x] - thr) <= window * R for x in range(lo, hi))
    return ok, True


# ---------------------------------------------------------------- page scores
U32 = 2.0 ** -24   # unit roundoff of fp32
# fp32 roundings on one column's page mass after its logits, counted generously:
# the exp2 of each key, the sum of a page's 16 weights, its log2, the wave and
# split merges of the running sum and maximum, the final exp2 of lse - LSE.
K_CHAIN = 40


def _f64(x):
    x = np.asarray(x)
    return oracle.bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def page_score_rtol(q, k, n_terms, kv_dtype):
    """Relative bound on a GPU page score against the fp64 oracle.

    A page score sums the softmax mass of the page over n_terms columns (block
    query x query head), all positive, in fp32 and in a fixed order. The bound
    has two parts:
      * The logits. s_t = scale * q.k_t accumulates head_dim products in fp32
        (bf16 products are exact in fp32; fp32 products round once more), so its
        error is at most head_dim * u * sum_d |q_d k_d| * scale <= head_dim * u *
        ||q|| ||k|| * scale (Cauchy-Schwarz), in log2 units E = that * log2(e).
        A softmax ratio whose numerator and denominator exponents are each off by
        at most E has relative error at most 2 ln2 E (to first order).
      * The fp32 chain after the logits: the log-domain values (scaled logit,
        page log-sum-exp, column log-sum-exp, their difference) are at most
        Lam = ||q|| ||k|| scale log2(e) in size, and four roundings of them cost
        ln2 * 4 Lam u in relative mass; K_CHAIN more roundings of O(1) values
        per column; then the n_terms - 1 additions of positive terms.
    So |S_gpu - S| <= (2 ln2 E + 4 ln2 Lam u + (K_CHAIN + n_terms - 1) u) S,
    page by page.
    q: the queries attended; k: every key row they may see (any superset)."""
    qf, kf = _f64(q), _f64(k)
    d = qf.shape[-1]
    qn = float(np.sqrt((qf.reshape(-1, d) ** 2).sum(axis=1)).max())
    kn = float(np.sqrt((kf.reshape(-1, d) ** 2).sum(axis=1)).max())
    lam = math.log2(math.e) / math.sqrt(d) * qn * kn
    E = lam * (d + 1) * U32
    ln2 = math.log(2.0)
    return 2.0 * ln2 * E + 4.0 * ln2 * lam * U32 + (K_CHAIN + n_terms - 1) * U32


def check_page_scores(gpu, ref, rtol, what=""):
    """Every page within rtol * S (plus 1e-30, for scores below fp32's range),
    and the observed worst relative error printed for the record."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    big = ref > 1e-6
    obs = float((err[big] / ref[big]).max()) if big.any() else 0.0
    print(f"page scores {what}: max relative error {obs:.2e} over pages with S > 1e-6, bound {rtol:.2e}",
          flush=True)
    bad = err > rtol * ref + 1e-30
    assert not bad.any(), (what, np.argwhere(bad)[:5], gpu[bad][:5], ref[bad][:5])
    return obs
