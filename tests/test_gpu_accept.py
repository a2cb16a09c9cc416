"""GPU parity of s3r_spec_accept against the fp64 oracle (accept counts and
emitted tokens bit-exact outside the near-tie windows), the p == q and one-hot
closed forms, the hand-worked cases, the commit of ctx_lens, and the
distributional exactness of GPU-emitted tokens (chi-square over 1e6 trials
against exact enumeration on a 16-token Markov toy)."""
import json
import os

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from oracle import enumeration
from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import accept_mismatch_exempt, dev, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_small.json")


def _gpu_accept(tl, dl, d, ua, us, T=1.0, ctx=None):
    from rl_rollout_amd import s3r
    ctx_t = dev(ctx.astype(np.int32)) if ctx is not None else None
    a, out = s3r.s3r_spec_accept(dev(tl), dev(dl), dev(d.astype(np.int32)), dev(ua.astype(np.float32)),
                                 dev(us.astype(np.float32)), T, ctx_lens=ctx_t)
    torch.cuda.synchronize()
    return host(a), host(out), (host(ctx_t) if ctx_t is not None else None)


def _parity(tl, dl, d, ua, us, T=1.0):
    a_g, out_g, _ = _gpu_accept(tl, dl, d, ua, us, T)
    a_r, out_r = oracle.spec_accept(tl, dl, d, ua, us, T)
    exempt = 0
    for b in range(tl.shape[0]):
        ok, ex = accept_mismatch_exempt(tl[b], dl[b], d[b], ua[b], us[b], T, a_g[b], out_g[b], a_r[b], out_r[b])
        assert ok, (b, a_g[b], out_g[b], a_r[b], out_r[b])
        exempt += int(ex)
    return a_g, out_g, exempt


def test_hand_worked_cases_on_gpu():
    for case in json.load(open(GOLDEN))["cases"]:
        tl = np.log(np.array(case["p"], dtype=np.float64)).astype(np.float32)[None]
        dl = np.log(np.array(case["q"], dtype=np.float64)).astype(np.float32)[None]
        a, out, _ = _gpu_accept(tl, dl, np.array([case["draft_tokens"]]), np.array([case["u_accept"]]),
                                np.array([case["u_sample"]]))
        assert a[0] == case["num_accepted"], case["name"]
        assert list(out[0]) == case["out_tokens"], case["name"]


def test_tiny_fp32_workload_parity_and_commit():
    w = W.TINY_FP32.with_(num_seqs=64)
    x = synth.make_accept_inputs(w, 0)
    print("accept tiny fp32 B=64 V=512", flush=True)
    a_g, out_g, exempt = _parity(x.target_logits, x.draft_logits, x.draft_tokens, x.u_accept, x.u_sample)
    assert exempt == 0
    ctx = np.arange(64, dtype=np.int32) * 3
    a2, out2, ctx2 = _gpu_accept(x.target_logits, x.draft_logits, x.draft_tokens, x.u_accept, x.u_sample, ctx=ctx)
    np.testing.assert_array_equal(ctx2, ctx + a2 + 1)
    np.testing.assert_array_equal(a2, a_g)


@pytest.mark.parametrize("sigma", [0.3, 0.4985])
def test_bf16_full_vocab_parity(sigma):
    w = W.QWEN3_1P7B_16K
    x = synth.make_accept_inputs(w, 1, num_seqs=12, draft_noise=sigma)
    print(f"accept bf16 V={w.vocab} sigma={sigma} B=12", flush=True)
    a_g, _, exempt = _parity(x.target_logits, x.draft_logits, x.draft_tokens, x.u_accept, x.u_sample)
    assert exempt <= 1


def test_temperature_and_non_multiple_of_8_vocab():
    rng = np.random.default_rng(3)
    B, gamma, V = 16, 3, 1001
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.6, (B, gamma, V))).astype(np.float32)
    d = synth.gumbel_max_tokens(dl, 0.7, rng)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    _parity(tl, dl, d, ua, us, T=0.7)


def test_p_equals_q_accepts_all_on_gpu():
    rng = np.random.default_rng(4)
    B, gamma, V = 32, 4, 3000
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = tl[:, :gamma].copy()
    d = rng.integers(0, V, (B, gamma)).astype(np.int32)
    ua = rng.random((B, gamma), dtype=np.float32)
    ua[0] = np.float32(1.0 - 2 ** -24)
    us = rng.random(B, dtype=np.float32)
    a, out, _ = _gpu_accept(tl, dl, d, ua, us)
    assert (a == gamma).all()
    np.testing.assert_array_equal(out[:, :gamma], d)
    _, out_r = oracle.spec_accept(tl, dl, d, ua, us)
    np.testing.assert_array_equal(out[:, gamma], out_r[:, gamma])


def test_one_hot_draft_on_gpu():
    rng = np.random.default_rng(5)
    B, V, x = 64, 40, 7
    tl = rng.normal(0, 1, (B, 2, V)).astype(np.float32)
    dl = np.full((B, 1, V), -1e4, dtype=np.float32)
    dl[:, 0, x] = 0.0
    d = np.full((B, 1), x, dtype=np.int32)
    ua = rng.random((B, 1), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    a, out, _ = _gpu_accept(tl, dl, d, ua, us)
    for b in range(B):
        p = oracle.softmax_row(tl[b, 0], 1.0)
        if abs(float(ua[b, 0]) - p[x]) > 1e-6:
            assert a[b] == (1 if ua[b, 0] < p[x] else 0)
        if a[b] == 0:
            assert out[b, 0] != x


def test_gpu_emitted_tokens_follow_dense_distribution_chi_square():
    """1e6 trials, first token (16 cells) and first two tokens (256 cells)."""
    from test_oracle_accept import chi_square_pooled, markov_step_inputs

    p, q = synth.markov_tables(16, seed=21, alpha=4.0)
    gamma, trials = 2, 1_000_000
    rng = np.random.default_rng(2024)

    def sampler(tl, dl, d, ua, us):
        a, out, _ = _gpu_accept(tl.astype(np.float32), dl.astype(np.float32), d, ua, us)
        return a, out

    prev = np.zeros(trials, dtype=np.int64)
    a, out = sampler(*markov_step_inputs(p, q, prev, gamma, rng))
    first = out[:, 0].astype(np.int64)
    second = out[:, 1].astype(np.int64)
    need = a == 0
    a2, out2 = sampler(*markov_step_inputs(p, q, first[need], gamma, rng))
    second[need] = out2[:, 0]
    exact = enumeration.joint_first_tokens(p, q, 0, gamma, 2)
    s1, d1 = chi_square_pooled(np.bincount(first, minlength=16), exact.sum(axis=1))
    s2, d2 = chi_square_pooled(np.bincount(first * 16 + second, minlength=256), exact.reshape(-1))
    print(f"chi2 first={s1:.1f} (df {d1}) pair={s2:.1f} (df {d2})", flush=True)
    assert s1 < stats.chi2.ppf(0.999, d1)
    assert s2 < stats.chi2.ppf(0.999, d2)


def test_long_block_gamma_70():
    """gamma = 70: the decision tests the drafts 64 at a time, so accepted prefixes
    longer than one wave take a second round."""
    rng = np.random.default_rng(21)
    B, gamma, V = 12, 70, 2000
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.05, (B, gamma, V))).astype(np.float32)
    dl[:4] = tl[:4, :gamma]                  # p == q: every draft kept, then the bonus draw
    d = synth.gumbel_max_tokens(dl, 1.0, rng)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    print(f"accept gamma={gamma} V={V}", flush=True)
    a, out, _ = _parity(tl, dl, d, ua, us)
    assert (a[:4] == gamma).all()
    assert (a[4:] < gamma).any()


def test_large_vocabulary_262147():
    """A 262147-token vocabulary (not a multiple of 8): five row-statistics chunks
    and 65 residual chunks per row, the last one ragged."""
    rng = np.random.default_rng(22)
    B, gamma, V = 6, 4, 262147
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.3, (B, gamma, V))).astype(np.float32)
    d = synth.gumbel_max_tokens(dl, 1.0, rng)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    print(f"accept gamma={gamma} V={V}", flush=True)
    _parity(tl, dl, d, ua, us)


@pytest.mark.parametrize("cpw,V,dtype", [(3, 151936, "bf16"), (8, 151936, "bf16"), (3, 40961, "f32"), (5, 20480, "f32")])
def test_residual_chunk_groups(cpw, V, dtype):
    """Residual workgroups over groups of cpw vocab chunks (the plan's choice on
    large batches, forced here): 38 chunks in groups of 3 (the last group of 2) and
    of 8; a ragged last chunk (V = 40961, not a multiple of 8); 5 chunks in one
    group. Bit-exact with the oracle, as with one chunk per workgroup."""
    rng = np.random.default_rng(40 + cpw)
    B, gamma = 10, 4
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.4, (B, gamma, V))).astype(np.float32)
    dl[:2] = tl[:2, :gamma]  # every draft kept: the bonus draw reads one row
    d = synth.gumbel_max_tokens(dl, 1.0, rng)
    if dtype == "bf16":  # bf16 bit patterns
        tl = synth.f32_to_bf16_bits(tl)
        dl = synth.f32_to_bf16_bits(dl)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    print(f"accept residual groups cpw={cpw} V={V} {dtype}", flush=True)
    old = os.environ.get("S3R_ACCEPT_CPW")
    os.environ["S3R_ACCEPT_CPW"] = str(cpw)
    try:
        a, _, _ = _parity(tl, dl, d, ua, us)
    finally:
        if old is None:
            del os.environ["S3R_ACCEPT_CPW"]
        else:
            os.environ["S3R_ACCEPT_CPW"] = old
    assert (a[:2] == gamma).all()


@pytest.mark.parametrize("dtype,V,T", [("f32", 8192, 1.0), ("bf16", 8192, 0.8), ("f32", 1001, 0.8),
                                       ("bf16", 1001, 1.0)])
def test_masked_logits(dtype, V, T):
    """Rows with -inf logits (tokens masked out upstream): half of the sequences
    keep only each row's 40 largest logits, the other half mask their first 2048
    tokens, so whole load groups, whole waves and a whole row chunk's first rounds
    see only -inf. Masked tokens have probability 0 on both sides. T = 0.8 makes
    the float tail of log2(e)/T negative."""
    rng = np.random.default_rng(23)
    B, gamma = 16, 4
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.4, (B, gamma, V))).astype(np.float32)
    for b in range(0, B, 2):
        for arr in (tl[b], dl[b]):
            for r in range(arr.shape[0]):
                kth = np.sort(arr[r])[-40]
                arr[r][arr[r] < kth] = -np.inf
    head = min(2048, V - 10)
    tl[1::2, :, :head] = -np.inf
    dl[1::2, :, :head] = -np.inf
    d = synth.gumbel_max_tokens(dl, T, rng)
    # a drafted token its own draft row masks (q = 0) that the target keeps: kept
    x0 = int(np.argmax(tl[0, 0]))
    dl[0, 0, x0] = -np.inf
    d[0, 0] = x0
    # a drafted token both rows mask (q = p = 0): rejected, never emitted
    x2 = int(np.flatnonzero(np.isinf(tl[2, 0]) & np.isinf(dl[2, 0]))[0])
    d[2, 0] = x2
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    t_masked = np.isinf(tl)
    if dtype == "bf16":
        tl = synth.f32_to_bf16_bits(tl)
        dl = synth.f32_to_bf16_bits(dl)
    print(f"accept masked logits {dtype} V={V} T={T}", flush=True)
    a, out, _ = _parity(tl, dl, d, ua, us, T=T)
    assert a[0] >= 1 and out[0, 0] == x0
    assert a[2] == 0 and out[2, 0] != x2 and not t_masked[2, 0, out[2, 0]]
    assert (out >= -1).all() and (out < V).all()
    for b in range(B):  # every emitted token is one its target row allows
        for j in range(int(a[b]) + 1):
            assert not t_masked[b, j, out[b, j]], (b, j)
