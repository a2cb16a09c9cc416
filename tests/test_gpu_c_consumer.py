"""A plain C program (tests/c_consumer/s3r_c_step.c, built by rl_rollout_amd.build
with gcc against libs3r.so and the HIP runtime only) runs one step's verify,
selection, one draft step and the accept with its commit on the GPU, with no
Python or torch in its process. Its outputs must match the fp64 oracle to the
usual bars, and equal bit for bit what the Python binding returns for the same
inputs (the same library and the same deterministic kernels)."""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from rl_rollout_amd import s3r, synth
from rl_rollout_amd import workloads as W
from rl_rollout_amd.build import C_CONSUMER_OUT

from gpu_util import TOL, check_page_scores, dev, host, max_row_rel_err, page_score_rtol, upload_cache

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_fp32", W.TINY_FP32, 0, None, 1),
    # bf16 GQA (two query heads per kv head), ragged histories over several pages
    # and partial tails, the full vocabulary, draft step 3
    ("bf16_gqa_ragged", W.QWEN3_1P7B_16K.with_(num_seqs=3, num_q_heads=4, num_kv_heads=2, spare_steps=2,
                                               ctx_range=(0, 3000), budget=0.25), 5,
     np.array([37, 1500, 2990]), 3),
]


def _write(d, name, arr):
    np.ascontiguousarray(arr).tofile(os.path.join(d, name + ".bin"))


def _read(d, name, dtype, shape):
    return np.fromfile(os.path.join(d, name + ".bin"), dtype=dtype).reshape(shape)


@pytest.mark.parametrize("name,w,seed,lens,j", CASES, ids=[c[0] for c in CASES])
def test_c_program_step_matches_the_oracle_and_the_binding(tmp_path, name, w, seed, lens, j):
    if not os.path.exists(C_CONSUMER_OUT):
        pytest.skip(f"{C_CONSUMER_OUT} is not built: run rl_rollout_amd.build.build()")
    a = synth.make_attn_inputs(w, seed, ctx_lens=lens)
    x = synth.make_accept_inputs(w, seed)
    B, G1, Hq, D = a.q_verify.shape
    Hkv = a.k_cache.shape[1]
    NB, maxp = a.k_cache.shape[0], a.page_table.shape[1]
    V = x.target_logits.shape[-1]
    max_sel = oracle.num_selected(maxp, w.budget)
    scale = 1.0 / math.sqrt(D)
    d = str(tmp_path)
    for key, arr in (("k_cache", a.k_cache), ("v_cache", a.v_cache), ("page_table", a.page_table),
                     ("ctx_lens", a.ctx_lens), ("q_verify", a.q_verify), ("q_draft", a.q_draft[j - 1]),
                     ("target_logits", x.target_logits), ("draft_logits", x.draft_logits),
                     ("draft_tokens", x.draft_tokens), ("u_accept", x.u_accept), ("u_sample", x.u_sample)):
        _write(d, key, arr)
    kvd = 1 if a.k_cache.dtype == np.uint16 else 0
    ld = 1 if x.target_logits.dtype == np.uint16 else 0
    meta = dict(B=B, Hq=Hq, Hkv=Hkv, D=D, NB=NB, maxp=maxp, G1=G1, gamma=G1 - 1, V=V, kv_dtype=kvd,
                logits_dtype=ld, max_sel=max_sel, draft_step=j, budget=w.budget, scale=scale,
                temperature=w.temperature)
    with open(os.path.join(d, "meta.txt"), "w") as f:
        for k, v in meta.items():
            f.write(f"{k} {float(v)!r}\n")
    print(f"C caller {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} lens={[int(L) for L in a.ctx_lens]} max_sel={max_sel} j={j} V={V}",
          flush=True)
    r = subprocess.run([C_CONSUMER_OUT, d], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr

    fdt = np.uint16 if kvd else np.float32
    out = _read(d, "verify_out", fdt, (B, G1, Hq, D))
    scores = _read(d, "page_scores", np.float32, (B, maxp))
    sel = _read(d, "sel", np.int32, (B, max_sel))
    nsel = _read(d, "nsel", np.int32, (B,))
    dout = _read(d, "draft_out", fdt, (B, Hq, D))
    nacc = _read(d, "num_accepted", np.int32, (B,))
    toks = _read(d, "out_tokens", np.int32, (B, G1))
    ctx_after = _read(d, "ctx_after", np.int32, (B,))

    # against the oracle
    # bf16 outputs as exact float64 values, as the binding's host() gives them
    val = (lambda t: oracle.bf16_bits_to_f64(t)) if kvd else (lambda t: t)
    ref, ref_scores = oracle.dense_verify_attn(a.q_verify, a.k_cache, a.v_cache, a.page_table, a.ctx_lens)
    assert max_row_rel_err(val(out), ref) <= TOL[w.kv_dtype]
    check_page_scores(scores, ref_scores, page_score_rtol(a.q_verify, a.k_cache, G1 * Hq, w.kv_dtype), name)
    ref_sel = oracle.select_budget(scores.astype(np.float64), a.ctx_lens, w.page_size, w.budget)
    for b in range(B):
        assert nsel[b] == len(ref_sel[b])
        assert list(sel[b, :nsel[b]]) == list(ref_sel[b])
        assert (sel[b, nsel[b]:] == -1).all()
    dref = oracle.sparse_draft_attn(a.q_draft[j - 1], a.k_cache, a.v_cache, a.page_table, a.ctx_lens, ref_sel, j)
    assert max_row_rel_err(val(dout), dref) <= TOL[w.kv_dtype]
    a_ref, t_ref = oracle.spec_accept(x.target_logits, x.draft_logits, x.draft_tokens, x.u_accept, x.u_sample,
                                      w.temperature)
    assert list(nacc) == list(a_ref)
    assert (toks == t_ref).all()
    assert list(ctx_after) == list(a.ctx_lens + nacc + 1)

    # against the Python binding on the same inputs: bit for bit
    kv = upload_cache(a)
    pout, pscores = s3r.s3r_dense_verify_attn(kv, dev(a.q_verify))
    psel, pns = s3r.s3r_select_budget(pscores, kv.ctx_lens, w.budget, max_sel)
    pd = s3r.s3r_sparse_draft_attn(kv, dev(a.q_draft[j - 1]), psel, pns, j)
    ctx = kv.ctx_lens.clone()
    pa, pt = s3r.s3r_spec_accept(dev(x.target_logits), dev(x.draft_logits), dev(x.draft_tokens), dev(x.u_accept),
                                 dev(x.u_sample), w.temperature, ctx_lens=ctx)
    torch.cuda.synchronize()
    for what, c_val, p_val in (("verify", val(out), host(pout)), ("scores", scores, host(pscores)),
                               ("sel", sel, host(psel)), ("nsel", nsel, host(pns)), ("draft", val(dout), host(pd)),
                               ("accepted", nacc, host(pa)), ("tokens", toks, host(pt)),
                               ("ctx", ctx_after, host(ctx))):
        assert c_val.dtype == p_val.dtype and c_val.shape == p_val.shape, what
        assert np.array_equal(c_val, p_val), what
