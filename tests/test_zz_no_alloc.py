"""The allocation-free accept entry point (s3r_spec_accept_no_alloc) against the
workspace entry point (s3r_spec_accept) on the same inputs, bit for bit: two
calls in a row on the static workspace, the second with fewer sequences, a
shorter block and a smaller vocabulary, so its stale contents from the first call
must not leak into the second."""
import numpy as np
import pytest
import torch

from rl_rollout_amd import synth

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _inputs(B, gamma, V, seed, bf16):
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dl = (tl[:, :gamma] + rng.normal(0, 0.4, (B, gamma, V))).astype(np.float32)
    d = synth.gumbel_max_tokens(dl, 1.0, rng)
    ua = rng.random((B, gamma), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    if bf16:
        tl, dl = synth.f32_to_bf16_bits(tl), synth.f32_to_bf16_bits(dl)
    return [dev(x) for x in (tl, dl, d, ua, us)]


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_no_alloc_accept_matches_the_workspace_entry_point(bf16):
    from rl_rollout_amd import s3r
    for B, gamma, V, seed in ((96, 6, 151936, 1), (17, 3, 5003, 2)):
        print(f"no-alloc accept B={B} gamma={gamma} V={V} bf16={bf16}", flush=True)
        tl, dl, d, ua, us = _inputs(B, gamma, V, seed, bf16)
        ctx0 = torch.arange(B, dtype=torch.int32, device="cuda") * 7 + 100
        ctx_a, ctx_b = ctx0.clone(), ctx0.clone()
        a_ref, t_ref = s3r.s3r_spec_accept(tl, dl, d, ua, us, 0.9, ctx_lens=ctx_a)
        acc = torch.full((B,), -5, dtype=torch.int32, device="cuda")
        toks = torch.full((B, gamma + 1), -5, dtype=torch.int32, device="cuda")
        s3r.s3r_spec_accept_no_alloc(tl, dl, d, ua, us, acc, toks, 0.9, ctx_lens=ctx_b)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(acc), host(a_ref))
        np.testing.assert_array_equal(host(toks), host(t_ref))
        np.testing.assert_array_equal(host(ctx_b), host(ctx_a))
        assert (host(ctx_b) == host(ctx0) + host(acc) + 1).all()


def test_no_alloc_accept_rejects_shapes_beyond_its_workspace():
    """More than 4 MiB of workspace (5000 sequences at gamma 8 over 262144 tokens):
    rejected before any launch, outputs untouched."""
    from rl_rollout_amd import s3r
    B, gamma, V = 5000, 8, 262144
    assert s3r.spec_accept_workspace_size(B, gamma, V) > 4 << 20
    f = s3r.raw["s3r_spec_accept_no_alloc"]
    acc = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    st = f(B, gamma, V, 1, 256, 256, 1, 1, 1, 1.0, acc.data_ptr(), 1, None, None)
    torch.cuda.synchronize()
    assert st == 3
    assert (host(acc) == -5).all()
