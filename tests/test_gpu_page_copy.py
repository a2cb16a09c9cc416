"""s3r_pack_pages / s3r_unpack_pages: byte-exact copies of whole pages (K and V
tiles of every kv head) between the paged cache and a staging buffer, checked
against a NumPy gather and scatter of the same blocks; block ids out of range
leave their slot or block untouched; a pack, a move through host memory and an
unpack into other blocks restores every page bit for bit."""
import numpy as np
import pytest
import torch

from rl_rollout_amd import synth
from rl_rollout_amd import workloads as W

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().cpu().view(torch.uint8).numpy()


@pytest.mark.parametrize("case", ["bf16_8kv_d128", "fp32_1kv_d64"])
def test_pack_unpack_exact(case):
    from rl_rollout_amd import s3r
    if case == "bf16_8kv_d128":
        w = W.QWEN3_1P7B_16K.with_(num_seqs=3, ctx_range=(0, 900), spare_steps=2)
    else:
        w = W.TINY_FP32.with_(num_seqs=3)
    a = synth.make_attn_inputs(w, 51, ctx_lens=np.array([100, 500, 250]) if case[0] == "b" else None)
    kv = s3r.KVCache(dev(a.k_cache), dev(a.v_cache), dev(a.page_table.astype(np.int32)),
                     dev(a.ctx_lens.astype(np.int32)))
    nb = a.k_cache.shape[0]
    rng = np.random.default_rng(3)
    blocks = rng.choice(nb, size=min(nb, 37), replace=False).astype(np.int32)
    blocks[5] = -1           # skipped
    blocks[11] = nb          # skipped
    pb = s3r.page_bytes(kv)
    run = pb // 2
    print(f"pack/unpack {case}: {len(blocks)} pages of {pb} bytes", flush=True)
    staging = torch.full((len(blocks), pb), 0xAB, dtype=torch.uint8, device="cuda")
    s3r.s3r_pack_pages(kv, dev(blocks), staging)
    torch.cuda.synchronize()
    st = staging.cpu().numpy()
    kb = a.k_cache.view(np.uint8).reshape(nb, run)
    vb = a.v_cache.view(np.uint8).reshape(nb, run)
    for i, b in enumerate(blocks):
        if 0 <= b < nb:
            np.testing.assert_array_equal(st[i, :run], kb[b])
            np.testing.assert_array_equal(st[i, run:], vb[b])
        else:
            assert (st[i] == 0xAB).all()
    # through host memory and back into other blocks of a second cache
    host = staging.cpu().pin_memory()
    back = host.to("cuda", non_blocking=True)
    k2 = torch.zeros_like(kv.k_cache)
    v2 = torch.zeros_like(kv.v_cache)
    kv2 = s3r.KVCache(k2, v2, kv.page_table, kv.ctx_lens)
    dest = np.roll(np.arange(nb, dtype=np.int32), 7)[: len(blocks)]
    dest[5], dest[11] = -3, nb + 2                      # skipped on the way in too
    s3r.s3r_unpack_pages(kv2, dev(dest), back)
    torch.cuda.synchronize()
    k2b = _bytes(k2).reshape(nb, run)
    v2b = _bytes(v2).reshape(nb, run)
    written = set()
    for i, (src, dst) in enumerate(zip(blocks, dest)):
        if 0 <= src < nb and 0 <= dst < nb:
            np.testing.assert_array_equal(k2b[dst], kb[src])
            np.testing.assert_array_equal(v2b[dst], vb[src])
            written.add(int(dst))
    untouched = [b for b in range(nb) if b not in written]
    assert (k2b[untouched] == 0).all() and (v2b[untouched] == 0).all()
