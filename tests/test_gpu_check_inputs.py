"""s3r_check_step_inputs: valid step inputs report nothing, and every problem
planted on the host (a length past the page table, a page id out of range, a
count above max_sel, a duplicate or out-of-range selected page, a draft token
outside the vocabulary, a NaN or infinity in a slot read with zero weight) is
reported on its own sequence with the bit that names it. The check only compares the values it reads, so the planted values are never
used as addresses."""
import numpy as np
import pytest
import torch

from rl_rollout_amd import workloads as W

from gpu_util import host

pytestmark = pytest.mark.gpu

LEN, PAGE, NUM_SEL, SEL_RANGE, SEL_DUP, TOKEN, SLOT = 1, 2, 4, 8, 16, 32, 64


def _setup(per_head=False):
    from rl_rollout_amd.step import DecodeStep, build_inputs
    w = W.QWEN3_1P7B_16K.with_(num_seqs=8, ctx_range=(300, 3000), budget=0.1)
    layers, table, ctx, acc, max_pages, nb = build_inputs(w, 29, steps=2)
    st = DecodeStep(layers, table, ctx, acc, w.gamma, w.budget, w.temperature, per_head_selection=per_head)
    st.seed_scores()
    torch.cuda.synchronize()
    return w, st, layers, table, ctx, acc, nb


@pytest.mark.parametrize("per_head", [False, True])
def test_valid_step_inputs_report_nothing(per_head):
    w, st, *_ = _setup(per_head)
    print(f"check inputs: valid, per_head={per_head}", flush=True)
    assert st.check_inputs() == {}


def test_planted_problems_are_reported_on_their_sequence():
    from rl_rollout_amd import s3r
    w, st, layers, table, ctx, acc, nb = _setup()
    lens = host(ctx).astype(np.int64)
    tab, c = table.clone(), ctx.clone()
    sel, ns, tok = st.sel[0].clone(), st.nsel[0].clone(), acc["draft_tokens"].clone()
    maxp = tab.shape[1]
    assert int(ns[4]) >= 2
    c[1] = maxp * 16                              # the block would run past the page table
    tab[2, (int(lens[2]) + 2) // 16] = nb + 5     # a page the block writes
    ns[3] = sel.shape[1] + 1                      # more pages than the selection holds
    sel[4, 1] = sel[4, 0]                         # one page twice
    sel[5, 0] = int(lens[5]) // 16                # the partial last page is not a candidate
    tok[6, 2] = w.vocab                           # outside the vocabulary
    print("check inputs: planted problems on sequences 1..6", flush=True)
    kv = s3r.KVCache(layers[0]["k_cache"], layers[0]["v_cache"], tab, c)
    e = host(s3r.s3r_check_step_inputs(kv, w.block_len, sel, ns, tok, w.vocab))
    assert e[0] == 0 and e[7] == 0
    assert e[1] & LEN
    assert e[2] == PAGE
    # the count is clamped to max_sel, as the drafts clamp it: the row's unused
    # entries (-1) are then read and reported as well
    assert e[3] & NUM_SEL and e[3] & ~(NUM_SEL | SEL_RANGE) == 0
    assert e[4] == SEL_DUP
    assert e[5] == SEL_RANGE
    assert e[6] == TOKEN
    assert s3r.describe_check(torch.from_numpy(e))[4] == ["sel_duplicate"]
    # without the selection and the tokens only the lengths and pages are checked
    e2 = host(s3r.s3r_check_step_inputs(kv, w.block_len))
    assert e2[1] & LEN and e2[2] == PAGE and e2[[0, 3, 4, 5, 6, 7]].sum() == 0


def test_planted_duplicate_in_a_per_kv_head_selection():
    from rl_rollout_amd import s3r
    w, st, layers, table, ctx, acc, nb = _setup(per_head=True)
    sel, ns = st.sel[0].clone(), st.nsel[0].clone()
    assert int(ns[2, 3]) >= 2
    sel[2, 3, 1] = sel[2, 3, 0]
    print("check inputs: per-head duplicate on sequence 2, head 3", flush=True)
    e = host(s3r.s3r_check_step_inputs(st.kv[0], w.block_len, sel, ns))
    assert e[2] == SEL_DUP
    assert np.delete(e, 2).sum() == 0


@pytest.mark.parametrize("cache", ["k", "v"])
def test_nonfinite_slot_read_with_zero_weight_is_reported(cache):
    """A NaN or an infinity in the slots a step reads with zero weight (positions at
    and after L_b of the pages holding the block) is reported; the same value in
    the attended history before L_b, or in a page past the block, is not this
    check's business."""
    from rl_rollout_amd import s3r
    w, st, layers, table, ctx, acc, nb = _setup()
    lens = host(ctx).astype(np.int64)
    tab = host(table)
    k, v = layers[0]["k_cache"].clone(), layers[0]["v_cache"].clone()
    t = k if cache == "k" else v
    D = w.head_dim

    def poison(b, pos, val, head=3, dim=5):
        blk = int(tab[b, pos // 16])
        if cache == "k":
            t[blk, head, pos % 16, dim] = val
        else:
            t[blk, head, dim, pos % 16] = val

    poison(1, int(lens[1]) + 1, float("nan"))                    # inside the block
    poison(2, int(lens[2]) + w.block_len, float("inf"))          # past the block, same page or the next
    last = (int(lens[3]) + w.block_len - 1) // 16 * 16 + 15
    poison(3, last, float("-inf"), head=7, dim=D - 1)            # the last slot of the step's last page
    poison(4, int(lens[4]) - 1, float("nan"))                    # attended history: not reported
    print(f"check inputs: non-finite {cache} slots on sequences 1..4", flush=True)
    kv = s3r.KVCache(k, v, table, ctx)
    e = host(s3r.s3r_check_step_inputs(kv, w.block_len))
    expect = np.zeros(w.num_seqs, dtype=np.int64)
    expect[[1, 2, 3]] = SLOT
    if (int(lens[2]) + w.block_len) // 16 > (int(lens[2]) + w.block_len - 1) // 16:
        expect[2] = 0      # the poisoned position opened a page the step does not read
    np.testing.assert_array_equal(e, expect)
