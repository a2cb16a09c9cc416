"""A whole step captured in a HIP graph (StepGraph) against the same step run
eagerly from the same state: outputs, page scores, selections, accept counts,
tokens, committed lengths and the cache contents must agree bit for bit (every
kernel is deterministic). Replayed several times, with eager steps, host syncs
and torch work between the replays, each replay checked."""
import pytest
import torch

from rl_rollout_amd import workloads as W

pytestmark = pytest.mark.gpu


def _state(st, layers):
    t = {"ctx": st.ctx, "num_accepted": st.num_accepted, "out_tokens": st.out_tokens}
    for l, layer in enumerate(layers):
        t[f"k{l}"] = layer["k_cache"]
        t[f"v{l}"] = layer["v_cache"]
        t[f"scores{l}"] = st.scores[l]
        t[f"sel{l}"] = st.sel[l]
        t[f"nsel{l}"] = st.nsel[l]
        t[f"out_verify{l}"] = st.out_verify[l]
        t[f"out_draft{l}"] = st.out_draft[l]
    return t


@pytest.mark.parametrize("gamma", [None, 3])
def test_graph_replay_equals_the_eager_step(gamma):
    from rl_rollout_amd.step import DecodeStep, StepGraph, build_inputs
    w = W.QWEN3_1P7B_16K_POSITIONS.with_(num_seqs=8, ctx_range=(1000, 3000), num_layers=2)
    layers, table, ctx, acc, max_pages, nb = build_inputs(w, 41, steps=12)
    st = DecodeStep(layers, table, ctx, acc, w.gamma, w.budget, w.temperature)
    st.seed_scores()
    st.run(0, gamma)                     # eager: loads every kernel the step uses
    torch.cuda.synchronize()
    graph = StepGraph(st, gamma)
    for s in range(1, 5):
        print(f"graph replay {s}, gamma={gamma}", flush=True)
        state = _state(st, layers)
        saved = {k: v.clone() for k, v in state.items()}
        st.run(s, gamma)                 # eager
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in state.items()}
        for k, v in state.items():       # back to the state before the step
            v.copy_(saved[k])
        _ = (saved["ctx"].float() * 2).sum().item()   # unrelated eager torch work and a sync
        graph.replay(s)
        torch.cuda.synchronize()
        for k, v in state.items():
            assert torch.equal(v, eager[k]), (s, k)
