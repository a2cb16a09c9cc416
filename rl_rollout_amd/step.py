"""One S3R decode step over device-resident tensors, for one or more attention
layers, issued through the C ABI on torch's current stream.

Order of a step (wispaper.ai, "S3R drafts sparsely and verifies densely";
rit.work, "Как разреженный черновик сохраняет ответы плотной модели"):
  1. for draft step j = 1 .. gamma, for every layer: write the draft token's K/V
     row at L_b + j - 1, then sparse draft attention of its query over the
     layer's selected pages plus the tail (with draft_rows, no write: the draft
     reads the rows at L_b .. L_b + j - 1 from the draft-row buffers);
  2. for every layer: write the gamma + 1 block rows at L_b .. L_b + gamma (they
     replace the draft rows), then dense verify attention of the block, which
     also refreshes the layer's page scores;
  3. exact speculative accept over the block's logits, which commits
     ctx_lens[b] += a_b + 1;
  4. for every layer: budget selection over the new committed length, for the
     next step's drafts.
Logits and draft tokens are inputs (the model's projections are outside this
path). All layers share one page table and one ctx_lens array; each layer has its
own K/V pool, page scores and selection. Buffers are allocated once, at
construction; a step launches kernels only.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import torch

from . import s3r


def _direct(name: str, fn: Callable):
    return fn()


class DecodeStep:
    def __init__(self, layers: Sequence[Dict[str, torch.Tensor]], page_table: torch.Tensor, ctx_lens: torch.Tensor,
                 accept: Dict[str, torch.Tensor], gamma: int, budget, temperature: float = 1.0,
                 before_attn: Optional[Callable[[], None]] = None, run: Optional[Callable] = None,
                 fused_append: bool = False, per_head_selection: bool = False,
                 draft_rows: Optional[bool] = None, max_budget: Optional[float] = None):
        """layers[l]: k_cache, v_cache, q_verify [B][G1][Hq][D], q_draft [gamma][B][Hq][D],
        k_draft/v_draft [gamma][B][1][Hkv][D], k_block/v_block [B][G1][Hkv][D].
        accept: target_logits [B][G1][V], draft_logits [B][gamma][V], draft_tokens [B][gamma],
        u_accept [steps][B][gamma], u_sample [steps][B].
        budget: one sparse budget ratio for every sequence, or one per sequence (a
        sequence of B floats or a float64 tensor [B]); per-sequence budgets can be
        changed between steps with set_budgets, up to max_budget (default: the
        largest given).
        before_attn is called before every attention launch (e.g. a cache flush);
        run(name, fn) wraps every launch (e.g. an event timer). fused_append: the
        draft and verify launches write their own K/V rows (the *_append entry
        points) instead of a separate s3r_append_kv launch before each; measured
        on MI355X the separate launches are faster (stores issued while the chip
        streams KV cost more than the launch they save), so it is off by default."""
        self.fused_append = fused_append
        # per_head_selection: page scores and page sets per kv head (verify with
        # s3r_dense_verify_attn_head_scores, select over B x Hkv rows, drafts with a
        # page set per kv head: s3r_sparse_draft_attn_rows, or
        # s3r_sparse_draft_attn_head_sel after an append) instead of one set per
        # sequence.
        self.per_head = per_head_selection
        if per_head_selection and fused_append:
            raise ValueError("per-kv-head selection runs with separate append launches")
        # draft_rows (default unless fused_append): the drafts read the in-flight
        # draft tokens' K/V from the k_draft/v_draft buffers
        # (s3r_sparse_draft_attn_rows) and no draft row is appended; the verify
        # block's append writes those positions. Measured on MI355X: the step of
        # the 1.7B-like 16K workload is 2.7 % shorter than with an append launch
        # before each draft (each draft is 0.8 us longer, four appends are saved),
        # and the 8B-like 24K step is unchanged.
        if draft_rows is None:
            draft_rows = not fused_append
        self.draft_rows = draft_rows
        if draft_rows and fused_append:
            raise ValueError("draft_rows and fused_append are exclusive")
        self.layers = list(layers)
        self.ctx = ctx_lens
        self.table = page_table
        self.acc = accept
        self.gamma = gamma
        self.G1 = gamma + 1
        self.temperature = float(temperature)
        self.before_attn = before_attn or (lambda: None)
        self.run_op = run or _direct
        B, max_pages = page_table.shape
        dev = page_table.device
        self.kv = [s3r.KVCache(l["k_cache"], l["v_cache"], page_table, ctx_lens) for l in self.layers]
        Hq = self.layers[0]["q_verify"].shape[2]
        rows = (B, self.kv[0].num_kv_heads) if per_head_selection else (B,)
        # budget per selection row (sequence, or sequence x kv head), or None for a scalar budget
        self.budgets = None
        if isinstance(budget, (int, float)):
            self.budget = float(budget)
        else:
            b = torch.as_tensor(budget, dtype=torch.float64).flatten()
            if b.numel() != B:
                raise ValueError(f"{b.numel()} budgets for {B} sequences")
            self.budget = float(b.max()) if max_budget is None else float(max_budget)
            n_rows = B * (rows[1] if per_head_selection else 1)
            self.budgets = torch.empty((n_rows,), dtype=torch.float64, device=dev)
            self.set_budgets(b)
        self.max_sel = max(1, math.ceil(self.budget * max_pages))
        self.scores = [torch.zeros(rows + (max_pages,), dtype=torch.float32, device=dev) for _ in self.layers]
        self.sel = [torch.full(rows + (self.max_sel,), -1, dtype=torch.int32, device=dev) for _ in self.layers]
        self.nsel = [torch.zeros(rows, dtype=torch.int32, device=dev) for _ in self.layers]
        self.lens_rows = torch.zeros((B * self.kv[0].num_kv_heads,), dtype=torch.int32, device=dev)
        self.out_draft = [torch.empty_like(l["q_draft"][0]) for l in self.layers]
        # the draft-row buffers are the k_draft/v_draft inputs themselves, seen as
        # [gamma][B][Hkv][D] (views: rows the caller writes there between steps are read)
        Hkv, D = self.kv[0].num_kv_heads, self.kv[0].head_dim
        self.rows_k = [l["k_draft"].view(gamma, B, Hkv, D) for l in self.layers]
        self.rows_v = [l["v_draft"].view(gamma, B, Hkv, D) for l in self.layers]
        self.out_verify = [torch.empty_like(l["q_verify"]) for l in self.layers]
        self.verify_ws = torch.empty(max(1, s3r.dense_verify_workspace_size(self.kv[0], Hq, self.G1)),
                                     dtype=torch.uint8, device=dev)
        V = accept["target_logits"].shape[2]
        self.accept_ws = torch.empty(max(1, s3r.spec_accept_workspace_size(B, gamma, V)), dtype=torch.uint8,
                                     device=dev)
        self.num_accepted = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.out_tokens = torch.full((B, self.G1), -1, dtype=torch.int32, device=dev)
        self._horizons = {}

    def horizon(self, gamma: Optional[int]):
        """Inputs and buffers for a draft horizon gamma <= the construction gamma:
        contiguous leading slices of the block queries and rows, the logits, the
        draft tokens and the uniforms, built on first use and kept (so steps at a
        horizon seen before allocate nothing)."""
        if gamma is None or gamma == self.gamma:
            return None
        if not 1 <= gamma < self.gamma:
            raise ValueError(f"horizon {gamma} outside 1..{self.gamma}")
        h = self._horizons.get(gamma)
        if h is None:
            G1 = gamma + 1
            a = self.acc
            h = dict(
                q_verify=[l["q_verify"][:, :G1].contiguous() for l in self.layers],
                k_block=[l["k_block"][:, :G1].contiguous() for l in self.layers],
                v_block=[l["v_block"][:, :G1].contiguous() for l in self.layers],
                out_verify=[torch.empty_like(l["q_verify"][:, :G1]).contiguous() for l in self.layers],
                target_logits=a["target_logits"][:, :G1].contiguous(),
                draft_logits=a["draft_logits"][:, :gamma].contiguous(),
                draft_tokens=a["draft_tokens"][:, :gamma].contiguous(),
                u_accept=a["u_accept"][:, :, :gamma].contiguous(),
                out_tokens=torch.full((self.table.shape[0], G1), -1, dtype=torch.int32, device=self.table.device),
            )
            self._horizons[gamma] = h
        return h

    def set_budgets(self, budgets) -> None:
        """New per-sequence budgets (B floats, none above the construction's
        max_budget), used from the next selection on."""
        if self.budgets is None:
            raise ValueError("the step was built with one budget for every sequence")
        b = torch.as_tensor(budgets, dtype=torch.float64).flatten()
        if float(b.max()) > self.budget:
            raise ValueError(f"budget {float(b.max())} above the maximum {self.budget}")
        if self.per_head:
            b = b.repeat_interleave(self.budgets.numel() // b.numel())
        self.budgets.copy_(b)

    def check_inputs(self) -> Dict[int, List[str]]:
        """Device-input checks of the next step (s3r_check_step_inputs; a host sync, for
        debug runs): every layer's lengths and page-table entries for the block, its
        selection, and the draft tokens. Returns {sequence: [problems]}, empty when
        all is well."""
        V = self.acc["draft_logits"].shape[2]
        bad: Dict[int, List[str]] = {}
        for l in range(self.num_layers):
            e = s3r.s3r_check_step_inputs(self.kv[l], self.G1, self.sel[l], self.nsel[l],
                                          self.acc["draft_tokens"] if l == 0 else None, V)
            for b, probs in s3r.describe_check(e).items():
                seen = bad.setdefault(b, [])
                seen.extend(p for p in probs if p not in seen)
        return bad

    def replace_accept(self, accept: Dict[str, torch.Tensor]) -> None:
        """Swap in other logits, draft tokens and uniforms of the same shapes."""
        self.acc = accept
        self._horizons = {}

    @property
    def num_layers(self) -> int:
        return len(self.layers)

    def seed_scores(self) -> None:
        """Page scores for the first drafts: one verify per layer whose block sits at
        L_b - G1 .. L_b - 1, as if the previous step had accepted every draft, then
        a selection over L_b."""
        prev = (self.ctx - self.G1).clamp_min(0).to(torch.int32).contiguous()
        for l, layer in enumerate(self.layers):
            kv_prev = s3r.KVCache(layer["k_cache"], layer["v_cache"], self.table, prev)
            if self.per_head:
                s3r.s3r_dense_verify_attn_head_scores(kv_prev, layer["q_verify"], out=self.out_verify[l],
                                                      head_page_scores=self.scores[l], workspace=self.verify_ws)
            else:
                s3r.s3r_dense_verify_attn(kv_prev, layer["q_verify"], out=self.out_verify[l],
                                          page_scores=self.scores[l], workspace=self.verify_ws)
        self.select_phase()

    def _check_horizons(self, horizons) -> None:
        if horizons is not None and (not self.draft_rows or self.per_head):
            raise ValueError("a horizon per sequence needs draft-row mode and one page set per sequence")

    def draft_phase(self, j: int, horizons: Optional[torch.Tensor] = None) -> None:
        """Draft step j for every layer (horizons: int32 [B], sequences with
        horizons[b] < j are skipped)."""
        self._check_horizons(horizons)
        for l, layer in enumerate(self.layers):
            kv = self.kv[l]
            kr, vr = layer["k_draft"][j - 1], layer["v_draft"][j - 1]
            if self.draft_rows:
                self.before_attn()
                self.run_op(f"draft{j}", lambda: s3r.s3r_sparse_draft_attn_rows(
                    kv, layer["q_draft"][j - 1], self.rows_k[l], self.rows_v[l], self.sel[l], self.nsel[l], j,
                    out=self.out_draft[l], horizons=horizons))
                continue
            if self.fused_append:
                self.before_attn()
                self.run_op(f"draft{j}", lambda: s3r.s3r_sparse_draft_attn_append(
                    kv, layer["q_draft"][j - 1], kr, vr, self.sel[l], self.nsel[l], j, out=self.out_draft[l]))
                continue
            self.run_op("append", lambda: s3r.s3r_append_kv(kv, kr, vr, offset=j - 1))
            self.before_attn()
            draft = s3r.s3r_sparse_draft_attn_head_sel if self.per_head else s3r.s3r_sparse_draft_attn
            self.run_op(f"draft{j}", lambda: draft(kv, layer["q_draft"][j - 1], self.sel[l], self.nsel[l], j,
                                                   out=self.out_draft[l]))

    def verify_phase(self, gamma: Optional[int] = None, horizons: Optional[torch.Tensor] = None) -> None:
        """Append and verify the block of gamma + 1 rows (horizons: int32 [B], the
        block of sequence b is its first horizons[b] + 1 queries)."""
        self._check_horizons(horizons)
        h = self.horizon(gamma)
        for l, layer in enumerate(self.layers):
            kv = self.kv[l]
            kb, vb = (layer["k_block"], layer["v_block"]) if h is None else (h["k_block"][l], h["v_block"][l])
            q, out = (layer["q_verify"], self.out_verify[l]) if h is None else (h["q_verify"][l], h["out_verify"][l])
            if self.fused_append:
                self.before_attn()
                self.run_op("verify", lambda: s3r.s3r_dense_verify_attn_append(
                    kv, q, kb, vb, out=out, page_scores=self.scores[l], workspace=self.verify_ws))
                continue
            self.run_op("append", lambda: s3r.s3r_append_kv(kv, kb, vb, offset=0))
            self.before_attn()
            if self.per_head:
                self.run_op("verify", lambda: s3r.s3r_dense_verify_attn_head_scores(
                    kv, q, out=out, head_page_scores=self.scores[l], workspace=self.verify_ws))
            else:
                self.run_op("verify", lambda: s3r.s3r_dense_verify_attn(kv, q, out=out, page_scores=self.scores[l],
                                                                        workspace=self.verify_ws, horizons=horizons))

    def accept_phase(self, s: int, gamma: Optional[int] = None, horizons: Optional[torch.Tensor] = None,
                     uniforms: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> None:
        """uniforms: (u_accept [B][gamma], u_sample [B]) read instead of step s's
        (fixed buffers for a captured graph)."""
        self._check_horizons(horizons)
        h = self.horizon(gamma)
        a = self.acc if h is None else h
        ua, us = (a["u_accept"][s], self.acc["u_sample"][s]) if uniforms is None else uniforms
        toks = self.out_tokens if h is None else h["out_tokens"]
        self.run_op("accept", lambda: s3r.s3r_spec_accept(a["target_logits"], a["draft_logits"], a["draft_tokens"],
                                                          ua, us, self.temperature,
                                                          ctx_lens=self.ctx, num_accepted=self.num_accepted,
                                                          out_tokens=toks, workspace=self.accept_ws,
                                                          horizons=horizons))

    def _budget_arg(self):
        return self.budget if self.budgets is None else self.budgets

    def select_phase(self) -> None:
        if self.per_head:
            B, H = self.nsel[0].shape
            self.lens_rows.view(B, H).copy_(self.ctx[:, None].expand(B, H))
        for l in range(self.num_layers):
            if self.per_head:
                B, H, P = self.scores[l].shape
                self.run_op("select", lambda: s3r.s3r_select_budget(
                    self.scores[l].view(B * H, P), self.lens_rows, self._budget_arg(), self.max_sel,
                    sel_pages=self.sel[l].view(B * H, self.max_sel), num_sel=self.nsel[l].view(B * H),
                    max_budget=self.budget))
            else:
                self.run_op("select", lambda: s3r.s3r_select_budget(self.scores[l], self.ctx, self._budget_arg(),
                                                                    self.max_sel, sel_pages=self.sel[l],
                                                                    num_sel=self.nsel[l], max_budget=self.budget))

    def run(self, s: int, gamma: Optional[int] = None, horizons: Optional[torch.Tensor] = None,
            uniforms: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> None:
        """One whole step; s indexes the step's uniforms; gamma (default: the
        construction gamma) is this step's draft horizon, or, with horizons (int32
        [B] on the device, each in 0 .. gamma), the largest of the sequences' own
        horizons: sequence b drafts horizons[b] tokens, verifies them plus one, and
        tests only those drafts."""
        g = self.gamma if gamma is None else gamma
        for j in range(1, g + 1):
            self.draft_phase(j, horizons)
        self.verify_phase(gamma, horizons)
        self.accept_phase(s, gamma, horizons, uniforms)
        self.select_phase()


class StepGraph:
    """A whole step of a DecodeStep captured once in a HIP graph and replayed: the
    step's launches (drafts, append, verify, accept, selection; kernels only, no
    memory sets or allocations) become one graph launch. Each replay first copies
    step s's uniforms into the fixed buffers the captured accept reads.

    The step must have run eagerly at least once before (a kernel's first launch
    loads its code, which must not happen during capture), and the step's timer
    hook, if any, is bypassed while capturing. replay(s) then does what
    step.run(s, gamma) does."""

    def __init__(self, step: DecodeStep, gamma: Optional[int] = None):
        self.st = step
        self.gamma = gamma
        h = step.horizon(gamma)
        a = step.acc if h is None else h
        self.ua = a["u_accept"][0].clone()
        self.us = step.acc["u_sample"][0].clone()
        self.graph = torch.cuda.CUDAGraph()
        run_op = step.run_op
        step.run_op = _direct
        try:
            with torch.cuda.graph(self.graph):
                step.run(0, gamma, uniforms=(self.ua, self.us))
        finally:
            step.run_op = run_op

    def replay(self, s: int) -> None:
        h = self.st.horizon(self.gamma)
        a = self.st.acc if h is None else h
        self.ua.copy_(a["u_accept"][s])
        self.us.copy_(self.st.acc["u_sample"][s])
        self.graph.replay()


def build_inputs(w, seed: int, steps: int, max_pages: Optional[int] = None, ragged_alloc: bool = True,
                 draft_noise: Optional[float] = None, seq_noise=None):
    """Seeded device inputs for `steps` steps of workload w over w.num_layers layers
    (seq_noise: one draft-noise value per sequence).
    Returns (layers, page_table, ctx_lens, accept, max_pages, num_blocks)."""
    from . import synth
    G1 = w.block_len
    headroom = (steps + 2) * G1
    if max_pages is None:
        max_pages = math.ceil((w.ctx_range[1] + headroom) / w.page_size)
    lens, table, nb = synth.device_page_table(w, seed, max_pages, headroom=headroom if ragged_alloc else None)
    layers: List[Dict[str, torch.Tensor]] = []
    for l in range(w.num_layers):
        k, v = synth.device_layer_kv(w, seed, nb, l)
        layer = dict(k_cache=k, v_cache=v)
        layer.update(synth.device_layer_queries(w, seed, lens.shape[0], l))
        layers.append(layer)
    accept = synth.device_accept_inputs(w, seed, steps, draft_noise=draft_noise, seq_noise=seq_noise)
    ctx = torch.from_numpy(lens).cuda()
    return layers, table, ctx, accept, max_pages, nb
