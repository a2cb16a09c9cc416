"""Seeded synthetic inputs for the S3R hot path.

This module only draws and lays out input data; it holds none of the method's
arithmetic. Both the HIP path (through the binding) and the CPU oracle read the
arrays it returns.

Recipe (per workload and seed):
  * one numpy Generator(PCG64) per tensor, spawned from SeedSequence(seed) in a
    fixed order (lengths, block permutation, K, V, Q-verify, Q-draft, target
    logits, draft noise, draft-token Gumbel noise, u_accept, u_sample);
  * values drawn in float32, then rounded to bf16 (round to nearest even) as
    uint16 bit patterns when the workload is bf16;
  * every physical block is filled, including slots past a sequence's length,
    so a kernel that reads past the mask reads finite garbage that changes the
    result;
  * each sequence owns its pages: a seeded random permutation of physical blocks
    (no prefix sharing), so page gathers are scattered;
  * draft tokens are drawn from softmax(draft logits / T) by the Gumbel-max rule
    (argmax of logits / T + Gumbel noise), which is an exact draw from that
    distribution; uniforms are float32 in [0, 1).
For workloads too large for host generation, device_* functions draw the same
distributions with torch's seeded device generator (a different stream of
numbers, same recipe).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .workloads import Workload

_STREAMS = ("lens", "perm", "k", "v", "q_verify", "q_draft", "target", "noise", "gumbel",
            "u_accept", "u_sample", "k_new", "v_new")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gens(seed: int):
    ss = np.random.SeedSequence(seed)
    return dict(zip(_STREAMS, (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(len(_STREAMS)))))


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _decode(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


@dataclass
class AttnInputs:
    """Paged KV for one layer plus the queries of one decode step.

    k_cache [NB][Hkv][P][D], v_cache [NB][Hkv][D][P] (page-transposed V),
    page_table [B][max_pages] int32, ctx_lens [B] int32,
    q_verify [B][G1][Hq][D], q_draft [gamma][B][Hq][D],
    k_new/v_new [B][G1][Hkv][D]: rows a step appends at L_b .. L_b + G1 - 1.
    Float tensors are float32 or bf16 bit patterns (uint16).
    """
    k_cache: np.ndarray
    v_cache: np.ndarray
    page_table: np.ndarray
    ctx_lens: np.ndarray
    q_verify: np.ndarray
    q_draft: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray


@dataclass
class AcceptInputs:
    target_logits: np.ndarray   # [B][G1][V]
    draft_logits: np.ndarray    # [B][gamma][V]
    draft_tokens: np.ndarray    # [B][gamma] int32
    u_accept: np.ndarray        # [B][gamma] float32
    u_sample: np.ndarray        # [B] float32


def draw_ctx_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    lo, hi = w.ctx_range
    if lo == hi:
        return np.full(w.num_seqs, lo, dtype=np.int32)
    return rng.integers(lo, hi + 1, size=w.num_seqs, dtype=np.int64).astype(np.int32)


def make_page_table(num_seqs: int, max_pages: int, rng: np.random.Generator, spare_blocks: int = 3):
    """Random, disjoint logical -> physical block maps. Returns (table, num_blocks)."""
    num_blocks = num_seqs * max_pages + spare_blocks
    perm = rng.permutation(num_blocks)[: num_seqs * max_pages]
    return perm.reshape(num_seqs, max_pages).astype(np.int32), num_blocks


def make_attn_inputs(w: Workload, seed: int, ctx_lens: Optional[np.ndarray] = None,
                     max_pages: Optional[int] = None) -> AttnInputs:
    g = _gens(seed)
    lens = draw_ctx_lens(w, g["lens"]) if ctx_lens is None else np.asarray(ctx_lens, dtype=np.int32)
    B = lens.shape[0]
    mp = w.max_pages() if max_pages is None else int(max_pages)
    table, nb = make_page_table(B, mp, g["perm"])
    Hkv, Hq, D, P, G1 = w.num_kv_heads, w.num_q_heads, w.head_dim, w.page_size, w.block_len
    k = g["k"].standard_normal((nb, Hkv, P, D), dtype=np.float32)
    v = g["v"].standard_normal((nb, Hkv, D, P), dtype=np.float32)
    qv = g["q_verify"].standard_normal((B, G1, Hq, D), dtype=np.float32)
    qd = g["q_draft"].standard_normal((w.gamma, B, Hq, D), dtype=np.float32)
    kn = g["k_new"].standard_normal((B, G1, Hkv, D), dtype=np.float32)
    vn = g["v_new"].standard_normal((B, G1, Hkv, D), dtype=np.float32)
    dt = w.kv_dtype
    return AttnInputs(_cast(k, dt), _cast(v, dt), table, lens, _cast(qv, dt), _cast(qd, dt),
                      _cast(kn, dt), _cast(vn, dt))


def gumbel_max_tokens(logits: np.ndarray, temperature: float, rng: np.random.Generator) -> np.ndarray:
    """One exact draw per row from softmax(logits / T), via argmax(logits / T + G)."""
    x = _decode(logits).astype(np.float64) / float(np.float32(temperature))
    u = rng.random(x.shape)
    u = np.where(u <= 0.0, np.finfo(np.float64).tiny, u)
    return np.argmax(x - np.log(-np.log(u)), axis=-1).astype(np.int32)


def noise_scales(w: Workload, draft_noise: Optional[float] = None) -> np.ndarray:
    """Draft-noise standard deviation per draft position (float32 [gamma]): the
    workload's position profile if it has one (and no override is given), else
    one value for every position."""
    if draft_noise is None and w.position_noise:
        if len(w.position_noise) < w.gamma:
            raise ValueError("position_noise shorter than gamma")
        return np.asarray(w.position_noise[: w.gamma], dtype=np.float32)
    sigma = w.draft_noise if draft_noise is None else draft_noise
    return np.full(w.gamma, sigma, dtype=np.float32)


def noise_grid(w: Workload, num_seqs: int, draft_noise: Optional[float] = None,
               seq_noise: Optional[np.ndarray] = None) -> np.ndarray:
    """Draft-noise standard deviation per (sequence, draft position), float32
    [B][gamma]: one value per sequence for every position if seq_noise is given,
    else noise_scales for every sequence."""
    if seq_noise is None:
        return np.broadcast_to(noise_scales(w, draft_noise)[None, :], (num_seqs, w.gamma))
    sn = np.asarray(seq_noise, dtype=np.float32).reshape(-1)
    if sn.shape[0] != num_seqs:
        raise ValueError(f"{sn.shape[0]} noise values for {num_seqs} sequences")
    return np.broadcast_to(sn[:, None], (num_seqs, w.gamma))


def make_accept_inputs(w: Workload, seed: int, num_seqs: Optional[int] = None,
                       draft_noise: Optional[float] = None, seq_noise: Optional[np.ndarray] = None) -> AcceptInputs:
    g = _gens(seed)
    B = w.num_seqs if num_seqs is None else int(num_seqs)
    V, G1, gm = w.vocab, w.block_len, w.gamma
    t32 = (g["target"].standard_normal((B, G1, V), dtype=np.float32) * np.float32(w.target_std))
    n32 = g["noise"].standard_normal((B, gm, V), dtype=np.float32) * noise_grid(w, B, draft_noise, seq_noise)[:, :, None]
    d32 = t32[:, :gm, :] + n32
    tl = _cast(t32, w.logits_dtype)
    dl = _cast(d32, w.logits_dtype)
    tokens = gumbel_max_tokens(dl, w.temperature, g["gumbel"])
    ua = g["u_accept"].random((B, gm), dtype=np.float32)
    us = g["u_sample"].random(B, dtype=np.float32)
    return AcceptInputs(tl, dl, tokens, ua, us)


# ---------------------------------------------------------------- toy Markov policy

def markov_tables(vocab: int, seed: int, min_prob: float = 1e-4, alpha: float = 2.0):
    """Row-stochastic dense (p) and draft (q) tables for the exactness tests.

    Rows are Dirichlet(alpha) draws; a row with an entry below min_prob is redrawn,
    so every cell of a two-token joint keeps an expected count worth testing."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def table():
        rows = []
        while len(rows) < vocab:
            r = rng.dirichlet(np.full(vocab, alpha))
            if r.min() >= min_prob:
                rows.append(r)
        return np.array(rows)

    return table(), table()


# ---------------------------------------------------------------- device-side generation

def _torch_gen(seed: int, stream: str, layer: int = 0):
    import torch
    g = torch.Generator(device="cuda")
    key = [seed, _STREAMS.index(stream)] + ([layer] if layer else [])
    g.manual_seed(int(np.random.SeedSequence(key).generate_state(1)[0]))
    return g


def _randn_dev(shape, dtype, seed, stream, scale=1.0, layer=0, chunk_elems=1 << 28):
    """N(0, scale^2) on the GPU. Unit-scale tensors are drawn directly in `dtype`
    (torch rounds to nearest even); scaled ones are drawn in float32 chunks,
    scaled, then rounded, so the float32 staging stays small."""
    import torch
    g = _torch_gen(seed, stream, layer)
    out = torch.empty(shape, dtype=dtype, device="cuda")
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - s)
        if scale == 1.0:
            flat[s:s + n] = torch.randn(n, generator=g, device="cuda", dtype=dtype)
        else:
            x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
            x.mul_(scale)
            flat[s:s + n].copy_(x)
    return out


def device_page_table(w: Workload, seed: int, max_pages: int, ctx_lens: Optional[np.ndarray] = None,
                      headroom: Optional[int] = None):
    """Context lengths and a seeded page table on the GPU.

    With `headroom` (tokens) each sequence owns only the blocks its length plus
    the headroom needs, ceil((L_b + headroom) / P) capped at max_pages, drawn from
    one random permutation of the pool; table entries past them are -1 and are
    never read. Without it every sequence owns max_pages blocks. Returns
    (lens numpy int32, table torch int32 [B][max_pages], num_blocks)."""
    import torch
    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    lens = (draw_ctx_lens(w, np.random.Generator(np.random.PCG64(ss[0]))) if ctx_lens is None
            else np.asarray(ctx_lens, dtype=np.int32))
    B = lens.shape[0]
    perm_rng = np.random.Generator(np.random.PCG64(ss[1]))
    if headroom is None:
        table, nb = make_page_table(B, max_pages, perm_rng)
    else:
        P = w.page_size
        owned = np.minimum(max_pages, -(-(lens.astype(np.int64) + int(headroom)) // P))
        nb = int(owned.sum()) + 3
        perm = perm_rng.permutation(nb)
        table = np.full((B, max_pages), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            table[b, :owned[b]] = perm[o:o + owned[b]]
            o += int(owned[b])
    return lens, torch.from_numpy(table).cuda(), nb


def device_layer_kv(w: Workload, seed: int, num_blocks: int, layer: int = 0):
    """K [NB][Hkv][P][D] and page-transposed V [NB][Hkv][D][P] of one layer, N(0, 1)."""
    import torch
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    Hkv, D, P = w.num_kv_heads, w.head_dim, w.page_size
    return (_randn_dev((num_blocks, Hkv, P, D), dt, seed, "k", layer=layer),
            _randn_dev((num_blocks, Hkv, D, P), dt, seed, "v", layer=layer))


def device_layer_queries(w: Workload, seed: int, num_seqs: int, layer: int = 0):
    """One step's queries and appended rows of one layer: q_verify [B][G1][Hq][D],
    q_draft [gamma][B][Hq][D], k_draft/v_draft [gamma][B][1][Hkv][D] (row of draft
    step j), k_block/v_block [B][G1][Hkv][D] (the verify block's rows)."""
    import torch
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    B, Hkv, Hq, D, G1 = num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim, w.block_len
    return dict(
        q_verify=_randn_dev((B, G1, Hq, D), dt, seed, "q_verify", layer=layer),
        q_draft=_randn_dev((w.gamma, B, Hq, D), dt, seed, "q_draft", layer=layer),
        k_draft=_randn_dev((w.gamma, B, 1, Hkv, D), dt, seed, "k_new", layer=layer),
        v_draft=_randn_dev((w.gamma, B, 1, Hkv, D), dt, seed, "v_new", layer=layer),
        k_block=_randn_dev((B, G1, Hkv, D), dt, seed + 1_000_003, "k_new", layer=layer),
        v_block=_randn_dev((B, G1, Hkv, D), dt, seed + 1_000_003, "v_new", layer=layer),
    )


def device_attn_inputs(w: Workload, seed: int, max_pages: int, ctx_lens: Optional[np.ndarray] = None,
                       headroom: Optional[int] = None, layer: int = 0):
    """The AttnInputs recipe drawn directly on the GPU (torch tensors) for one
    layer: a dict with k_cache, v_cache, page_table, ctx_lens, num_blocks and the
    device_layer_queries tensors."""
    import torch
    lens, table, nb = device_page_table(w, seed, max_pages, ctx_lens, headroom)
    k, v = device_layer_kv(w, seed, nb, layer)
    d = dict(k_cache=k, v_cache=v, page_table=table, ctx_lens=torch.from_numpy(lens).cuda(), num_blocks=nb)
    d.update(device_layer_queries(w, seed, lens.shape[0], layer))
    return d


def device_accept_inputs(w: Workload, seed: int, steps: int, draft_noise: Optional[float] = None,
                         seq_noise: Optional[np.ndarray] = None):
    """Logits, Gumbel-max draft tokens and per-step uniforms on the GPU (seq_noise:
    one draft-noise value per sequence, as in noise_grid)."""
    import torch
    B, V, G1, gm = w.num_seqs, w.vocab, w.block_len, w.gamma
    dt = torch.bfloat16 if w.logits_dtype == "bf16" else torch.float32
    t32 = _randn_dev((B, G1, V), torch.float32, seed, "target", scale=w.target_std)
    n32 = _randn_dev((B, gm, V), torch.float32, seed, "noise")
    n32.mul_(torch.from_numpy(np.ascontiguousarray(noise_grid(w, B, draft_noise, seq_noise))).cuda()[:, :, None])
    tl = t32.to(dt)
    dl = (t32[:, :gm] + n32).to(dt)
    del t32, n32
    g = _torch_gen(seed, "gumbel")
    x = dl.float() / float(np.float32(w.temperature))
    u = torch.rand(x.shape, generator=g, device="cuda", dtype=torch.float64).clamp_min_(1e-300)
    tokens = torch.argmax(x.double() - torch.log(-torch.log(u)), dim=-1).to(torch.int32).contiguous()
    del x, u
    ga = _torch_gen(seed, "u_accept")
    gs = _torch_gen(seed, "u_sample")
    ua = torch.rand((steps, B, gm), generator=ga, device="cuda", dtype=torch.float32)
    us = torch.rand((steps, B), generator=gs, device="cuda", dtype=torch.float32)
    return dict(target_logits=tl.contiguous(), draft_logits=dl.contiguous(), draft_tokens=tokens,
                u_accept=ua, u_sample=us)
