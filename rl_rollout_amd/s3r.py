"""Thin ctypes binding of libs3r.so (C ABI in include/s3r.h).

Argument marshalling only: every function takes torch tensors that already live
on the GPU, checks their dtype, device and contiguity, allocates outputs and
workspace with torch when the caller does not pass them, and calls the C entry
point of the same name on torch's current HIP stream. All computation happens in
the library's kernels. Importing this module loads the library and raises if it
is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, List, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("S3R_LIB", os.path.join(_PKG, "libs3r.so"))

S3R_F32 = 0
S3R_BF16 = 1
PAGE_SIZE = 16

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rl_rollout_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

_c_int = ctypes.c_int32
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t


class PagedKV(ctypes.Structure):
    """Mirror of s3r_paged_kv."""
    _fields_ = [
        ("k_cache", _c_ptr), ("v_cache", _c_ptr), ("page_table", _c_ptr), ("ctx_lens", _c_ptr),
        ("num_blocks", _c_int), ("num_kv_heads", _c_int), ("page_size", _c_int), ("head_dim", _c_int),
        ("max_pages_per_seq", _c_int), ("dtype", _c_int),
    ]


_P_KV = ctypes.POINTER(PagedKV)


def _sig(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_status_string = _sig("s3r_status_string", ctypes.c_char_p, _c_int)
_version = _sig("s3r_version", _c_int)
_append = _sig("s3r_append_kv", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr)
_verify_ws = _sig("s3r_dense_verify_workspace_size", _c_size, _P_KV, _c_int, _c_int, _c_int)
_verify = _sig("s3r_dense_verify_attn", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, ctypes.c_float, _c_ptr,
               _c_ptr, _c_ptr, _c_size, _c_ptr)
_select = _sig("s3r_select_budget", _c_int, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, ctypes.c_double, _c_ptr, _c_ptr,
               _c_int, _c_ptr, _c_size, _c_ptr)
_select_rows = _sig("s3r_select_budget_rows", _c_int, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_ptr, ctypes.c_double,
                    _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr)
_draft = _sig("s3r_sparse_draft_attn", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, ctypes.c_float, _c_ptr, _c_ptr,
              _c_int, _c_ptr, _c_ptr, _c_size, _c_ptr)
_verify_app = _sig("s3r_dense_verify_attn_append", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                   ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr)
_verify_head = _sig("s3r_dense_verify_attn_head_scores", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, ctypes.c_float,
                    _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr)
_draft_head = _sig("s3r_sparse_draft_attn_head_sel", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, ctypes.c_float,
                   _c_ptr, _c_ptr, _c_int, _c_ptr, _c_ptr, _c_size, _c_ptr)
_draft_app = _sig("s3r_sparse_draft_attn_append", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                  ctypes.c_float, _c_ptr, _c_ptr, _c_int, _c_ptr, _c_ptr, _c_size, _c_ptr)
_draft_rows = _sig("s3r_sparse_draft_attn_rows", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                   ctypes.c_int64, ctypes.c_int64, ctypes.c_float, _c_ptr, _c_ptr, _c_int, _c_int, _c_ptr, _c_ptr,
                   _c_size, _c_ptr)
_verify_ragged = _sig("s3r_dense_verify_attn_ragged", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr,
                      ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr)
_draft_ragged = _sig("s3r_sparse_draft_attn_ragged", _c_int, _P_KV, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                     ctypes.c_int64, ctypes.c_int64, ctypes.c_float, _c_ptr, _c_ptr, _c_int, _c_int, _c_ptr, _c_ptr,
                     _c_ptr, _c_size, _c_ptr)
_check_inputs = _sig("s3r_check_step_inputs", _c_int, _P_KV, _c_int, _c_int, _c_ptr, _c_ptr, _c_int, _c_int, _c_ptr,
                     _c_int, _c_int, _c_ptr, _c_ptr)
_select_ws = _sig("s3r_select_budget_workspace_size", _c_size, _c_int, _c_int)
_draft_ws = _sig("s3r_sparse_draft_workspace_size", _c_size, _P_KV, _c_int, _c_int)
_page_bytes = _sig("s3r_page_bytes", _c_size, _P_KV)
_pack = _sig("s3r_pack_pages", _c_int, _P_KV, _c_ptr, _c_int, _c_ptr, _c_ptr)
_unpack = _sig("s3r_unpack_pages", _c_int, _P_KV, _c_ptr, _c_int, _c_ptr, _c_ptr)
_accept_ws = _sig("s3r_spec_accept_workspace_size", _c_size, _c_int, _c_int, _c_int)
_accept = _sig("s3r_spec_accept", _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
               ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr)
_accept_ragged = _sig("s3r_spec_accept_ragged", _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                      _c_ptr, _c_ptr, _c_ptr, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr)
_accept_no_alloc = _sig("s3r_spec_accept_no_alloc", _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr,
                        _c_ptr, _c_ptr, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr)


class S3RError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return _status_string(int(status)).decode()


def version() -> int:
    return int(_version())


def _check(status: int, where: str):
    if status != 0:
        raise S3RError(status, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return S3R_BF16
    if dt == torch.float32:
        return S3R_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


class KVCache:
    """A paged KV cache of one layer (k [NB][Hkv][16][D], v [NB][Hkv][D][16])."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                 ctx_lens: torch.Tensor):
        _need(k_cache, "k_cache", (torch.bfloat16, torch.float32))
        _need(v_cache, "v_cache", k_cache.dtype)
        _need(page_table, "page_table", torch.int32)
        _need(ctx_lens, "ctx_lens", torch.int32)
        nb, hkv, p, d = k_cache.shape
        if tuple(v_cache.shape) != (nb, hkv, d, p):
            raise ValueError(f"v_cache must be [{nb}][{hkv}][{d}][{p}], got {tuple(v_cache.shape)}")
        if page_table.dim() != 2 or ctx_lens.dim() != 1 or ctx_lens.shape[0] != page_table.shape[0]:
            raise ValueError("page_table must be [B][max_pages] and ctx_lens [B]")
        self.k_cache, self.v_cache, self.page_table, self.ctx_lens = k_cache, v_cache, page_table, ctx_lens
        self.desc = PagedKV(k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(), ctx_lens.data_ptr(),
                            nb, hkv, p, d, page_table.shape[1], _dtype_code(k_cache.dtype))

    @property
    def num_seqs(self) -> int:
        return self.page_table.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k_cache.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k_cache.shape[3]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    @property
    def dtype(self) -> torch.dtype:
        return self.k_cache.dtype


def s3r_append_kv(kv: KVCache, k_rows: torch.Tensor, v_rows: torch.Tensor, offset: int = 0) -> None:
    """Write rows [B][R][Hkv][D] at positions ctx_lens[b] + offset + r."""
    _need(k_rows, "k_rows", kv.dtype)
    _need(v_rows, "v_rows", kv.dtype)
    B, R = k_rows.shape[0], k_rows.shape[1]
    if tuple(k_rows.shape) != (kv.num_seqs, R, kv.num_kv_heads, kv.head_dim) or v_rows.shape != k_rows.shape:
        raise ValueError("k_rows/v_rows must be [B][R][Hkv][D]")
    _check(_append(ctypes.byref(kv.desc), B, int(offset), R, k_rows.data_ptr(), v_rows.data_ptr(), _stream()),
           "s3r_append_kv")


def dense_verify_workspace_size(kv: KVCache, num_q_heads: int, block_len: int) -> int:
    return int(_verify_ws(ctypes.byref(kv.desc), kv.num_seqs, num_q_heads, block_len))


def _need_horizons(horizons: torch.Tensor, B: int) -> None:
    _need(horizons, "horizons", torch.int32)
    if tuple(horizons.shape) != (B,):
        raise ValueError("horizons must be [B] int32")


def s3r_dense_verify_attn(kv: KVCache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
                          page_scores: Optional[torch.Tensor] = None, want_scores: bool = True,
                          scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                          horizons: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [B][G1][Hq][D] -> (out [B][G1][Hq][D], page_scores [B][max_pages] float32 or None).
    horizons (int32 [B], s3r_dense_verify_attn_ragged): sequence b's block is its first
    horizons[b] + 1 queries; later out rows are zeros and add nothing to the scores."""
    _need(q, "q", kv.dtype)
    B, G1, Hq, D = q.shape
    if B != kv.num_seqs or D != kv.head_dim:
        raise ValueError("q must be [B][G1][Hq][D] matching the cache")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    if want_scores and page_scores is None:
        page_scores = torch.empty((B, kv.max_pages), dtype=torch.float32, device=q.device)
    if page_scores is not None:
        _need(page_scores, "page_scores", torch.float32)
    ws_bytes = dense_verify_workspace_size(kv, Hq, G1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if horizons is not None:
        _need_horizons(horizons, B)
        _check(_verify_ragged(ctypes.byref(kv.desc), B, Hq, G1, q.data_ptr(), horizons.data_ptr(), sc,
                              out.data_ptr(), _ptr(page_scores), workspace.data_ptr(), workspace.numel(), _stream()),
               "s3r_dense_verify_attn_ragged")
        return out, page_scores
    _check(_verify(ctypes.byref(kv.desc), B, Hq, G1, q.data_ptr(), sc, out.data_ptr(), _ptr(page_scores),
                   workspace.data_ptr(), workspace.numel(), _stream()), "s3r_dense_verify_attn")
    return out, page_scores


def s3r_dense_verify_attn_append(kv: KVCache, q: torch.Tensor, k_block: torch.Tensor, v_block: torch.Tensor,
                                 out: Optional[torch.Tensor] = None, page_scores: Optional[torch.Tensor] = None,
                                 want_scores: bool = True, scale: Optional[float] = None,
                                 workspace: Optional[torch.Tensor] = None
                                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Writes k_block/v_block [B][G1][Hkv][D] at positions ctx_lens[b] + i, then
    as s3r_dense_verify_attn: q [B][G1][Hq][D] -> (out, page_scores or None)."""
    _need(q, "q", kv.dtype)
    _need(k_block, "k_block", kv.dtype)
    _need(v_block, "v_block", kv.dtype)
    B, G1, Hq, D = q.shape
    if B != kv.num_seqs or D != kv.head_dim:
        raise ValueError("q must be [B][G1][Hq][D] matching the cache")
    if tuple(k_block.shape) != (B, G1, kv.num_kv_heads, D) or v_block.shape != k_block.shape:
        raise ValueError("k_block/v_block must be [B][G1][Hkv][D]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    if want_scores and page_scores is None:
        page_scores = torch.empty((B, kv.max_pages), dtype=torch.float32, device=q.device)
    if page_scores is not None:
        _need(page_scores, "page_scores", torch.float32)
    ws_bytes = dense_verify_workspace_size(kv, Hq, G1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_verify_app(ctypes.byref(kv.desc), B, Hq, G1, q.data_ptr(), k_block.data_ptr(), v_block.data_ptr(), sc,
                       out.data_ptr(), _ptr(page_scores), workspace.data_ptr(), workspace.numel(), _stream()),
           "s3r_dense_verify_attn_append")
    return out, page_scores


def s3r_dense_verify_attn_head_scores(kv: KVCache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
                                      head_page_scores: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                                      workspace: Optional[torch.Tensor] = None
                                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """q [B][G1][Hq][D] -> (out [B][G1][Hq][D], head_page_scores [B][Hkv][max_pages] float32)."""
    _need(q, "q", kv.dtype)
    B, G1, Hq, D = q.shape
    if B != kv.num_seqs or D != kv.head_dim:
        raise ValueError("q must be [B][G1][Hq][D] matching the cache")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    if head_page_scores is None:
        head_page_scores = torch.empty((B, kv.num_kv_heads, kv.max_pages), dtype=torch.float32, device=q.device)
    _need(head_page_scores, "head_page_scores", torch.float32)
    if tuple(head_page_scores.shape) != (B, kv.num_kv_heads, kv.max_pages):
        raise ValueError("head_page_scores must be [B][Hkv][max_pages]")
    ws_bytes = dense_verify_workspace_size(kv, Hq, G1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_verify_head(ctypes.byref(kv.desc), B, Hq, G1, q.data_ptr(), sc, out.data_ptr(), head_page_scores.data_ptr(),
                        workspace.data_ptr(), workspace.numel(), _stream()), "s3r_dense_verify_attn_head_scores")
    return out, head_page_scores


def s3r_sparse_draft_attn_head_sel(kv: KVCache, q: torch.Tensor, sel_pages: torch.Tensor, num_sel: torch.Tensor,
                                   draft_step: int, out: Optional[torch.Tensor] = None,
                                   scale: Optional[float] = None) -> torch.Tensor:
    """q [B][Hq][D], sel_pages [B][Hkv][max_sel], num_sel [B][Hkv] -> out [B][Hq][D]."""
    _need(q, "q", kv.dtype)
    _need(sel_pages, "sel_pages", torch.int32)
    _need(num_sel, "num_sel", torch.int32)
    B, Hq, D = q.shape
    if sel_pages.dim() != 3 or tuple(sel_pages.shape[:2]) != (B, kv.num_kv_heads):
        raise ValueError("sel_pages must be [B][Hkv][max_sel]")
    if tuple(num_sel.shape) != (B, kv.num_kv_heads):
        raise ValueError("num_sel must be [B][Hkv]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_draft_head(ctypes.byref(kv.desc), B, Hq, int(draft_step), q.data_ptr(), sc, sel_pages.data_ptr(),
                       num_sel.data_ptr(), sel_pages.shape[2], out.data_ptr(), None, 0, _stream()),
           "s3r_sparse_draft_attn_head_sel")
    return out


def s3r_select_budget(page_scores: torch.Tensor, ctx_lens: torch.Tensor, budget, max_sel: int,
                      sel_pages: Optional[torch.Tensor] = None, num_sel: Optional[torch.Tensor] = None,
                      page_size: int = PAGE_SIZE, max_budget: Optional[float] = None
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """page_scores [B][max_pages] -> (sel_pages [B][max_sel] int32, num_sel [B] int32).
    budget: a float for every row, or a float64 GPU tensor [B] of one budget per row
    (s3r_select_budget_rows), each lowered to max_budget (default: the tensor's
    largest value, read back to the host)."""
    _need(page_scores, "page_scores", torch.float32)
    _need(ctx_lens, "ctx_lens", torch.int32)
    B, MP = page_scores.shape
    if sel_pages is None:
        sel_pages = torch.empty((B, max_sel), dtype=torch.int32, device=page_scores.device)
    if num_sel is None:
        num_sel = torch.empty((B,), dtype=torch.int32, device=page_scores.device)
    _need(sel_pages, "sel_pages", torch.int32)
    _need(num_sel, "num_sel", torch.int32)
    if isinstance(budget, torch.Tensor):
        _need(budget, "budget", torch.float64)
        if tuple(budget.shape) != (B,):
            raise ValueError("a per-row budget must be [B]")
        mb = float(budget.max()) if max_budget is None else float(max_budget)
        _check(_select_rows(page_scores.data_ptr(), ctx_lens.data_ptr(), B, MP, page_size, budget.data_ptr(), mb,
                            sel_pages.data_ptr(), num_sel.data_ptr(), sel_pages.shape[1], None, 0, _stream()),
               "s3r_select_budget_rows")
        return sel_pages, num_sel
    _check(_select(page_scores.data_ptr(), ctx_lens.data_ptr(), B, MP, page_size, float(budget),
                   sel_pages.data_ptr(), num_sel.data_ptr(), sel_pages.shape[1], None, 0, _stream()),
           "s3r_select_budget")
    return sel_pages, num_sel


def s3r_sparse_draft_attn(kv: KVCache, q: torch.Tensor, sel_pages: torch.Tensor, num_sel: torch.Tensor,
                          draft_step: int, out: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None) -> torch.Tensor:
    """q [B][Hq][D] of draft step j (1-based) -> out [B][Hq][D]."""
    _need(q, "q", kv.dtype)
    _need(sel_pages, "sel_pages", torch.int32)
    _need(num_sel, "num_sel", torch.int32)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_draft(ctypes.byref(kv.desc), B, Hq, int(draft_step), q.data_ptr(), sc, sel_pages.data_ptr(),
                  num_sel.data_ptr(), sel_pages.shape[1], out.data_ptr(), None, 0, _stream()),
           "s3r_sparse_draft_attn")
    return out


def s3r_sparse_draft_attn_append(kv: KVCache, q: torch.Tensor, k_row: torch.Tensor, v_row: torch.Tensor,
                                 sel_pages: torch.Tensor, num_sel: torch.Tensor, draft_step: int,
                                 out: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> torch.Tensor:
    """Writes k_row/v_row ([B][Hkv][D], or [B][1][Hkv][D]) at ctx_lens[b] + draft_step - 1,
    then as s3r_sparse_draft_attn: q [B][Hq][D] -> out [B][Hq][D]."""
    _need(q, "q", kv.dtype)
    _need(k_row, "k_row", kv.dtype)
    _need(v_row, "v_row", kv.dtype)
    _need(sel_pages, "sel_pages", torch.int32)
    _need(num_sel, "num_sel", torch.int32)
    B, Hq, D = q.shape
    if k_row.numel() != B * kv.num_kv_heads * D or v_row.shape != k_row.shape:
        raise ValueError("k_row/v_row must hold [B][Hkv][D]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_draft_app(ctypes.byref(kv.desc), B, Hq, int(draft_step), q.data_ptr(), k_row.data_ptr(),
                      v_row.data_ptr(), sc, sel_pages.data_ptr(), num_sel.data_ptr(), sel_pages.shape[1],
                      out.data_ptr(), None, 0, _stream()), "s3r_sparse_draft_attn_append")
    return out


def s3r_sparse_draft_attn_rows(kv: KVCache, q: torch.Tensor, k_rows: torch.Tensor, v_rows: torch.Tensor,
                               sel_pages: torch.Tensor, num_sel: torch.Tensor, draft_step: int,
                               out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                               horizons: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Draft step j (1-based) reading the in-flight draft tokens' rows from k_rows/v_rows
    ([>= j][B][Hkv][D] views; row r is position ctx_lens[b] + r) instead of the cache, which
    is read only below ctx_lens[b] and not written. The row and sequence dimensions may
    have any strides (e.g. a permuted [B][rows][Hkv][D] buffer); Hkv and D must be
    contiguous. sel_pages [B][max_sel] with num_sel [B], or [B][Hkv][max_sel] with
    num_sel [B][Hkv] (a page set per kv head). q [B][Hq][D] -> out [B][Hq][D].
    horizons (int32 [B], s3r_sparse_draft_attn_ragged): sequences with draft_step >
    horizons[b] are skipped and their out rows left as they were."""
    _need(q, "q", kv.dtype)
    _need(sel_pages, "sel_pages", torch.int32)
    _need(num_sel, "num_sel", torch.int32)
    B, Hq, D = q.shape
    for t, name in ((k_rows, "k_rows"), (v_rows, "v_rows")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != kv.dtype:
            raise ValueError(f"{name} must be a GPU tensor of the cache dtype")
        if t.dim() != 4 or t.stride(3) != 1 or t.stride(2) != D:
            raise ValueError(f"{name} must be a [rows][B][Hkv][D] view with Hkv and D contiguous")
    if (tuple(k_rows.shape[1:]) != (B, kv.num_kv_heads, D) or k_rows.shape[0] < int(draft_step)
            or v_rows.shape != k_rows.shape or v_rows.stride() != k_rows.stride()):
        raise ValueError("k_rows/v_rows must be [>= draft_step][B][Hkv][D] views with equal strides")
    per_head = sel_pages.dim() == 3
    if per_head:
        if tuple(sel_pages.shape[:2]) != (B, kv.num_kv_heads) or tuple(num_sel.shape) != (B, kv.num_kv_heads):
            raise ValueError("per-kv-head sel_pages/num_sel must be [B][Hkv][max_sel] and [B][Hkv]")
    elif sel_pages.dim() != 2 or sel_pages.shape[0] != B or tuple(num_sel.shape) != (B,):
        raise ValueError("sel_pages/num_sel must be [B][max_sel] and [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", kv.dtype)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if horizons is not None:
        _need_horizons(horizons, B)
        _check(_draft_ragged(ctypes.byref(kv.desc), B, Hq, int(draft_step), q.data_ptr(), k_rows.data_ptr(),
                             v_rows.data_ptr(), k_rows.stride(0), k_rows.stride(1), sc, sel_pages.data_ptr(),
                             num_sel.data_ptr(), sel_pages.shape[-1], 1 if per_head else 0, horizons.data_ptr(),
                             out.data_ptr(), None, 0, _stream()), "s3r_sparse_draft_attn_ragged")
        return out
    _check(_draft_rows(ctypes.byref(kv.desc), B, Hq, int(draft_step), q.data_ptr(), k_rows.data_ptr(),
                       v_rows.data_ptr(), k_rows.stride(0), k_rows.stride(1), sc, sel_pages.data_ptr(),
                       num_sel.data_ptr(), sel_pages.shape[-1], 1 if per_head else 0, out.data_ptr(), None, 0,
                       _stream()), "s3r_sparse_draft_attn_rows")
    return out


def spec_accept_workspace_size(num_seqs: int, gamma: int, vocab: int) -> int:
    return int(_accept_ws(num_seqs, gamma, vocab))


def s3r_spec_accept(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_tokens: torch.Tensor,
                    u_accept: torch.Tensor, u_sample: torch.Tensor, temperature: float = 1.0,
                    ctx_lens: Optional[torch.Tensor] = None, num_accepted: Optional[torch.Tensor] = None,
                    out_tokens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    horizons: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """-> (num_accepted [B] int32, out_tokens [B][gamma+1] int32); ctx_lens (if given) += a + 1.
    horizons (int32 [B], s3r_spec_accept_ragged): sequence b tests only its first
    horizons[b] drafts (bonus from target row horizons[b])."""
    _need(target_logits, "target_logits", (torch.bfloat16, torch.float32))
    _need(draft_logits, "draft_logits", target_logits.dtype)
    _need(draft_tokens, "draft_tokens", torch.int32)
    _need(u_accept, "u_accept", torch.float32)
    _need(u_sample, "u_sample", torch.float32)
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V) or tuple(draft_tokens.shape) != (B, gamma):
        raise ValueError("draft_logits must be [B][gamma][V] and draft_tokens [B][gamma]")
    if tuple(u_accept.shape) != (B, gamma) or tuple(u_sample.shape) != (B,):
        raise ValueError("u_accept must be [B][gamma] and u_sample [B]")
    dev = target_logits.device
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G1), dtype=torch.int32, device=dev)
    if ctx_lens is not None:
        _need(ctx_lens, "ctx_lens", torch.int32)
    ws_bytes = spec_accept_workspace_size(B, gamma, V)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if horizons is not None:
        _need_horizons(horizons, B)
        _check(_accept_ragged(B, gamma, V, _dtype_code(target_logits.dtype), target_logits.data_ptr(),
                              draft_logits.data_ptr(), draft_tokens.data_ptr(), u_accept.data_ptr(),
                              u_sample.data_ptr(), horizons.data_ptr(), float(temperature), num_accepted.data_ptr(),
                              out_tokens.data_ptr(), _ptr(ctx_lens), workspace.data_ptr(), workspace.numel(),
                              _stream()), "s3r_spec_accept_ragged")
        return num_accepted, out_tokens
    _check(_accept(B, gamma, V, _dtype_code(target_logits.dtype), target_logits.data_ptr(), draft_logits.data_ptr(),
                   draft_tokens.data_ptr(), u_accept.data_ptr(), u_sample.data_ptr(), float(temperature),
                   num_accepted.data_ptr(), out_tokens.data_ptr(), _ptr(ctx_lens), workspace.data_ptr(),
                   workspace.numel(), _stream()), "s3r_spec_accept")
    return num_accepted, out_tokens


def s3r_spec_accept_no_alloc(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_tokens: torch.Tensor,
                             u_accept: torch.Tensor, u_sample: torch.Tensor, num_accepted: torch.Tensor,
                             out_tokens: torch.Tensor, temperature: float = 1.0,
                             ctx_lens: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """s3r_spec_accept on the library's static per-GPU workspace, for callers that
    cannot allocate: the outputs are the caller's, and neither this wrapper nor
    the library allocates. Calls that overlap on one GPU race."""
    _need(target_logits, "target_logits", (torch.bfloat16, torch.float32))
    _need(draft_logits, "draft_logits", target_logits.dtype)
    _need(draft_tokens, "draft_tokens", torch.int32)
    _need(u_accept, "u_accept", torch.float32)
    _need(u_sample, "u_sample", torch.float32)
    _need(num_accepted, "num_accepted", torch.int32)
    _need(out_tokens, "out_tokens", torch.int32)
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V) or tuple(draft_tokens.shape) != (B, gamma):
        raise ValueError("draft_logits must be [B][gamma][V] and draft_tokens [B][gamma]")
    if tuple(u_accept.shape) != (B, gamma) or tuple(u_sample.shape) != (B,):
        raise ValueError("u_accept must be [B][gamma] and u_sample [B]")
    if tuple(num_accepted.shape) != (B,) or tuple(out_tokens.shape) != (B, G1):
        raise ValueError("num_accepted must be [B] and out_tokens [B][gamma+1]")
    if ctx_lens is not None:
        _need(ctx_lens, "ctx_lens", torch.int32)
    _check(_accept_no_alloc(B, gamma, V, _dtype_code(target_logits.dtype), target_logits.data_ptr(),
                            draft_logits.data_ptr(), draft_tokens.data_ptr(), u_accept.data_ptr(), u_sample.data_ptr(),
                            float(temperature), num_accepted.data_ptr(), out_tokens.data_ptr(), _ptr(ctx_lens),
                            _stream()), "s3r_spec_accept_no_alloc")
    return num_accepted, out_tokens


def page_bytes(kv: KVCache) -> int:
    """Bytes of one page (K and V tiles of every kv head) in a staging buffer."""
    return int(_page_bytes(ctypes.byref(kv.desc)))


def s3r_pack_pages(kv: KVCache, blocks: torch.Tensor, staging: Optional[torch.Tensor] = None) -> torch.Tensor:
    """blocks int32 [n] (device) -> staging uint8 [n][page_bytes]: the pages' K and V tiles."""
    _need(blocks, "blocks", torch.int32)
    n = blocks.numel()
    if staging is None:
        staging = torch.empty((n, page_bytes(kv)), dtype=torch.uint8, device=blocks.device)
    _need(staging, "staging", torch.uint8)
    if staging.numel() < n * page_bytes(kv):
        raise ValueError("staging holds fewer than n pages")
    _check(_pack(ctypes.byref(kv.desc), blocks.data_ptr(), n, staging.data_ptr(), _stream()), "s3r_pack_pages")
    return staging


def s3r_unpack_pages(kv: KVCache, blocks: torch.Tensor, staging: torch.Tensor) -> None:
    """staging uint8 [n][page_bytes] -> the blocks int32 [n] of the cache."""
    _need(blocks, "blocks", torch.int32)
    _need(staging, "staging", torch.uint8)
    n = blocks.numel()
    if staging.numel() < n * page_bytes(kv):
        raise ValueError("staging holds fewer than n pages")
    _check(_unpack(ctypes.byref(kv.desc), blocks.data_ptr(), n, staging.data_ptr(), _stream()), "s3r_unpack_pages")


# bits of s3r_check_step_inputs' per-sequence error word
CHECK_BITS = {1: "ctx_len", 2: "page_id", 4: "num_sel", 8: "sel_range", 16: "sel_duplicate", 32: "draft_token",
              64: "nonfinite_slot"}


def s3r_check_step_inputs(kv: KVCache, block_len: int, sel_pages: Optional[torch.Tensor] = None,
                          num_sel: Optional[torch.Tensor] = None, draft_tokens: Optional[torch.Tensor] = None,
                          vocab: int = 0, errors: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device-input checks of a step: -> errors int32 [B], bits as CHECK_BITS (0: all
    well). sel_pages [B][max_sel] with num_sel [B], or [B][Hkv][max_sel] with [B][Hkv];
    draft_tokens [B][gamma] with the vocabulary size."""
    B = kv.num_seqs
    per_head = False
    max_sel = 0
    if sel_pages is not None:
        _need(sel_pages, "sel_pages", torch.int32)
        _need(num_sel, "num_sel", torch.int32)
        per_head = sel_pages.dim() == 3
        max_sel = sel_pages.shape[-1]
    gamma = 0
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", torch.int32)
        gamma = draft_tokens.shape[1]
    if errors is None:
        errors = torch.empty((B,), dtype=torch.int32, device=kv.k_cache.device)
    _need(errors, "errors", torch.int32)
    _check(_check_inputs(ctypes.byref(kv.desc), B, int(block_len), _ptr(sel_pages), _ptr(num_sel), max_sel,
                         1 if per_head else 0, _ptr(draft_tokens), gamma, int(vocab), errors.data_ptr(), _stream()),
           "s3r_check_step_inputs")
    return errors


def describe_check(errors: torch.Tensor) -> Dict[int, List[str]]:
    """{sequence: [problem names]} for the sequences with a non-zero error word."""
    e = errors.cpu().tolist()
    return {b: [n for bit, n in CHECK_BITS.items() if v & bit] for b, v in enumerate(e) if v}


# raw entry points, for host-side validation tests that pass NULL pointers
raw = {
    "s3r_append_kv": _append, "s3r_dense_verify_attn": _verify, "s3r_dense_verify_workspace_size": _verify_ws,
    "s3r_select_budget": _select, "s3r_sparse_draft_attn": _draft, "s3r_spec_accept": _accept,
    "s3r_spec_accept_workspace_size": _accept_ws, "s3r_status_string": _status_string, "s3r_version": _version,
    "s3r_dense_verify_attn_append": _verify_app, "s3r_sparse_draft_attn_append": _draft_app,
    "s3r_dense_verify_attn_head_scores": _verify_head, "s3r_sparse_draft_attn_head_sel": _draft_head,
    "s3r_sparse_draft_attn_rows": _draft_rows, "s3r_select_budget_rows": _select_rows,
    "s3r_dense_verify_attn_ragged": _verify_ragged, "s3r_sparse_draft_attn_ragged": _draft_ragged,
    "s3r_spec_accept_ragged": _accept_ragged, "s3r_check_step_inputs": _check_inputs,
    "s3r_page_bytes": _page_bytes, "s3r_pack_pages": _pack, "s3r_unpack_pages": _unpack,
    "s3r_select_budget_workspace_size": _select_ws, "s3r_sparse_draft_workspace_size": _draft_ws,
    "s3r_spec_accept_no_alloc": _accept_no_alloc,
}
