"""The C-ABI library loads and exports every symbol include/s3r.h declares, and
host-side validation rejects bad arguments before any launch. No GPU: every call
here fails validation (or is a pure host query) and never reaches the runtime."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s3r.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s3r_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def s3r():
    from rl_rollout_amd import s3r as mod
    return mod


def test_header_declares_the_four_hot_path_calls():
    syms = declared_symbols()
    for name in ("s3r_select_budget", "s3r_sparse_draft_attn", "s3r_dense_verify_attn", "s3r_spec_accept"):
        assert name in syms


def test_library_exports_every_declared_symbol(s3r):
    out = subprocess.run(["nm", "-D", "--defined-only", s3r.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (s3r_\w+)", out.stdout))
    missing = [s for s in declared_symbols() if s not in exported]
    assert not missing, missing
    for s in declared_symbols():
        getattr(ctypes.CDLL(s3r.LIB_PATH), s)


def test_status_strings_and_version(s3r):
    assert s3r.status_string(0) == "success"
    assert s3r.status_string(3) == "insufficient workspace"
    assert s3r.status_string(99) == "unknown status"
    assert s3r.version() >= 100


def _kv(s3r, **kw):
    f = dict(k_cache=256, v_cache=256, page_table=1, ctx_lens=1, num_blocks=10, num_kv_heads=8, page_size=16,
             head_dim=128, max_pages_per_seq=100, dtype=1)
    f.update(kw)
    return s3r.PagedKV(**f)


INV, NSUP, WS = 1, 2, 3


@pytest.mark.parametrize("field,value,expect", [
    ("k_cache", None, INV), ("page_table", None, INV), ("ctx_lens", None, INV),
    ("num_blocks", 0, INV), ("num_kv_heads", 0, INV), ("dtype", 7, INV),
    ("page_size", 32, NSUP), ("head_dim", 96, NSUP), ("max_pages_per_seq", 0, INV),
])
def test_verify_rejects_bad_cache(s3r, field, value, expect):
    kv = _kv(s3r, **{field: value})
    st = s3r.raw["s3r_dense_verify_attn"](ctypes.byref(kv), 4, 16, 5, 1, 0.1, 1, None, 1, 1 << 40, None)
    assert st == expect


def test_verify_argument_checks(s3r):
    f = s3r.raw["s3r_dense_verify_attn"]
    kv = _kv(s3r)
    big = 1 << 40
    assert f(None, 4, 16, 5, 1, 0.1, 1, None, 1, big, None) == INV
    assert f(ctypes.byref(kv), 0, 16, 5, 1, 0.1, 1, None, 1, big, None) == INV        # no sequences
    assert f(ctypes.byref(kv), 4, 12, 5, 1, 0.1, 1, None, 1, big, None) == INV        # 12 % 8 != 0
    assert f(ctypes.byref(kv), 4, 16, 0, 1, 0.1, 1, None, 1, big, None) == INV        # empty block
    assert f(ctypes.byref(kv), 4, 16, 5, None, 0.1, 1, None, 1, big, None) == INV     # q NULL
    assert f(ctypes.byref(kv), 4, 16, 5, 1, 0.1, None, None, 1, big, None) == INV     # out NULL
    assert f(ctypes.byref(kv), 4, 16, 5, 1, float("nan"), 1, None, 1, big, None) == INV
    assert f(ctypes.byref(kv), 4, 16, 5, 1, -1.0, 1, None, 1, big, None) == INV
    assert f(ctypes.byref(kv), 4, 64, 5, 1, 0.1, 1, None, 1, big, None) == NSUP       # 5 * 8 rows > 32
    need = s3r.raw["s3r_dense_verify_workspace_size"](ctypes.byref(kv), 4, 16, 5)
    assert need > 0
    assert f(ctypes.byref(kv), 4, 16, 5, 256, 0.1, 1, None, 1, need - 1, None) == WS
    assert f(ctypes.byref(kv), 4, 16, 5, 256, 0.1, 1, None, None, need, None) == WS
    assert f(ctypes.byref(kv), 4, 16, 5, 8, 0.1, 1, None, 1, need, None) == INV         # q not 16-byte aligned
    kv_mis = _kv(s3r, k_cache=264)
    assert f(ctypes.byref(kv_mis), 4, 16, 5, 256, 0.1, 1, None, 1, need, None) == INV  # cache not aligned
    assert s3r.raw["s3r_dense_verify_workspace_size"](ctypes.byref(kv), 4, 12, 5) == 0


def test_select_argument_checks(s3r):
    f = s3r.raw["s3r_select_budget"]
    ok = dict(scores=1, lens=1, B=4, mp=100, P=16, s=0.05, sel=1, ns=1, max_sel=8)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["scores"], a["lens"], a["B"], a["mp"], a["P"], a["s"], a["sel"], a["ns"], a["max_sel"], None, 0,
                 None)

    assert call(scores=None) == INV
    assert call(sel=None) == INV
    assert call(B=0) == INV
    assert call(max_sel=0) == INV
    assert call(s=0.0) == INV
    assert call(s=1.5) == INV
    assert call(s=float("inf")) == INV
    assert call(P=8) == NSUP
    assert call(mp=32769, max_sel=32769) == NSUP       # more candidate pages than the LDS staging holds
    # max_sel must hold the largest selection: 0.1 of 1000 pages keeps 100
    assert call(mp=1000, s=0.1, max_sel=99) == INV
    assert call(mp=20000, max_sel=999) == INV          # 0.05 of 20000 keeps 1000
    assert call(mp=1024, s=0.05, max_sel=51) == INV    # 51.2 rounds up to 52


def test_draft_argument_checks(s3r):
    f = s3r.raw["s3r_sparse_draft_attn"]
    kv = _kv(s3r)
    assert f(ctypes.byref(kv), 4, 16, 0, 1, 0.1, 1, 1, 8, 1, None, 0, None) == INV    # step 0
    assert f(ctypes.byref(kv), 4, 16, 1, 1, 0.1, None, 1, 8, 1, None, 0, None) == INV  # sel NULL
    assert f(ctypes.byref(kv), 4, 16, 1, 1, 0.1, 1, 1, 0, 1, None, 0, None) == INV     # max_sel 0
    assert f(ctypes.byref(kv), 4, 48, 1, 256, 0.1, 1, 1, 8, 1, None, 0, None) == NSUP    # group 6
    assert f(ctypes.byref(kv), 4, 16, 1, 8, 0.1, 1, 1, 8, 1, None, 0, None) == INV       # q misaligned
    kv96 = _kv(s3r, head_dim=96)
    assert f(ctypes.byref(kv96), 4, 16, 1, 256, 0.1, 1, 1, 8, 1, None, 0, None) == NSUP


def test_accept_argument_checks(s3r):
    f = s3r.raw["s3r_spec_accept"]
    need = s3r.spec_accept_workspace_size(4, 3, 1000)
    assert need > 0

    def call(B=4, g=3, V=1000, dt=1, tl=256, dl=256, T=1.0, ws=1, wsb=None):
        return f(B, g, V, dt, tl, dl, 1, 1, 1, T, 1, 1, None, ws, need if wsb is None else wsb, None)

    assert call(B=0) == INV
    assert call(g=0) == INV
    assert call(dt=5) == INV
    assert call(tl=None) == INV
    assert call(T=0.0) == INV
    assert call(T=float("nan")) == INV
    assert call(dl=258) == INV           # logits not 16-byte aligned
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert s3r.spec_accept_workspace_size(0, 3, 10) == 0


def test_append_argument_checks(s3r):
    f = s3r.raw["s3r_append_kv"]
    kv = _kv(s3r)
    assert f(ctypes.byref(kv), 4, 0, 0, 1, 1, None) == INV
    assert f(ctypes.byref(kv), 4, -1, 1, 1, 1, None) == INV
    assert f(ctypes.byref(kv), 4, 0, 1, None, 1, None) == INV


def test_fused_append_entry_points_reject_missing_rows_and_share_the_checks(s3r):
    fv = s3r.raw["s3r_dense_verify_attn_append"]
    fd = s3r.raw["s3r_sparse_draft_attn_append"]
    kv = _kv(s3r)
    # verify: kv, B, Hq, G1, q, k_block, v_block, scale, out, scores, ws, bytes, stream
    assert fv(ctypes.byref(kv), 4, 16, 5, 256, None, 256, 0.1, 1, None, 1, 1 << 40, None) == INV
    assert fv(ctypes.byref(kv), 4, 16, 5, 256, 256, None, 0.1, 1, None, 1, 1 << 40, None) == INV
    assert fv(ctypes.byref(kv), 4, 16, 5, 256, 256, 256, 0.1, 1, None, 1, 0, None) == WS
    assert fv(ctypes.byref(_kv(s3r, head_dim=96)), 4, 16, 5, 256, 256, 256, 0.1, 1, None, 1, 1 << 40, None) == NSUP
    # draft: kv, B, Hq, step, q, k_row, v_row, scale, sel, nsel, max_sel, out, ws, bytes, stream
    assert fd(ctypes.byref(kv), 4, 16, 1, 256, None, 256, 0.1, 1, 1, 8, 1, None, 0, None) == INV
    assert fd(ctypes.byref(kv), 4, 16, 0, 256, 256, 256, 0.1, 1, 1, 8, 1, None, 0, None) == INV
    assert fd(ctypes.byref(kv), 4, 48, 1, 256, 256, 256, 0.1, 1, 1, 8, 1, None, 0, None) == NSUP


def test_draft_rows_entry_point_checks(s3r):
    f = s3r.raw["s3r_sparse_draft_attn_rows"]
    kv = _kv(s3r)
    rs, ss = 4 * 8 * 128, 8 * 128  # [rows][B][Hkv][D] strides of the bf16 test cache

    # kv, B, Hq, step, q, k_rows, v_rows, row_stride, seq_stride, scale, sel, nsel, max_sel, per_head, out,
    # ws, bytes, stream
    def call(Hq=16, step=1, kr=256, vr=256, r=rs, s_=ss, flag=0):
        return f(ctypes.byref(kv), 4, Hq, step, 256, kr, vr, r, s_, 0.1, 1, 1, 8, flag, 1, None, 0, None)

    assert call(kr=None) == INV          # k_rows NULL
    assert call(vr=None) == INV          # v_rows NULL
    assert call(kr=264) == INV           # misaligned
    assert call(flag=2) == INV
    assert call(step=0) == INV
    assert call(r=-8) == INV             # negative stride
    assert call(s_=4) == INV             # 8 bytes: not a multiple of 16
    assert call(Hq=48) == NSUP           # group 6


def test_select_rows_entry_point_checks(s3r):
    f = s3r.raw["s3r_select_budget_rows"]
    # scores, lens, B, max_pages, page_size, budgets, max_budget, sel, nsel, max_sel, ws, bytes, stream
    assert f(1, 1, 4, 100, 16, None, 0.05, 1, 1, 8, None, 0, None) == INV     # budgets NULL
    assert f(1, 1, 0, 100, 16, 1, 0.05, 1, 1, 8, None, 0, None) == INV        # no rows
    assert f(1, 1, 4, 100, 16, 1, 0.05, 1, 1, 0, None, 0, None) == INV        # max_sel 0
    assert f(1, 1, 4, 100, 8, 1, 0.05, 1, 1, 8, None, 0, None) == NSUP        # page size 8
    assert f(1, 1, 4, 100, 16, 1, 0.0, 1, 1, 8, None, 0, None) == INV         # max_budget not in (0, 1]
    assert f(1, 1, 4, 100, 16, 1, 1.5, 1, 1, 200, None, 0, None) == INV
    assert f(1, 1, 4, 100, 16, 1, float("nan"), 1, 1, 8, None, 0, None) == INV
    # max_sel must hold a row at max_budget: 0.1 of 1000 pages keeps 100 (a float32
    # 0.1 would keep 101)
    assert f(1, 1, 4, 1000, 16, 1, 0.1, 1, 1, 99, None, 0, None) == INV
    assert f(1, 1, 4, 32769, 16, 1, 0.1, 1, 1, 4000, None, 0, None) == NSUP


def test_ragged_entry_point_checks(s3r):
    """The entry points with a draft horizon per sequence reject a NULL horizons
    array and otherwise validate as their uniform counterparts (no launch here)."""
    kv = _kv(s3r)
    fv = s3r.raw["s3r_dense_verify_attn_ragged"]
    # kv, B, Hq, G1, q, horizons, scale, out, scores, ws, bytes, stream
    assert fv(ctypes.byref(kv), 4, 16, 5, 256, None, 0.1, 256, 256, 256, 1 << 30, None) == INV
    assert fv(ctypes.byref(kv), 4, 16, 5, None, 256, 0.1, 256, 256, 256, 1 << 30, None) == INV   # q NULL
    assert fv(ctypes.byref(kv), 4, 16, 0, 256, 256, 0.1, 256, 256, 256, 1 << 30, None) == INV    # empty block
    fd = s3r.raw["s3r_sparse_draft_attn_ragged"]
    rs, ss = 4 * 8 * 128, 8 * 128

    # kv, B, Hq, step, q, k_rows, v_rows, row_stride, seq_stride, scale, sel, nsel, max_sel, per_head, horizons,
    # out, ws, bytes, stream
    def draft(hz=256, kr=256, step=1, Hq=16):
        return fd(ctypes.byref(kv), 4, Hq, step, 256, kr, 256, rs, ss, 0.1, 1, 1, 8, 0, hz, 1, None, 0, None)

    assert draft(hz=None) == INV
    assert draft(kr=None) == INV
    assert draft(step=0) == INV
    assert draft(Hq=48) == NSUP
    fa = s3r.raw["s3r_spec_accept_ragged"]
    # B, gamma, V, dtype, tl, dl, dt, ua, us, horizons, T, nacc, out, ctx, ws, bytes, stream
    assert fa(4, 3, 100, 1, 256, 256, 1, 1, 1, None, 1.0, 1, 1, None, 256, 1 << 20, None) == INV
    assert fa(4, 0, 100, 1, 256, 256, 1, 1, 1, 1, 1.0, 1, 1, None, 256, 1 << 20, None) == INV     # gamma 0
    assert fa(4, 3, 100, 1, 256, 256, 1, 1, 1, 1, 0.0, 1, 1, None, 256, 1 << 20, None) == INV     # T = 0
    assert fa(4, 3, 100, 1, 256, 256, 1, 1, 1, 1, 1.0, 1, 1, None, 256, 0, None) == WS


def test_check_step_inputs_entry_point_checks(s3r):
    f = s3r.raw["s3r_check_step_inputs"]
    kv = _kv(s3r)

    # kv, B, block_len, sel, nsel, max_sel, per_head, tokens, gamma, vocab, errors, stream
    def call(B=4, blk=5, sel=1, nsel=1, ms=8, flag=0, tok=None, g=0, V=0, err=1):
        return f(ctypes.byref(kv), B, blk, sel, nsel, ms, flag, tok, g, V, err, None)

    assert call(err=None) == INV            # no error array
    assert call(B=0) == INV
    assert call(blk=0) == INV
    assert call(blk=1 << 30) == INV         # block beyond the page table
    assert call(nsel=None) == INV           # selection without counts
    assert call(sel=None) == INV            # counts without selection
    assert call(ms=0) == INV
    assert call(flag=2) == INV
    assert call(tok=1, g=0, V=10) == INV    # tokens without gamma
    assert call(tok=1, g=4, V=0) == INV     # tokens without a vocabulary


def test_page_copy_entry_point_checks(s3r):
    kv = _kv(s3r)
    # bf16, 8 kv heads, head_dim 128: K and V runs of 8 * 16 * 128 * 2 bytes each
    assert s3r.raw["s3r_page_bytes"](ctypes.byref(kv)) == 2 * 8 * 16 * 128 * 2
    assert s3r.raw["s3r_page_bytes"](None) == 0
    for name in ("s3r_pack_pages", "s3r_unpack_pages"):
        f = s3r.raw[name]
        # kv, blocks, n, staging, stream
        assert f(ctypes.byref(kv), None, 4, 256, None) == INV      # blocks NULL
        assert f(ctypes.byref(kv), 256, 4, None, None) == INV      # staging NULL
        assert f(ctypes.byref(kv), 256, 0, 256, None) == INV       # no pages
        assert f(ctypes.byref(kv), 256, 4, 264, None) == INV       # misaligned staging
        assert f(None, 256, 4, 256, None) == INV


def test_every_op_has_a_workspace_size(s3r):
    kv = _kv(s3r)
    assert s3r.raw["s3r_select_budget_workspace_size"](4, 100) == 0
    assert s3r.raw["s3r_sparse_draft_workspace_size"](ctypes.byref(kv), 4, 16) == 0


def test_no_alloc_accept_checks(s3r):
    """The allocation-free accept validates as s3r_spec_accept, then rejects shapes
    whose workspace exceeds its static 4 MiB (no launch, no device query)."""
    f = s3r.raw["s3r_spec_accept_no_alloc"]

    # B, gamma, V, dtype, tl, dl, tokens, ua, us, T, num_accepted, out_tokens, ctx, stream
    def call(B=4, g=3, V=1000, dt=1, tl=256, dl=256, T=1.0, na=1):
        return f(B, g, V, dt, tl, dl, 1, 1, 1, T, na, 1, None, None)

    assert call(B=0) == INV
    assert call(dt=5) == INV
    assert call(tl=None) == INV
    assert call(na=None) == INV
    assert call(T=0.0) == INV
    assert call(dl=258) == INV
    assert s3r.spec_accept_workspace_size(5000, 8, 262144) > 4 << 20
    assert call(B=5000, g=8, V=262144) == WS
