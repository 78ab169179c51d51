"""The C ABI library loads and exports what include/qkv.h declares; host-side
configuration checks (CPU only: no call here touches a GPU)."""
import ctypes
import os
import re

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from tiered_quantization_eviction_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from tiered_quantization_eviction_amd import build
        build.build()
    return L, L.lib()


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(qkv_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("qkv_append", "qkv_decode_attend", "qkv_route", "qkv_quantize_window", "qkv_create",
                 "qkv_destroy", "qkv_rank_tiers", "qkv_export", "qkv_workspace_bytes"):
        assert must in names


def test_library_exports_every_declared_symbol():
    _, lib = _lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_config_checks_on_host():
    L, lib = _lib()
    for cfg in (W.TINY, W.DRIFT, W.STRESS):
        c = L.make_config(cfg)
        assert lib.qkv_check_config(ctypes.byref(c)) == 0, cfg.name
        assert L.workspace_bytes(c) > 0
    bad = [dict(n_q_heads=12, n_kv_heads=4),     # G = 3
           dict(head_dim=96),
           dict(window=12),
           dict(n_sink=17),
           dict(quant_bits=3),
           dict(max_ctx=0)]
    for kw in bad:
        c = L.make_config(W.TINY, **kw) if "max_ctx" not in kw else L.make_config(W.TINY, max_ctx=0)
        if "max_ctx" not in kw:
            for k, v in kw.items():
                setattr(c, k, v)
        assert lib.qkv_check_config(ctypes.byref(c)) == L.EINVAL, kw
        assert L.workspace_bytes(c) == 0
    # eight heads per KV head at d = 128: every window size; with rotary keys
    # the attention LDS does not fit
    for window, rope, ok in ((8, 0, True), (16, 0, True), (32, 0, True), (16, 1, False)):
        c = L.make_config(W.STRESS, max_ctx=65536)
        c.window, c.rope = window, rope
        assert (lib.qkv_check_config(ctypes.byref(c)) == 0) == ok, (window, rope)


def test_score_window_checks_on_host():
    """A rolling score window belongs to HqeKV and spans at most one period."""
    L, lib = _lib()
    for window, ok in ((0, True), (20, True), (64, True), (65, False), (-1, False)):
        c = L.make_config(W.HQEKV)
        c.score_window = window
        assert (lib.qkv_check_config(ctypes.byref(c)) == 0) == ok, window
    for cfg in (W.TINY, W.H2O):
        c = L.make_config(cfg)
        c.score_window = 1
        assert lib.qkv_check_config(ctypes.byref(c)) == L.EINVAL, cfg.name


def test_chunk_checks_on_host():
    """Chunk ranking belongs to HqeKV: chunks of 1 to 64 positions, at most
    4096 of them per (sequence, KV head)."""
    L, lib = _lib()
    for chunk, max_ctx, ok in ((0, 65792, True), (32, 65792, True), (64, 65792, True), (65, 65792, False),
                               (16, 65792, False), (16, 65536, True), (-1, 65792, False)):
        c = L.make_config(W.HQEKV, max_ctx=max_ctx)
        c.chunk = chunk
        assert (lib.qkv_check_config(ctypes.byref(c)) == 0) == ok, (chunk, max_ctx)
    c = L.make_config(W.TINY)
    c.chunk = 32
    assert lib.qkv_check_config(ctypes.byref(c)) == L.EINVAL


def test_plan_capacities_matches_the_oracle_budget_arithmetic():
    """QEvict notes 4.3 Eq.(3) through the library's planner against the
    oracle's capacity and payload arithmetic (itself pinned to the pages'
    100 MB example): Llama-3.1-8B geometry (32 layers, 8 KV heads, d = 128),
    several windows, budgets and splits q."""
    import math
    from oracle import budget
    L, lib = _lib()
    for window in (8, 16, 32):
        for q in (0.0, 0.3, 0.7, 1.0):
            for mb in (40.0, 100.0, 1000.0):
                c = L.make_config(W.DRIFT, window=window)
                layers = 32
                per_tok = budget.kv_bytes_per_token(layers, c.n_kv_heads, c.head_dim, 2)
                b_hist = mb * 2 ** 20 - (c.n_sink + c.n_recent) * per_tok
                m_full = window * per_tok
                m_quant = layers * c.n_kv_heads * budget.window_ledger_bytes(window, c.head_dim, 2, 32)
                want = budget.tier_capacities(b_hist, q, m_full, m_quant)
                got = L.plan_capacities(c, mb * 2 ** 20, q, layers)
                assert got == want, (window, q, mb, got, want)
    c = L.make_config(W.DRIFT)
    for bad in ((-1.0, 0.5, 1), (2 ** 30, 1.5, 1), (2 ** 30, 0.5, 0), (1000.0, 0.5, 1)):
        with pytest.raises(ValueError):
            L.plan_capacities(c, *bad)
    with pytest.raises(ValueError):
        L.plan_capacities(L.make_config(W.HQEKV), 2 ** 30, 0.5, 1)
    # the single-layer drift capacities at the bytes they occupy
    kf, kq = W.DRIFT.k_full, W.DRIFT.k_quant
    per_tok = budget.kv_bytes_per_token(1, 8, 128, 2)
    b = (5 + 64) * per_tok + kf * 16 * per_tok + kq * 8 * budget.window_ledger_bytes(16, 128, 2, 32)
    q = kq * 8 * budget.window_ledger_bytes(16, 128, 2, 32) / (b - (5 + 64) * per_tok)
    got = L.plan_capacities(c, b, q, 1)
    assert abs(got[0] - kf) <= 1 and abs(got[1] - kq) <= 1, got
    assert math.isfinite(q)


def test_strerror_and_info_arguments():
    L, lib = _lib()
    assert lib.qkv_strerror(L.ERANGE).decode().startswith("quantization parameter")
    assert lib.qkv_create(None, None, 0, None, None) == L.EINVAL
    assert lib.qkv_append(None, None, None, 1, None) == L.EINVAL
    assert lib.qkv_route(None, None) == L.EINVAL


def test_workspace_holds_payload_of_config3():
    """Unit-indexed pages of the 32K x 16 workload and a ledger pool of
    K_f + K_q slots per sequence (only Full and Quantized windows hold codes);
    a 32-layer cache holds 32 layers' pages and one pool of 32 times the slots."""
    L, _ = _lib()
    c = L.make_config(W.DRIFT)
    U = 1 + -(-(W.DRIFT.total_tokens - 5) // 16)
    pages = 16 * U * 8 * 2 * 16 * 128 * 2
    slot = 8 * (512 + 512 + 512 + 256)
    ledger = 16 * (W.DRIFT.k_full + W.DRIFT.k_quant) * slot
    assert pages + ledger <= L.workspace_bytes(c) <= pages + ledger + 64 * 2 ** 20
    c32 = L.make_config(W.DRIFT.replace(prefill=4096, steps=64), n_layers=32)
    U32 = 1 + -(-(4096 + 64 - 5) // 16)
    pages32 = 32 * 16 * U32 * 8 * 2 * 16 * 128 * 2
    ledger32 = 32 * 16 * min(W.DRIFT.k_full + W.DRIFT.k_quant, U32) * slot
    assert pages32 + ledger32 <= L.workspace_bytes(c32) <= pages32 + ledger32 + 32 * 2 ** 20
    c.n_layers = 129
    assert L.workspace_bytes(c) == 0
    h = L.make_config(W.H2O, n_layers=2)
    assert L.workspace_bytes(h) == 0                 # layers belong to the window policy


def test_snapshot_and_ranking_arguments_checked_on_host():
    """qkv_import / qkv_export refuse a missing cache or buffer, and the
    stateless ranking refuses more entries than its LDS sort holds (8192),
    all before any device work (the pointers below are never dereferenced)."""
    L, lib = _lib()
    assert "qkv_import" in declared_functions()
    fake = ctypes.c_void_p(256)
    assert lib.qkv_import(None, 0, fake, 1, None) == L.EINVAL
    assert lib.qkv_export(None, 0, fake, 1, None) == L.EINVAL
    assert lib.qkv_export_bytes(None, 0) == 0
    assert lib.qkv_rank_tiers(fake, fake, fake, 8193, fake, 1, fake, None) == L.EINVAL
    assert lib.qkv_rank_tiers(fake, fake, fake, 0, fake, 1, fake, None) == L.EINVAL
    assert lib.qkv_rank_tiers(fake, fake, fake, 16, fake, 255, fake, None) == L.EINVAL


def test_binding_checks_dtype_and_shape():
    """The binding refuses tensors whose element size or shape the C call
    would read or write past (checked on host tensors: no GPU needed)."""
    import torch
    L, _ = _lib()
    L._check_tensor(torch.zeros((2, 3), dtype=torch.bfloat16), "x", (2, 3), "16")
    L._check_tensor(torch.zeros((2, 3), dtype=torch.int16), "x", (2, 3), "16")
    L._check_tensor(torch.zeros((2, 3), dtype=torch.float32), "x", (2, 3), "f32")
    for t, shape, kind in ((torch.zeros((2, 3), dtype=torch.float32), (2, 3), "16"),
                           (torch.zeros((2, 3), dtype=torch.bfloat16), (2, 3), "f32"),
                           (torch.zeros((2, 4), dtype=torch.int16), (2, 3), "16"),
                           (torch.zeros((3, 2), dtype=torch.float32), (2, 3), "f32")):
        with pytest.raises(ValueError):
            L._check_tensor(t, "x", shape, kind)


def test_rope_config_checks_on_host():
    """Keys before the rotary embedding: the window policy with windows of at
    most one 16-token tile; the workspace adds the keys as appended (the
    pages' key half) and the table is set through qkv_set_rope."""
    L, lib = _lib()
    c = L.make_config(W.TINY.replace(rope_base=10000.0))
    assert c.rope == 1 and lib.qkv_check_config(ctypes.byref(c)) == 0
    plain = L.make_config(W.TINY)
    assert plain.rope == 0
    U = 1 + -(-(W.TINY.total_tokens - W.TINY.n_sink) // W.TINY.window)
    assert L.workspace_bytes(c) - L.workspace_bytes(plain) >= U * W.TINY.n_kv_heads * 16 * W.TINY.head_dim * 2
    d = L.make_config(W.DRIFT.replace(rope_base=500000.0))
    assert lib.qkv_check_config(ctypes.byref(d)) == 0
    for bad in (dict(window=32), dict(rope=2), dict(rope=-1)):
        e = L.make_config(W.STRESS if "window" in bad else W.TINY, rope=1)
        for k, v in bad.items():
            setattr(e, k, v)
        assert lib.qkv_check_config(ctypes.byref(e)) == L.EINVAL, bad
    h = L.make_config(W.H2O, rope=1)
    assert lib.qkv_check_config(ctypes.byref(h)) == L.EINVAL       # the window policy only
    assert lib.qkv_set_rope(None, ctypes.c_void_p(256), 1 << 20) == L.EINVAL


def test_window_policy_context_limit():
    """The routing sort holds 16384 candidates: a window-policy cache may
    have up to 16383 windows per sequence (about 262K tokens at 16-token
    windows), one more is refused."""
    L, lib = _lib()
    for max_ctx, ok in ((5 + 16382 * 16, True), (5 + 16383 * 16, False), (140000, True)):
        c = L.make_config(W.TINY.replace(window=16, omega=16, n_sink=5), max_ctx=max_ctx)
        assert (lib.qkv_check_config(ctypes.byref(c)) == 0) == ok, max_ctx


def test_h2o_context_limit():
    """The H2O routing sort holds 16384 candidates (8-byte keys, 128 KB of
    LDS): a per-token heavy-hitter cache may hold up to 16384 positions, one
    more is refused."""
    L, lib = _lib()
    for max_ctx, ok in ((8192, True), (16384, True), (16385, False)):
        c = L.make_config(W.H2O, max_ctx=max_ctx)
        assert (lib.qkv_check_config(ctypes.byref(c)) == 0) == ok, max_ctx


def test_sweep_configs_are_accepted_on_host():
    """Every configuration of the random parity sweep is one the library
    accepts (checked on the host, no GPU)."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from _sweep import N_CASES, N_TOKEN_CASES, draw, draw_h2o, draw_hqekv, head_limit_cases
    L, lib = _lib()
    cases = ([draw(i) for i in range(N_CASES)] + [draw_hqekv(i) for i in range(N_TOKEN_CASES)] +
             [draw_h2o(i) for i in range(N_TOKEN_CASES)] + [(c, 0) for c in head_limit_cases().values()])
    for cfg, splits in cases:
        c = L.make_config(cfg, n_splits=splits)
        assert lib.qkv_check_config(ctypes.byref(c)) == 0, cfg
        assert L.workspace_bytes(c) > 0
