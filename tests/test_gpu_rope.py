"""Rotary keys around the quantized tier on the GPU against the oracle.

QEvict notes, section 4.4 (Algorithm 1's promotion step and the paragraph on
promoted keys' positions): keys arrive before the rotary embedding; pages hold
them rotated once at their positions, the ledger quantizes them before the
rotation, the quantized tier is read rotated at the tokens' positions and a
promoted window is rotated again at them.  The oracle (oracle.rope,
oracle.qevict with a table) fixes every step; the bars are those of the other
parity tests: tiers, ledgers (codes and parameters) and full-precision
contents (rotated keys included) bit for bit, outputs within 2e-3, masses and
scores within 1e-4 relative.
"""
import numpy as np
import pytest

import workloads as W

from _harness import log
from test_gpu_qevict import _run_parity, _small_drift

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_quantization_eviction_amd  # noqa: F401  (raises if the library is missing)
    return torch


def _promotions(seqs):
    return sum(len(e.promoted) for sq in seqs.values() for e in sq.events)


def test_rope_tiny_parity(torch_cuda):
    """d = 64, four heads per KV head, 8-token windows (rows 8..15 of each
    quantized tile hold no token)."""
    _run_parity(W.TINY.replace(rope_base=10000.0), torch_cuda, label="rope-tiny")


def test_rope_int4_tiny_parity(torch_cuda):
    _run_parity(W.TINY.replace(rope_base=10000.0, quant_bits=4), torch_cuda, label="rope-int4-tiny")


@pytest.mark.parametrize("splits", [1, 5])
def test_rope_small_drift_parity(torch_cuda, splits):
    """d = 128, 16-token windows, the query switch and the promotions after it."""
    cfg = _small_drift(rope_base=500000.0)
    _, seqs = _run_parity(cfg, torch_cuda, n_splits=splits, check_ledger_every=2, label=f"rope-drift s={splits}")
    assert _promotions(seqs) > 0


def test_rope_g8_parity(torch_cuda):
    """Eight heads per KV head (d = 64; at d = 128 eight heads need 32-token
    windows) with 16-token windows, ragged prompt."""
    c = W.TINY.replace(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=64, prefill=1003, steps=48, window=16,
                       omega=16, n_sink=5, n_recent=32, k_full=8, k_quant=24, rope_base=10000.0)
    _run_parity(c, torch_cuda, n_splits=3, label="rope-g8")


def test_rope_identity_table_matches_the_plain_cache(torch_cuda):
    """With an identity table (cos 1, sin 0) a rotary cache holds exactly what
    the plain cache holds (tiers, full-precision keys, ledgers bitwise); its
    quantized tier is read through the rotated-key operands (float32
    dequantized keys in two fp16 limbs) instead of the code operands, so
    outputs and scores agree to rounding."""
    from tiered_quantization_eviction_amd import Cache, make_config
    from _harness import gpu_inputs
    torch = torch_cuda
    cfg = _small_drift(steps=48)
    K, V, Q = gpu_inputs(cfg, W.Workload(cfg))
    ident = torch.zeros((cfg.total_tokens, cfg.head_dim // 2, 2), dtype=torch.float32, device="cuda")
    ident[..., 0] = 1.0
    caches = [Cache(make_config(cfg)), Cache(make_config(cfg, rope=1))]
    caches[1].set_rope(ident)
    outs = [torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
            for _ in caches]
    P = cfg.prefill
    for c in caches:
        c.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous())
    for s in range(cfg.steps):
        for c, o in zip(caches, outs):
            c.append(K[:, :, P + s:P + s + 1].contiguous(), V[:, :, P + s:P + s + 1].contiguous())
            c.decode_attend(Q[:, s].contiguous(), o)
            if (s + 1) % cfg.omega == 0:
                c.route()
        torch.cuda.synchronize()
        d = float((outs[0] - outs[1]).abs().max())
        assert d <= 1e-5, f"step {s}: {d}"
    for what in ("tiers", "keys", "kcodes", "kparams", "vcodes", "vparams"):
        a, b = caches[0].export(what), caches[1].export(what)
        torch.cuda.synchronize()
        assert torch.equal(a, b), what
    sa, sb = (c.export("scores").view(torch.float32).cpu().numpy() for c in caches)
    np.testing.assert_allclose(sa, sb, rtol=1e-5, atol=1e-9)
    log("[rope-identity] outputs within 1e-5, scores within 1e-5, tiers/keys/ledger equal")


def test_rope_requires_a_table(torch_cuda):
    from tiered_quantization_eviction_amd import Cache, QkvError, make_config
    from tiered_quantization_eviction_amd import _lib as L
    torch = torch_cuda
    cfg = W.TINY.replace(rope_base=10000.0)
    c = Cache(make_config(cfg))
    K = torch.zeros((1, 1, 4, cfg.head_dim), dtype=torch.int16, device="cuda")
    with pytest.raises(QkvError) as e:
        c.append(K, K)
    assert e.value.code == L.ESTATE
    short = torch.zeros((cfg.total_tokens - 1, cfg.head_dim // 2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(QkvError):
        c.set_rope(short)
    plain = Cache(make_config(W.TINY))
    with pytest.raises(QkvError):
        plain.set_rope(torch.zeros((cfg.total_tokens, cfg.head_dim // 2, 2), dtype=torch.float32, device="cuda"))


def test_rope_snapshot_restore_continues_bitwise(torch_cuda):
    """A rotary cache restored from its snapshot (the raw keys included: the
    ledger packs from them at later demotions) continues exactly like the
    original: outputs, tiers, scores and ledgers bitwise through the query
    switch and the promotions after it."""
    from tiered_quantization_eviction_amd import Cache, make_config
    from _harness import gpu_inputs
    torch = torch_cuda
    cfg = _small_drift(rope_base=500000.0)
    wl = W.Workload(cfg)
    K, V, Q = gpu_inputs(cfg, wl)
    table = torch.from_numpy(wl.rope()).cuda()
    a = Cache(make_config(cfg))
    a.set_rope(table)
    P = cfg.prefill
    a.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous())
    outs = [torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(2)]

    def step(c, o, s):
        c.append(K[:, :, P + s:P + s + 1].contiguous(), V[:, :, P + s:P + s + 1].contiguous())
        c.decode_attend(Q[:, s].contiguous(), o)
        if (s + 1) % cfg.omega == 0:
            c.route()

    cut = 40                                        # mid-period, before the query switch
    for s in range(cut):
        step(a, outs[0], s)
    snap = a.snapshot()
    assert "keys_raw" in snap
    b = Cache(make_config(cfg))
    b.set_rope(table)
    b.restore(snap)
    for s in range(cut, cfg.steps):
        step(a, outs[0], s)
        step(b, outs[1], s)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {s}"
    for what in ("tiers", "scores", "ledger", "kcodes", "kparams", "keys", "keys_raw"):
        x, y = a.export(what), b.export(what)
        torch.cuda.synchronize()
        assert torch.equal(x, y), what
    log(f"[rope-snapshot] restored at step {cut}; {cfg.steps - cut} steps bitwise equal")
