"""The oracle's rotary embedding around the quantized tier, pinned (CPU).

QEvict notes, section 4.4 (Algorithm 1's promotion step and the paragraph on
promoted keys' positions): keys are quantized before the rotation and rotated
again at their original positions on promotion.  Pins that do not repeat the
oracle's formula: a rotation keeps norms; a dot product of rotated vectors
depends only on the position difference; an identity table reduces the
method to the unrotated one exactly; on data the 2-bit codec reproduces
exactly, a promoted window's keys equal the ones it held before its
demotion, and the quantized tier reads exactly the rotated keys; with every
window kept in full precision attention equals attention over keys rotated
by complex multiplication (an independent formulation).
"""
import numpy as np

import workloads as W
from oracle import qevict as oe
from oracle import rope as rp
from oracle.attention import attend
from oracle.numerics import bf16_to_f64, round_to_bf16


def test_rotation_keeps_norms_and_depends_on_position_differences():
    d, n = 64, 4096
    tb = W.rope_table(n, d, 10000.0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, d))
    y = rng.standard_normal((5, d))
    p = np.array([0, 7, 100, 1000, 3000])
    rx = rp.rotate(x, tb, p)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    np.testing.assert_allclose(rp.rotate(x, tb, np.zeros(5, int)), x, rtol=0, atol=0)   # position 0: identity
    for dp in (1, 37, 500):
        a = np.sum(rp.rotate(x, tb, p + dp) * rp.rotate(y, tb, p + 2), axis=1)
        b = np.sum(rp.rotate(x, tb, p + dp + 90) * rp.rotate(y, tb, p + 92), axis=1)
        np.testing.assert_allclose(a, b, rtol=2e-5, atol=2e-5)


def _cfg(**kw):
    return W.TINY.replace(rope_base=10000.0, **kw)


def _seq(cfg, kb, vb, table):
    s = oe.QEvictSequence(kb, vb, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                          k_full=cfg.k_full, k_quant=cfg.k_quant, bits=cfg.quant_bits, n_q_heads=cfg.n_q_heads,
                          rope_table=table)
    s.prefill(cfg.prefill)
    return s


def test_identity_table_is_the_unrotated_method():
    cfg = _cfg()
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qb = wl.queries(0)
    ident = np.zeros((cfg.total_tokens, cfg.head_dim // 2, 2), np.float32)
    ident[..., 0] = 1.0
    a, b = _seq(cfg, kb, vb, ident), _seq(cfg, kb, vb, None)
    for s in range(cfg.steps):
        oa, ma = a.step(s, qb[s])
        ob, mb = b.step(s, qb[s])
        np.testing.assert_array_equal(oa, ob)
        np.testing.assert_array_equal(ma, mb)
    np.testing.assert_array_equal(a.tier, b.tier)


def _four_level(cfg, rng):
    hkv, T, d, w = cfg.n_kv_heads, cfg.total_tokens, cfg.head_dim, cfg.window
    lv = np.array([-0.5, -0.25, 0.0, 0.25], np.float32)
    kc = rng.integers(0, 4, (hkv, T, d))
    for a in range(cfg.n_sink, T - w + 1, w):
        kc[:, a, :], kc[:, a + 1, :] = 0, 3
    vc = rng.integers(0, 4, (hkv, T, d))
    vc[:, :, 0::32], vc[:, :, 1::32] = 0, 3
    to_bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    return to_bits(lv[kc]), to_bits(lv[vc])


def test_promoted_keys_are_rotated_again_at_their_positions():
    """Lossless 2-bit data: every routing event changes which windows are
    quantized (the queries aim at random keys), and after every event the
    keys attention reads -- rotated stored keys of full-precision windows,
    rotation of the dequantized keys of quantized ones -- are the rotated
    original keys; after a promotion the stored content is the content the
    window held before its demotion."""
    cfg = _cfg(k_full=3, k_quant=6, steps=64)
    rng = np.random.default_rng(3)
    kb, vb = _four_level(cfg, rng)
    wl = W.Workload(cfg)
    tb = wl.rope()
    qb = wl.queries(0)
    seq = _seq(cfg, kb, vb, tb)
    pos = np.arange(cfg.total_tokens)
    korig = bf16_to_f64(kb)
    stored = np.stack([rp.rotate_stored(korig[g], tb, pos) for g in range(cfg.n_kv_heads)])
    exact = np.stack([rp.rotate(korig[g], tb, pos) for g in range(cfg.n_kv_heads)])
    promoted = 0
    for s in range(cfg.steps):
        seq.step(s, qb[s])
        if (s + 1) % cfg.omega:
            continue
        for u in range(1, seq.n_units):
            a, b = seq.span(u)
            if seq.tier[u] in (oe.FULL, oe.RECENT):
                np.testing.assert_array_equal(seq.kcur[:, a:b], stored[:, a:b])
            elif seq.tier[u] == oe.QUANT:
                np.testing.assert_array_equal(seq.kcur[:, a:b], exact[:, a:b])
        promoted += len(seq.events[-1].promoted)
    assert promoted > 0, "no window was promoted"


def test_full_capacity_is_attention_over_complex_rotated_keys():
    cfg = _cfg(k_full=10 ** 6, k_quant=0)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qb = wl.queries(0)
    tb = wl.rope()
    seq = _seq(cfg, kb, vb, tb)
    h = cfg.head_dim // 2
    korig = bf16_to_f64(kb)
    ang = tb.astype(np.float64)                                        # [T, h, 2]
    z = (korig[..., :h] + 1j * korig[..., h:]) * (ang[None, :, :, 0] + 1j * ang[None, :, :, 1])
    krot = round_to_bf16(np.concatenate([z.real, z.imag], axis=-1).astype(np.float32))
    V = bf16_to_f64(vb)
    for s in range(cfg.steps):
        o, _ = seq.step(s, qb[s])
        n = cfg.prefill + s + 1
        ref, _ = attend(bf16_to_f64(qb[s]), krot[:, :n], V[:, :n])
        np.testing.assert_allclose(o, ref, atol=1e-12)
