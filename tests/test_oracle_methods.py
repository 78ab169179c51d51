"""Oracle state machines checked against special cases and invariants (CPU).

QEvict: with K_f covering every window the method is exact attention; with
K_f = K_q = 0 it is sinks + recent (StreamingLLM at window granularity); on
data whose groups sit on four levels the INT2 tier is lossless; scores are
additive (Eq.1); tier sizes respect the capacities; evicted windows never
return; codes survive promote/demote cycles unchanged (Algorithm 1).
H2O: full budget is exact attention; uniform attention evicts the youngest
non-recent position (age bias, section 1.2); a far hotspot is retained.
HqeKV: tiers only move down (section 3.5).
"""
import numpy as np
import pytest

import workloads as W
from oracle import h2o as oh
from oracle import hqekv as oq
from oracle import qevict as oe
from oracle.attention import attend
from oracle.numerics import bf16_to_f64


def small_drift(**kw):
    base = dict(name="drift_small", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, prefill=2048, steps=160,
                window=16, omega=16, n_sink=5, n_recent=64, cluster_a=(60, 24), cluster_b=(4, 12),
                switch_step=64)
    base.update(kw)
    c = W.DRIFT.replace(**base)
    w0 = W.w0(c)
    return c.replace(k_full=kw.get("k_full", int(0.1 * w0)), k_quant=kw.get("k_quant", int(0.3 * w0)))


def run(cfg, kb, vb, qb, steps=None):
    return oe.run_sequence(cfg, kb, vb, qb, steps=steps, record=True)


def test_qevict_full_capacity_is_exact_attention():
    cfg = W.TINY.replace(k_full=10 ** 6, k_quant=0)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qb = wl.queries(0)
    seq, outs, _ = run(cfg, kb, vb, qb)
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    for s in range(cfg.steps):
        n = cfg.prefill + s + 1
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :n], V[:, :n])
        np.testing.assert_allclose(outs[s], ref, atol=1e-12)
    assert not seq.ledger and not np.any(seq.tier == oe.EVICTED)


@pytest.mark.parametrize("n_sink", [W.TINY.n_sink, 0])
def test_qevict_zero_capacity_is_sinks_plus_recent(n_sink):
    """With no ranked capacity attention reads the sinks and the recent
    windows only; with no sink tokens the sink unit holds no position and
    keeps no tier."""
    cfg = W.TINY.replace(k_full=0, k_quant=0, n_sink=n_sink)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qb = wl.queries(0)
    seq, outs, _ = run(cfg, kb, vb, qb)
    if n_sink == 0:
        assert seq.tier[0] == oe.EMPTY and not np.any(seq.unit_of_pos == 0)
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    P, w, ns, nr, om = cfg.prefill, cfg.window, cfg.n_sink, cfg.n_recent, cfg.omega
    for s in range(cfg.steps):
        n = P + s + 1
        pos = np.arange(n)
        last = ns + ((pos - ns) // w + 1) * w - 1          # last position of each position's window
        events = [P + e + 1 for e in range(s) if (e + 1) % om == 0]
        if events:   # windows aged at the latest event are gone; later ones still recent
            keep = (pos < ns) | (last >= events[-1] - nr)
        else:
            keep = np.ones(n, bool)
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :n], V[:, :n], keep)
        np.testing.assert_allclose(outs[s], ref, atol=1e-12)


def _four_level_bits(cfg, rng):
    """K/V whose KIVI groups sit exactly on 4 levels {-0.5,-0.25,0,0.25}."""
    hkv, T, d, w = cfg.n_kv_heads, cfg.total_tokens, cfg.head_dim, cfg.window
    lv = np.array([-0.5, -0.25, 0.0, 0.25], np.float32)
    kc = rng.integers(0, 4, (hkv, T, d))
    ns = cfg.n_sink
    for a in range(ns, T - w + 1, w):                 # each window, each channel: both extremes
        kc[:, a, :], kc[:, a + 1, :] = 0, 3
    vc = rng.integers(0, 4, (hkv, T, d))
    vc[:, :, 0::32], vc[:, :, 1::32] = 0, 3           # each token, each 32-channel group
    to_bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    return to_bits(lv[kc]), to_bits(lv[vc])


def test_qevict_int2_lossless_on_four_level_data():
    cfg = W.TINY.replace(k_full=0, k_quant=10 ** 6)
    rng = np.random.default_rng(7)
    kb, vb = _four_level_bits(cfg, rng)
    qb = (np.asarray(rng.standard_normal((cfg.steps, cfg.n_q_heads, cfg.head_dim)), np.float32)
          .view(np.uint32) >> 16).astype(np.uint16)
    seq, outs, _ = run(cfg, kb, vb, qb)
    assert seq.ledger, "windows must have been quantized"
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    for s in range(cfg.steps):
        n = cfg.prefill + s + 1
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :n], V[:, :n])
        np.testing.assert_allclose(outs[s], ref, atol=1e-12)


def _sixteen_level_bits(cfg, rng):
    """K/V whose KIVI groups sit exactly on 16 levels -1 + k/8, k = 0..15."""
    hkv, T, d, w = cfg.n_kv_heads, cfg.total_tokens, cfg.head_dim, cfg.window
    lv = (-1.0 + np.arange(16) / 8.0).astype(np.float32)
    kc = rng.integers(0, 16, (hkv, T, d))
    for a in range(cfg.n_sink, T - w + 1, w):
        kc[:, a, :], kc[:, a + 1, :] = 0, 15
    vc = rng.integers(0, 16, (hkv, T, d))
    vc[:, :, 0::32], vc[:, :, 1::32] = 0, 15
    to_bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    return to_bits(lv[kc]), to_bits(lv[vc])


def test_qevict_int4_lossless_on_sixteen_level_data_and_int2_is_not():
    """QEvict notes section 6.5 (INT4 as the recoverable tier's precision):
    with every window quantized, data on 16 levels per group passes the
    4-bit tier exactly (attention equals exact attention); the 2-bit tier on
    the same data does not."""
    cfg = W.TINY.replace(k_full=0, k_quant=10 ** 6, quant_bits=4)
    rng = np.random.default_rng(11)
    kb, vb = _sixteen_level_bits(cfg, rng)
    qb = (np.asarray(rng.standard_normal((cfg.steps, cfg.n_q_heads, cfg.head_dim)), np.float32)
          .view(np.uint32) >> 16).astype(np.uint16)
    seq, outs, _ = run(cfg, kb, vb, qb)
    assert seq.ledger and all(L["bits"] == 4 and L["kcodes"].max() <= 15 for L in seq.ledger.values())
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    worst2 = 0.0
    seq2, outs2, _ = run(cfg.replace(quant_bits=2), kb, vb, qb)
    for s in range(cfg.steps):
        n = cfg.prefill + s + 1
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :n], V[:, :n])
        np.testing.assert_allclose(outs[s], ref, atol=1e-12)
        worst2 = max(worst2, float(np.abs(outs2[s] - ref).max()))
    assert worst2 > 1e-3


@pytest.mark.parametrize("bits", [2, 4])
def test_qevict_invariants_on_small_drift(bits):
    cfg = small_drift(quant_bits=bits)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qb = wl.queries(0)
    seq, outs, masses = run(cfg, kb, vb, qb)
    hq = cfg.n_q_heads
    for m in masses:                                   # every head's weights sum to 1
        np.testing.assert_allclose(m.sum(), hq, atol=1e-9)
    np.testing.assert_allclose(seq.score.sum(), cfg.steps * hq, atol=1e-8)   # Eq.(1) is additive
    evicted = set()
    codes_seen = {}
    for ev in seq.events:
        assert len(ev.full) <= cfg.k_full and len(ev.quant) <= cfg.k_quant
        assert not (set(ev.full) | set(ev.quant)) & evicted, "an evicted window returned"
        evicted |= set(ev.evicted)
    assert seq.tier[0] == oe.SINK
    # migration stability: a window's codes never change after its first pack
    seq2 = oe.QEvictSequence(kb, vb, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink,
                             n_recent=cfg.n_recent, k_full=cfg.k_full, k_quant=cfg.k_quant,
                             bits=cfg.quant_bits, n_q_heads=cfg.n_q_heads)
    seq2.prefill(cfg.prefill)
    cycles = 0
    for s in range(cfg.steps):
        seq2.step(s, qb[s])
        for u, L in seq2.ledger.items():
            sig = (L["kcodes"].tobytes(), L["vcodes"].tobytes(), L["kscale"].tobytes(), L["vzero"].tobytes())
            if u in codes_seen:
                assert codes_seen[u] == sig
            codes_seen[u] = sig
        cycles += sum(len(e.reused) for e in seq2.events[-1:]) if (s + 1) % cfg.omega == 0 else 0
    promoted = {u for e in seq.events for u in e.promoted}
    assert promoted, "the drift workload must force promotions"


def test_qevict_drift_promotes_cluster_b_after_switch():
    """The attention target moves to the early cluster B: some of its windows,
    quantized while cluster A was attended, come back to full precision."""
    cfg = small_drift()
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    seq, _, _ = run(cfg, kb, vb, wl.queries(0))
    b0, nb = cfg.cluster_b
    b_units = set(range(1 + b0, 1 + b0 + nb))
    early = [u for e in seq.events if e.step < cfg.switch_step for u in e.promoted]
    late = [u for e in seq.events if e.step >= cfg.switch_step for u in e.promoted]
    assert set(late) & b_units
    assert not set(early) & b_units


def test_h2o_full_budget_is_exact_attention():
    cfg = W.H2O.replace(n_kv_heads=1, n_q_heads=4, head_dim=32, prefill=24, steps=16,
                        n_sink=2, k_full=1000, n_recent=1000)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    qp = wl.prefill_queries(0, 0, cfg.prefill)
    qb = wl.queries(0)
    g = oh.H2OGroup(kb[0], vb[0], G=4, n_sink=2, n_heavy=1000, n_recent=1000)
    g.prefill(cfg.prefill, qp)
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    for s in range(cfg.steps):
        t = cfg.prefill + s
        out, w, dpos, victim = g.step(t, qb[s])
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :t + 1], V[:, :t + 1])
        np.testing.assert_allclose(out, ref, atol=1e-12)
        assert victim is None
    np.testing.assert_allclose(g.score.sum(), (cfg.prefill + cfg.steps) * 4, atol=1e-9)


def test_h2o_uniform_attention_evicts_youngest_non_recent():
    """Equal weights every step: older positions accumulate more (age bias),
    so each victim is the newest position just outside the recent window."""
    d = 8
    k = np.zeros((64, d), np.uint16)                  # identical keys -> uniform attention
    v = np.zeros((64, d), np.uint16)
    g = oh.H2OGroup(k, v, G=1, n_sink=1, n_heavy=4, n_recent=3)
    q = np.zeros((1, d), np.uint16)
    for t in range(9):
        g.append(t)
        _, w = g._attend(q)
        g.score += w
    g.trim()
    for t in range(9, 30):
        _, w, dpos, victim = g.step(t, q)
        outside = sorted(set(dpos) - set(np.sort(dpos)[-3:]) - {0})
        assert victim == outside[-1]
        assert len(g.pos) == 8


def test_h2o_far_hotspot_is_retained():
    cfg = W.H2O.replace(n_kv_heads=1, n_q_heads=2, head_dim=16, prefill=32, steps=64,
                        n_sink=1, k_full=4, n_recent=4)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    rng = np.random.default_rng(9)
    kf = bf16_to_f64(kb[0])
    hot = 3
    q_hot = ((np.float32(3.0) * kf[hot][None, :] + rng.standard_normal((2, 16))).astype(np.float32)
             .view(np.uint32) >> 16).astype(np.uint16)
    qp = np.repeat(q_hot[None], cfg.prefill, axis=0)
    g = oh.H2OGroup(kb[0], vb[0], G=2, n_sink=1, n_heavy=4, n_recent=4)
    g.prefill(cfg.prefill, qp)
    for s in range(cfg.steps):
        g.step(cfg.prefill + s, q_hot)
        assert hot in g.pos
        assert len(g.pos) <= 9


def test_hqekv_downgrade_only_and_shares():
    cfg = W.HQEKV.replace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=512, steps=128,
                          omega=32, init_queries=20)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    g = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=cfg.omega)
    g.prefill(cfg.prefill, wl.prefill_queries(0, cfg.prefill - 20, cfg.prefill))
    counts0 = np.bincount(g.tier[:cfg.prefill], minlength=5)
    assert counts0.tolist() == [102, 153, 153, 51, 53]
    prev = g.tier.copy()
    qb = wl.queries(0)
    for s in range(cfg.steps):
        g.step(s, cfg.prefill + s, qb[s])
        cur = g.tier
        seen = prev != 255
        assert np.all(cur[seen] >= prev[seen]), "a token moved to a higher precision"
        prev = cur.copy()


def test_hqekv_all_full_precision_is_exact_attention():
    cfg = W.HQEKV.replace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=256, steps=40,
                          omega=16, ratios=(1.0, 0, 0, 0, 0))
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    g = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=cfg.omega)
    g.prefill(cfg.prefill, wl.prefill_queries(0, cfg.prefill - 20, cfg.prefill))
    qb = wl.queries(0)
    K, V = bf16_to_f64(kb), bf16_to_f64(vb)
    for s in range(cfg.steps):
        t = cfg.prefill + s
        out, _, _ = g.step(s, t, qb[s])
        ref, _ = attend(bf16_to_f64(qb[s]), K[:, :t + 1], V[:, :t + 1])
        np.testing.assert_allclose(out, ref, atol=1e-12)


def test_hqekv_rolling_window_ranks_by_the_last_m_steps():
    """HqeKV notes 3.8 and 3.10: with a rolling window of the last m queries
    the metric of an event is the attention of the m decode steps before it.
    Checked against an accumulating run of the same (sequence, KV head): both
    runs share the first assignment (the same prompt queries) and so every
    tier until the second event, so the rolling run's metric there must equal
    the accumulating run's score growth over those m steps times the value
    range; and the rolling scores restart from 0 after each event."""
    cfg = W.HQEKV.replace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=512, steps=64,
                          omega=32, init_queries=20)
    m, P, T = 20, cfg.prefill, cfg.omega
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    acc = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=T)
    rol = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=T, window=m)
    pq = wl.prefill_queries(0, P - 20, P)
    acc.prefill(P, pq)
    rol.prefill(P, pq)
    np.testing.assert_array_equal(acc.tier, rol.tier)
    np.testing.assert_array_equal(rol.last_metric, acc.last_metric)
    assert not rol.score.any()
    qb = wl.queries(0)
    for s in range(T):
        if s == T - m:
            start = acc.score.copy()
        if s < T - m:
            before = rol.score.copy()
        acc.step(s, P + s, qb[s])
        rol.step(s, P + s, qb[s])
        if s < T - m:
            np.testing.assert_array_equal(rol.score, before)    # outside the window: no change
    grown = (acc.score - start) * rol.range
    np.testing.assert_allclose(rol.last_metric, grown, rtol=1e-9, atol=1e-12 * float(np.max(acc.score)))
    assert np.count_nonzero(rol.last_metric) > 0
    assert not rol.score.any()


def _bare_group(T, d=32, **kw):
    rng = np.random.default_rng(5)
    kb = (rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    g = oq.HqeKVGroup(kb, kb, G=4, **kw)
    g.tier[:T] = oq.BF16
    g.N = T
    g.last_event_N = 0
    return g


def test_hqekv_chunk_ranking_hand_example():
    """HqeKV notes 3.3 (implementation note): chunks ranked by the mean of
    their tokens' metrics, ties to the newer chunk, shares counted in chunks,
    the two best chunks FP16 whatever the shares say.  Chunks of 2 over 10
    tokens, metric = score (range 1): means 2, 5, 2, 0, 7; order c4, c1, c2
    (newer of the tie), c0, c3; one chunk per share -> c4 FP16, c1 INT4 but
    pinned FP16, c2 INT2, c0 INT1, c3 evicted."""
    g = _bare_group(10, ratios=(0.2, 0.2, 0.2, 0.2, 0.2), period=8, chunk=2)
    g.score[:10] = [1, 3, 10, 0, 2, 2, 0, 0, 8, 6]
    g.range[:] = 1.0
    g.event()
    B, I4, I2, I1, E = oq.BF16, oq.INT4, oq.INT2, oq.INT1, oq.EVICT
    assert g.tier[:10].tolist() == [I1, I1, B, B, I2, I2, E, E, B, B]
    np.testing.assert_array_equal(g.chunk_mean, [2, 5, 2, 0, 7])


def test_hqekv_chunk_mean_skips_evicted_and_ineligible_tokens():
    """A chunk's mean is over its live eligible tokens only: an evicted token
    and the tokens appended since the previous event do not count."""
    g = _bare_group(12, ratios=(0.5, 0.0, 0.0, 0.0, 0.5), period=8, chunk=4)
    g.score[:12] = [4, 100, 4, 4, 1, 1, 1, 1, 9, 9, 50, 50]
    g.range[:] = 1.0
    g.tier[1] = oq.EVICT
    g.last_event_N = 10            # tokens 10, 11 are not ranked at this event
    g.event()
    np.testing.assert_array_equal(g.chunk_mean, [4.0, 1.0, 9.0])
    assert g.tier[1] == oq.EVICT and g.tier[10] == oq.BF16 and g.tier[11] == oq.BF16


def test_hqekv_chunks_of_one_token_rank_like_tokens():
    """Chunks of one position are the per-token ranking (the FP16 pin is void
    when the FP16 share already holds two or more tokens)."""
    cfg = W.HQEKV.replace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=512, steps=96,
                          omega=32, init_queries=20)
    wl = W.Workload(cfg)
    kb, vb = wl.kv(0)
    tok = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=cfg.omega)
    one = oq.HqeKVGroup(kb[0], vb[0], G=4, ratios=cfg.ratios, period=cfg.omega, chunk=1)
    pq = wl.prefill_queries(0, cfg.prefill - 20, cfg.prefill)
    tok.prefill(cfg.prefill, pq)
    one.prefill(cfg.prefill, pq)
    qb = wl.queries(0)
    for s in range(cfg.steps):
        tok.step(s, cfg.prefill + s, qb[s])
        one.step(s, cfg.prefill + s, qb[s])
        np.testing.assert_array_equal(tok.tier, one.tier)
