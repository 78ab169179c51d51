"""GPU parity of the HIP path with the oracle (through the C ABI).

Bars: codes, parameters, tiers, ledger membership and promoted content
bit-exact; attention outputs within 2e-3 max-abs; accumulated scores within
1e-4 relative.  Sizes span several tiles, several splits and ragged tails.
"""
import numpy as np
import pytest

import workloads as W
from oracle import codec as oc
from oracle import qevict as oe
from oracle.numerics import bf16_to_f64, round_to_bf16_bits
from oracle.rank import rank_tiers as o_rank_tiers

from _harness import QEvictGPURun, gpu_inputs, log

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
SCORE_RTOL = 1e-4


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_quantization_eviction_amd  # noqa: F401  (raises if the library is missing)
    return torch


# ---------------------------------------------------------------------------
# stateless quantizer and ranking
# ---------------------------------------------------------------------------

def _bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return round_to_bf16_bits(x)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("tokens", [8, 16, 32, 48])
def test_quantize_k_per_channel_bitexact(torch_cuda, bits, tokens):
    from tiered_quantization_eviction_amd import _lib as L
    log(f"quantize K per-channel bits={bits} tokens={tokens}")
    rng = np.random.default_rng(100 + bits * 7 + tokens)
    xb = _bf16_bits(rng, (6, tokens, 128), scale=rng.uniform(0.2, 30.0, (6, 1, 128)))
    xb[0, :, 5] = xb[0, 0, 5]                              # a degenerate group
    codes, params = L.quantize_window(torch_cuda.from_numpy(xb.view(np.int16)).cuda(), L.KIND_K_PER_CHANNEL, bits)
    assert L.quantize_status() == 0
    codes, params = codes.cpu().numpy(), params.cpu().numpy().view(np.uint16)
    x = bf16_to_f64(xb).astype(np.float32)
    n_chunks = -(-tokens // 32)
    for blk in range(6):
        kc = np.zeros((1, tokens, 128), np.uint8)
        ks = np.zeros((1, 128, n_chunks), np.float16)
        kz = np.zeros_like(ks)
        kt = x[blk].T[None]
        for ci in range(n_chunks):
            t0, t1 = ci * 32, min(tokens, ci * 32 + 32)
            c, s, z = oc.uniform_quantize(kt[:, :, t0:t1], bits)
            kc[:, t0:t1, :] = c.transpose(0, 2, 1)
            ks[:, :, ci], kz[:, :, ci] = s, z
        np.testing.assert_array_equal(codes[blk], oc.canonical_k_codes(kc, bits)[0])
        np.testing.assert_array_equal(params[blk], oc.canonical_params(ks, kz)[0].view(np.uint16).reshape(-1))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("f32", [False, True])
def test_quantize_per_token_bitexact(torch_cuda, bits, f32):
    from tiered_quantization_eviction_amd import _lib as L
    log(f"quantize per-token bits={bits} f32={f32}")
    rng = np.random.default_rng(200 + bits + 10 * f32)
    if f32:
        x = (rng.standard_normal((3, 40, 128)) * rng.uniform(0.1, 9, (3, 40, 1))).astype(np.float32)
        dev = torch_cuda.from_numpy(x).cuda()
    else:
        xb = _bf16_bits(rng, (3, 40, 128), scale=3.0)
        x = bf16_to_f64(xb).astype(np.float32)
        dev = torch_cuda.from_numpy(xb.view(np.int16)).cuda()
    codes, params = L.quantize_window(dev, L.KIND_PER_TOKEN, bits)
    codes, params = codes.cpu().numpy(), params.cpu().numpy().view(np.uint16)
    for blk in range(3):
        c, s, z = oc.per_token_quantize(x[blk], bits)
        np.testing.assert_array_equal(codes[blk], oc.canonical_v_codes(c[None], bits)[0])
        np.testing.assert_array_equal(params[blk], oc.canonical_params(s, z).view(np.uint16).reshape(-1))


def test_quantize_int1_normal_codes_bitexact(torch_cuda):
    from tiered_quantization_eviction_amd import _lib as L
    log("quantize int1-normal")
    rng = np.random.default_rng(300)
    xb = _bf16_bits(rng, (2, 33, 128), scale=2.0)
    codes, params = L.quantize_window(torch_cuda.from_numpy(xb.view(np.int16)).cuda(), L.KIND_INT1_NORMAL, 1)
    codes, params = codes.cpu().numpy(), params.cpu().numpy().view(np.float16)
    x = bf16_to_f64(xb).astype(np.float32)
    for blk in range(2):
        c, m, sd = oc.int1_normal_quantize(x[blk])
        np.testing.assert_array_equal(codes[blk], oc.pack_codes(c.reshape(-1), 1))
        # mean and deviation are both summed in float64 and rounded once to
        # float32, then to float16, on both sides: compared bit for bit
        np.testing.assert_array_equal(params[blk].reshape(-1, 2)[:, 0].view(np.uint16), m.view(np.uint16))
        np.testing.assert_array_equal(params[blk].reshape(-1, 2)[:, 1].view(np.uint16), sd.view(np.uint16))


@pytest.mark.parametrize("bad", [1e6, np.nan, np.inf, -np.inf])
def test_quantize_range_error_latched(torch_cuda, bad):
    """A step above the float16 maximum, and a NaN or infinity in a group
    (refused like an out-of-range value, as the oracle's quantizer refuses
    it), latch QKV_ERANGE for either uniform kind; finite inputs leave the
    latch clear."""
    from tiered_quantization_eviction_amd import _lib as L
    log(f"quantize range error ({bad})")
    for kind in (L.KIND_PER_TOKEN, L.KIND_K_PER_CHANNEL):
        x = np.zeros((1, 8, 64), np.float32)
        L.quantize_window(torch_cuda.from_numpy(x).cuda(), kind, 2)
        assert L.quantize_status() == 0
        x[0, 3, 5] = bad
        L.quantize_window(torch_cuda.from_numpy(x).cuda(), kind, 2)
        assert L.quantize_status() == L.ERANGE, (kind, bad)
        assert L.quantize_status() == 0                # the latch clears when read
        with pytest.raises(oc.ParamRangeError):
            oc.uniform_quantize(x[0] if kind == L.KIND_PER_TOKEN else x[0].T, 2)


def test_rank_tiers_examples(torch_cuda):
    from tiered_quantization_eviction_amd import _lib as L
    import json, os
    log("rank tiers: printed examples")
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hqekv_8token_example.json")))
    m = np.array(g["acc_attention"], np.float32) * np.array(g["value_range"], np.float32)
    dev = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).cuda()
    t = L.rank_tiers(dev(m), dev(np.arange(8, dtype=np.int32)), dev(np.ones(8, np.uint8)),
                     dev(np.array([0, 2, 2, 2], np.int32))).cpu().numpy()
    exp = o_rank_tiers(m.astype(np.float64), np.arange(8), np.ones(8, bool), [0, 2, 2, 2])
    np.testing.assert_array_equal(t, exp)
    assert sorted(np.flatnonzero(t == 4) + 1) == [4, 7]
    # H2O capacity-6 step: rank the 4 non-recent positions, keep 3
    h = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "h2o_capacity6_example.json")))
    sc = np.array(h["scores_after"], np.float32)
    pos = np.array(h["positions"], np.int32)
    elig = np.array([p not in h["recent_after"] for p in h["positions"]], np.uint8)
    t = L.rank_tiers(dev(sc), dev(pos), dev(elig), dev(np.array([3], np.int32))).cpu().numpy()
    assert pos[t == 1].tolist() == [h["evicted"]]


@pytest.mark.parametrize("n", [1, 7, 100, 1000, 4096, 8192])
def test_rank_tiers_random_with_ties(torch_cuda, n):
    from tiered_quantization_eviction_amd import _lib as L
    log(f"rank tiers random n={n}")
    rng = np.random.default_rng(n)
    sc = rng.integers(0, max(2, n // 10), n).astype(np.float32) * np.float32(0.25)   # many ties
    pos = rng.permutation(n).astype(np.int32)
    el = (rng.random(n) > 0.2).astype(np.uint8)
    counts = np.array([n // 5, n // 3, 1], np.int32)
    dev = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).cuda()
    t = L.rank_tiers(dev(sc), dev(pos), dev(el), dev(counts)).cpu().numpy()
    np.testing.assert_array_equal(t, o_rank_tiers(sc, pos, el.astype(bool), counts.tolist()))


# ---------------------------------------------------------------------------
# QEvict end to end
# ---------------------------------------------------------------------------

def _oracle_seq(cfg, wl, b):
    k, v = wl.kv(b)
    seq = oe.QEvictSequence(k, v, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                            k_full=cfg.k_full, k_quant=cfg.k_quant, bits=cfg.quant_bits, group=cfg.group,
                            n_q_heads=cfg.n_q_heads, rope_table=wl.rope() if cfg.rope_base else None)
    seq.prefill(cfg.prefill)
    return seq, wl.queries(b)


def _check_ledger(run, seqs, cfg):
    U, B, H, w, d, bits = run.U, cfg.batch, cfg.n_kv_heads, cfg.window, cfg.head_dim, cfg.quant_bits
    flags = run.ledger_flags()
    kc = run.export_np("kcodes", np.uint8, (B, U, H, w * d * bits // 8))
    vc = run.export_np("vcodes", np.uint8, (B, U, H, w * d * bits // 8))
    kp = run.export_np("kparams", np.uint16, (B, U, H, d, 2))
    vp = run.export_np("vparams", np.uint16, (B, U, H, w, d // 32, 2))
    for b, seq in seqs.items():
        assert set(np.flatnonzero(flags[b])) == set(seq.ledger), "ledger membership differs"
        for u, Lg in seq.ledger.items():
            np.testing.assert_array_equal(kc[b, u], oc.canonical_k_codes(Lg["kcodes"], bits), err_msg=f"kcodes u={u}")
            np.testing.assert_array_equal(vc[b, u], oc.canonical_v_codes(Lg["vcodes"], bits), err_msg=f"vcodes u={u}")
            np.testing.assert_array_equal(kp[b, u], oc.canonical_params(Lg["kscale"], Lg["kzero"])[:, :, 0]
                                          .view(np.uint16), err_msg=f"kparams u={u}")
            np.testing.assert_array_equal(vp[b, u], oc.canonical_params(Lg["vscale"], Lg["vzero"]).view(np.uint16),
                                          err_msg=f"vparams u={u}")


def _check_event(run, seqs, cfg):
    """The library's record of the last routing event against the oracle's:
    counters exactly, the victims as a set (listed in non-increasing score
    order), the relative cut margins to the score tolerance (the library's
    come from float32 scores)."""
    recs = run.cache.last_event()
    scores = run.scores()
    for b, seq in seqs.items():
        ev, r = seq.events[-1], recs[b]
        exp = dict(tokens=ev.n_tokens, candidates=ev.candidates, full=len(ev.full), quant=len(ev.quant),
                   evicted=len(ev.evicted), promoted=len(ev.promoted), first_packs=len(ev.first_packed),
                   reused=len(ev.reused), demoted=len(ev.first_packed) + len(ev.reused))
        got = {k: r[k] for k in exp}
        assert got == exp, f"seq {b}: event record {got} != oracle {exp}"
        assert set(r["victims"]) == set(ev.evicted), f"seq {b}: victims"
        vs = scores[b][r["victims"]]
        assert np.all(vs[:-1] >= vs[1:]), f"seq {b}: victims not in rank order"
        for k, m in zip(("margin_full", "margin_quant"), ev.margins):
            if np.isinf(m):
                assert np.isinf(r[k]), (b, k, r[k])
            else:
                assert abs(r[k] - m) <= 2 * SCORE_RTOL, f"seq {b}: {k} {r[k]} vs oracle {m}"
        assert r["margin_min"] == min(r["margin_full"], r["margin_quant"])


def _check_content(run, seqs, cfg):
    """Full-precision content of sink/recent/full units, incl. promoted windows."""
    T, B, H, d = cfg.prefill + cfg.steps, cfg.batch, cfg.n_kv_heads, cfg.head_dim
    keys = run.export_np("keys", np.uint16, (B, H, T, d))
    vals = run.export_np("values", np.uint16, (B, H, T, d))
    for b, seq in seqs.items():
        acc = np.isin(seq.tier, (oe.SINK, oe.RECENT, oe.FULL))[seq.unit_of_pos[:seq.N]]
        idx = np.flatnonzero(acc)
        np.testing.assert_array_equal(bf16_to_f64(keys[b][:, idx]), seq.kcur[:, idx], err_msg="keys")
        np.testing.assert_array_equal(bf16_to_f64(vals[b][:, idx]), seq.vcur[:, idx], err_msg="values")


def _run_parity(cfg, torch_cuda, seq_ids=None, n_splits=0, check_ledger_every=1, mass_every=1, label="",
                fused=False):
    wl = W.Workload(cfg)
    log(f"[{label}] QEvict parity: {cfg.name} B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} "
        f"d={cfg.head_dim} P={cfg.prefill} steps={cfg.steps} w={cfg.window} splits={n_splits} fused={fused}")
    K, V, Q = gpu_inputs(cfg, wl)
    run = QEvictGPURun(cfg, K, V, Q, n_splits=n_splits, fused=fused)
    seq_ids = list(range(cfg.batch)) if seq_ids is None else seq_ids
    seqs, qs = {}, {}
    for b in seq_ids:
        seqs[b], qs[b] = _oracle_seq(cfg, wl, b)
    n_routes = 0
    worst = 0.0
    for s in range(cfg.steps):
        want_mass = (s % mass_every == 0)
        routed = run.step(want_mass=want_mass)
        torch_cuda.cuda.synchronize()
        out = run.out.cpu().numpy()
        mass = run.mass.cpu().numpy() if want_mass else None
        scores = run.scores()
        for b in seq_ids:
            o, m = seqs[b].step(s, qs[b][s])
            err = np.abs(out[b] - o).max()
            worst = max(worst, err)
            assert err <= OUT_TOL, f"step {s} seq {b}: out err {err}"
            if mass is not None:
                np.testing.assert_allclose(mass[b], m, rtol=SCORE_RTOL, atol=1e-7, err_msg=f"mass step {s}")
            np.testing.assert_allclose(scores[b], seqs[b].score, rtol=SCORE_RTOL, atol=1e-7,
                                       err_msg=f"scores step {s} seq {b}")
        if routed:
            n_routes += 1
            tiers = run.tiers()
            for b in seq_ids:
                ev = seqs[b].events[-1]
                exp = seqs[b].tier.copy()
                np.testing.assert_array_equal(tiers[b], exp, err_msg=f"tiers after event {n_routes} (step {s}) "
                                              f"seq {b}, margins {ev.margins}")
            _check_event(run, seqs, cfg)
            if n_routes % check_ledger_every == 0:
                _check_ledger(run, seqs, cfg)
                _check_content(run, seqs, cfg)
    log(f"[{label}] worst out err {worst:.3e}, routes {n_routes}, promotions "
        f"{sum(len(e.promoted) for sq in seqs.values() for e in sq.events)}")
    return run, seqs


def test_qevict_tiny_parity(torch_cuda):
    _run_parity(W.TINY, torch_cuda, label="tiny")


def _small_drift(**kw):
    base = dict(name="drift_small", batch=3, n_q_heads=16, n_kv_heads=4, head_dim=128, prefill=2048, steps=160,
                window=16, omega=16, n_sink=5, n_recent=64, cluster_a=(60, 24), cluster_b=(4, 12), switch_step=64)
    base.update(kw)
    c = W.DRIFT.replace(**base)
    w0 = W.w0(c)
    return c.replace(k_full=int(0.1 * w0), k_quant=int(0.3 * w0))


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_qevict_small_drift_parity(torch_cuda, splits):
    run, seqs = _run_parity(_small_drift(), torch_cuda, n_splits=splits, check_ledger_every=2,
                            label=f"drift_small s={splits}")
    assert any(e.promoted for sq in seqs.values() for e in sq.events)


def test_qevict_window32_g8_parity(torch_cuda):
    """Config-5 geometry at small size: G = 8, 32-token windows (two tiles per
    window), ragged prefill."""
    c = W.STRESS.replace(batch=2, prefill=3000, steps=96, n_q_heads=64, n_kv_heads=8)
    w0 = W.w0(c)
    c = c.replace(k_full=w0 // 4, k_quant=w0 // 2)
    _run_parity(c, torch_cuda, n_splits=5, check_ledger_every=1, label="w32g8")


def test_qevict_d64_window8_parity(torch_cuda):
    c = W.TINY.replace(batch=2, n_q_heads=8, n_kv_heads=2, prefill=515, steps=40, k_full=10, k_quant=20)
    _run_parity(c, torch_cuda, n_splits=4, label="d64w8")


@pytest.mark.parametrize("kf,kq", [(0, 0), (0, 10 ** 6), (10 ** 6, 0), (3, 0), (0, 5)])
def test_qevict_degenerate_capacities_parity(torch_cuda, kf, kq):
    """The method's degenerate budgets: no ranked windows at all (sinks plus
    recent, StreamingLLM at window granularity), every ranked window
    quantized, nothing quantized (full attention over everything kept), and
    small two-tier and quantized-only budgets that evict most windows."""
    c = W.TINY.replace(k_full=kf, k_quant=kq, steps=40)
    _run_parity(c, torch_cuda, label=f"degenerate kf={kf} kq={kq}")


def test_qevict_large_batch_multi_item_pack_parity(torch_cuda):
    """128 sequences: the pack/promote launch holds about 6 * CUs / 128
    workgroups per sequence, fewer than the (window, KV head) items of a
    routing event (12 windows x 4 KV heads at the first one), so every
    workgroup walks several items with the next item's window fetched ahead.
    Ledgers, contents and tiers of sampled sequences are compared bit for bit
    after every event."""
    c = W.TINY.replace(batch=128, n_q_heads=16, n_kv_heads=4, head_dim=128, prefill=520, steps=40, window=16,
                       omega=16, n_sink=5, n_recent=64, k_full=3, k_quant=12)
    _run_parity(c, torch_cuda, seq_ids=[0, 37, 64, 127], check_ledger_every=1, label="batch128")


def test_quantize_int1_float16_tie_rounds_twice(torch_cuda):
    """A value row of the HqeKV recipe (sequence 5, KV head 3, position 40690
    at a 65536-token prompt + 128 steps) whose population deviation rounds to
    exactly 1.81396484375 in float32: a float16 tie, which rounds to even
    (16194).  The float64 deviation lies just below the tie, so rounding it to
    float16 in one step would give 16193; the reading rounds to float32
    first."""
    from tiered_quantization_eviction_amd import _lib as L
    log("quantize int1-normal at a float16 tie")
    cfg = W.HQEKV.replace(steps=128)
    _, v = W.Workload(cfg).kv(5)
    row = v[3, 40690][None, None, :]                         # [1 block, 1 token, 128] bf16 bits
    x = bf16_to_f64(row).astype(np.float32)
    c, m, sd = oc.int1_normal_quantize(x[0])
    assert float(sd[0]) == 1.814453125 and sd.view(np.uint16)[0] == 16194
    x64 = x[0, 0].astype(np.float64)
    m32 = np.float32(x64.sum() / 128)
    s64 = np.sqrt(((x64 - np.float64(m32)) ** 2).sum() / 128)
    assert float(np.float32(s64)) == 1.81396484375 and np.float16(s64) != np.float16(np.float32(s64))
    codes, params = L.quantize_window(torch_cuda.from_numpy(row.view(np.int16)).cuda(), L.KIND_INT1_NORMAL, 1)
    params = params.cpu().numpy().view(np.uint16).reshape(-1)
    assert params[1] == 16194, params
    assert params[0] == m.view(np.uint16)[0]
    np.testing.assert_array_equal(codes.cpu().numpy()[0], oc.pack_codes(c.reshape(-1), 1))


# ---------------------------------------------------------------------------
# the INT4 recoverable tier (QEvict notes section 6.5: the recoverable tier's
# precision is one of the swept knobs; INT4 keeps fewer windows at a fixed
# byte budget, each with less error)
# ---------------------------------------------------------------------------

def test_qevict_int4_tiny_parity(torch_cuda):
    _run_parity(W.TINY.replace(quant_bits=4), torch_cuda, label="int4-tiny")


@pytest.mark.parametrize("splits", [1, 3])
def test_qevict_int4_small_drift_parity(torch_cuda, splits):
    """The drift recipe with a 4-bit recoverable tier at the capacities an
    INT2 tier of the same bytes would have bought half of (K_q halved):
    codes, parameters, promoted contents bit-exact; promotions after the
    query switch."""
    c = _small_drift(quant_bits=4)
    run, seqs = _run_parity(c.replace(k_quant=c.k_quant // 2), torch_cuda, n_splits=splits, check_ledger_every=2,
                            label=f"int4-drift s={splits}")
    assert any(e.promoted for sq in seqs.values() for e in sq.events)


def test_qevict_int4_window32_g8_parity(torch_cuda):
    c = W.STRESS.replace(batch=2, prefill=3000, steps=96, n_q_heads=64, n_kv_heads=8, quant_bits=4)
    w0 = W.w0(c)
    _run_parity(c.replace(k_full=w0 // 4, k_quant=w0 // 2), torch_cuda, n_splits=5, label="int4-w32g8")


def test_qevict_int4_d64_window8_parity(torch_cuda):
    c = W.TINY.replace(batch=2, n_q_heads=8, n_kv_heads=2, prefill=515, steps=40, k_full=10, k_quant=20, quant_bits=4)
    _run_parity(c, torch_cuda, n_splits=4, label="int4-d64w8")


# ---------------------------------------------------------------------------
# the decode step in one call (append folded into the attention launch)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "drift_small", "w32g8", "int4"])
def test_decode_step_parity(torch_cuda, name):
    """qkv_decode_step against the oracle: tiny (d = 64, 8-token windows,
    the new token in a new unit every 8 steps), the small drift layer (3
    splits, promotions), 32-token windows with G = 8 (the token in a
    window's second tile) and the INT4 tier."""
    cfgs = {"tiny": (W.TINY, 0),
            "drift_small": (_small_drift(), 3),
            "w32g8": (W.STRESS.replace(batch=2, prefill=3000, steps=96, n_q_heads=64, n_kv_heads=8,
                                       k_full=W.w0(W.STRESS.replace(prefill=3000, steps=96)) // 4,
                                       k_quant=W.w0(W.STRESS.replace(prefill=3000, steps=96)) // 2), 5),
            "int4": (_small_drift(quant_bits=4), 2)}
    cfg, splits = cfgs[name]
    _run_parity(cfg, torch_cuda, n_splits=splits, check_ledger_every=2, label=f"step-{name}", fused=True)


def test_decode_step_equals_append_then_attend(torch_cuda):
    """The one-call step and the two calls give the same bits: outputs and
    masses every step, tiers, scores, pages and ledgers at the end; a prompt
    shorter than the sink unit puts the first new tokens in the sink unit."""
    torch = torch_cuda
    for cfg in (_small_drift(steps=64), W.TINY.replace(prefill=2, steps=40)):
        K, V, Q = gpu_inputs(cfg, W.Workload(cfg))
        runs = [QEvictGPURun(cfg, K, V, Q, n_splits=3, fused=f) for f in (False, True)]
        for s in range(cfg.steps):
            for r in runs:
                r.step(want_mass=True)
            torch.cuda.synchronize()
            assert torch.equal(runs[0].out, runs[1].out), f"{cfg.name} step {s}: outputs"
            assert torch.equal(runs[0].mass, runs[1].mass), f"{cfg.name} step {s}: masses"
        for what in ("tiers", "scores", "keys", "values", "kcodes", "vcodes", "kparams", "vparams"):
            a, b = runs[0].cache.export(what), runs[1].cache.export(what)
            torch.cuda.synchronize()
            assert torch.equal(a, b), f"{cfg.name}: {what}"
        log(f"[decode-step] {cfg.name}: {cfg.steps} steps bitwise equal to append + attend")


def test_same_inputs_give_the_same_bits(torch_cuda):
    """Two caches fed the same inputs produce the same bits, launch after
    launch: the work of every attention launch is dealt to the waves by
    (split, wave) alone and every reduction runs in a fixed order, also in
    the all-full-precision launches before the first routing event (16
    sequences, 8 KV heads, an 8K prompt: 256 workgroups, as at full size)."""
    torch = torch_cuda
    cfg = _small_drift(batch=16, n_q_heads=32, n_kv_heads=8, prefill=8192, steps=48,
                       cluster_a=(200, 64), cluster_b=(8, 32), switch_step=30)
    K, V, Q = gpu_inputs(cfg, W.Workload(cfg))
    runs = [QEvictGPURun(cfg, K, V, Q, fused=True) for _ in range(2)]
    for s in range(cfg.steps):
        for r in runs:
            r.step(want_mass=True)
        torch.cuda.synchronize()
        assert torch.equal(runs[0].out, runs[1].out), f"step {s}: outputs"
        assert torch.equal(runs[0].mass, runs[1].mass), f"step {s}: masses"
    for what in ("tiers", "scores", "kcodes", "kparams", "keys"):
        a, b = runs[0].cache.export(what), runs[1].cache.export(what)
        torch.cuda.synchronize()
        assert torch.equal(a, b), what
    log(f"[same-bits] {cfg.steps} steps of two caches bitwise equal")


def test_qevict_long_context_parity(torch_cuda):
    """More than 8192 candidate windows at the first routing event (a
    140000-token prompt at 16-token windows: 8744 windows, a 16384-key sort
    that does not fit one key per thread): tiers, ledgers and contents
    bit-exact, outputs and scores to the usual bars."""
    c = W.TINY.replace(prefill=140000, steps=40, window=16, omega=16, n_sink=5, n_recent=32, k_full=100,
                       k_quant=300)
    _run_parity(c, torch_cuda, n_splits=4, label="long-context")


@pytest.mark.parametrize("window,bits", [(16, 2), (8, 2), (16, 4)])
def test_qevict_g8_d128_short_windows_parity(torch_cuda, window, bits):
    """Eight heads per KV head at d = 128 (the Llama-70B head geometry) with
    windows of one tile: a block's quantized windows take two rounds of
    query-limb staging (the LDS of eight waves holds the limbs of two
    windows); ragged prompt, several splits."""
    c = W.STRESS.replace(batch=2, prefill=3000, steps=64, n_q_heads=64, n_kv_heads=8, window=window, omega=window,
                         n_recent=32, quant_bits=bits)
    w0 = W.w0(c)
    c = c.replace(k_full=w0 // 6, k_quant=w0 // 2)
    _run_parity(c, torch_cuda, n_splits=5, check_ledger_every=2, label=f"g8-d128-w{window}-int{bits}")
