"""The oracle pinned to what the pages and the mathematics fix (CPU only).

Each test names the passage it checks.  The pins are chosen so that a
plausible slip in the oracle -- a dropped term, a wrong sign or index, a
transposed group axis, a wrong rounding or level count -- fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import budget, codec, h2o, hqekv, rank
from oracle.attention import attend, attend_bruteforce
from oracle.numerics import bf16_to_f64, round_to_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# H2O page, section 2.2: the capacity-6 worked step
# ---------------------------------------------------------------------------

def test_h2o_capacity6_example_scores_victim_cache():
    g = gold("h2o_capacity6_example.json")
    new, victim, kept = h2o.update_and_evict(g["positions"], g["scores_before"], g["weights"],
                                             n_heavy=g["n_heavy"], n_recent=g["n_recent"],
                                             n_sink=g["n_sink"], budget=g["budget"])
    np.testing.assert_allclose(new, g["scores_after"], rtol=0, atol=1e-12)
    assert victim == g["evicted"]
    assert kept.tolist() == g["cache_after"]


def test_h2o_capacity6_example_through_softmax():
    """The same step with the weights produced by attention: logits ln(w)
    (the printed weights sum to 1, so softmax returns them)."""
    g = gold("h2o_capacity6_example.json")
    w = np.array(g["weights"])
    assert abs(w.sum() - 1.0) < 1e-12
    q = np.array([[1.0]])
    k = np.log(w)[None, :, None]                   # d = 1: logit_i = ln w_i
    v = np.zeros_like(k)
    _, p = attend(q, k, v)
    new, victim, kept = h2o.update_and_evict(g["positions"], g["scores_before"], p[0],
                                             n_heavy=3, n_recent=3, budget=6)
    np.testing.assert_allclose(new, g["scores_after"], atol=1e-12)
    assert victim == 8 and kept.tolist() == g["cache_after"]


# ---------------------------------------------------------------------------
# HqeKV notes, section 3.7: the 8-token ranking example
# ---------------------------------------------------------------------------

def test_hqekv_8token_joint_metric_order_and_tiers():
    g = gold("hqekv_8token_example.json")
    m = hqekv.joint_metric(g["acc_attention"], g["value_range"])
    np.testing.assert_allclose(m, g["joint"], atol=5e-4)
    pos = np.arange(8)
    ranked = rank.order(m, pos)
    assert (ranked + 1).tolist() == g["order_1based"]
    counts = hqekv.share_counts(g["ratios"], 8)
    assert counts == [0, 2, 2, 2]
    t = hqekv.assign(m, pos, np.ones(8, bool), counts)
    names = {hqekv.INT4: "int4", hqekv.INT2: "int2", hqekv.INT1: "int1_normal", hqekv.EVICT: "evicted"}
    got = {v: sorted((np.flatnonzero(t == k) + 1).tolist()) for k, v in names.items()}
    for k, v in g["tiers"].items():
        assert got[k] == sorted(v), k


def test_hqekv_example_attention_only_ranking_differs():
    """The example's point: ranking by attention alone would evict t6 and keep
    t7; the joint metric keeps t6 (1-bit) and evicts t7."""
    g = gold("hqekv_8token_example.json")
    a = np.array(g["acc_attention"])
    t_att = hqekv.assign(a, np.arange(8), np.ones(8, bool), [0, 2, 2, 2])
    assert t_att[5] == hqekv.EVICT and t_att[6] != hqekv.EVICT


# ---------------------------------------------------------------------------
# QEvict notes, section 4.5: Eq.(3) worked example; capacity arithmetic
# ---------------------------------------------------------------------------

def test_qevict_eq3_capacity_example():
    g = gold("qevict_capacity_example.json")
    assert budget.kv_bytes_per_token(1, 8, 128, 2) == g["bytes_per_token_per_layer"]
    assert budget.kv_bytes_per_token(g["layers"], 8, 128, 2) == g["bytes_per_token"]
    # M_f of an 8-token window across all layers = 8 * 128 KiB = 1 MiB
    assert g["window"] * g["bytes_per_token"] == 1024 * 1024
    kf, kq = budget.tier_capacities(g["b_hist_mb"], g["q"], g["m_full_mb"], g["m_quant_mb"])
    assert (kf, kq) == (g["k_full"], g["k_quant"])
    assert kf * g["window"] == g["full_tokens"] and kq * g["window"] == g["quant_tokens"]
    # the page rounds M_q; the unrounded 1 MB * 2/16 * 1.05 gives one window fewer
    assert budget.tier_capacities(100, 0.7, 1.0, 2 / 16 * 1.05)[1] == 533


def test_kivi_payload_and_capacity_arithmetic():
    g = gold("payload_examples.json")
    bpe = budget.payload_bytes_per_elem(g["bits"], g["group"], g["param_bytes"])
    assert bpe == g["bytes_per_elem"]
    assert round(2.0 / bpe, 2) == g["compression_vs_bf16"]
    # the oracle's own ledger layout carries exactly that payload at 32-token windows
    assert budget.window_ledger_bytes(32, 128, 2) / (2 * 32 * 128) == g["bytes_per_elem"]
    assert budget.kv_bytes_per_token(32, 8, 128, 2) == g["bytes_per_token"]
    assert g["request_tokens"] * g["bytes_per_token"] == g["request_bytes"]
    assert g["request_tokens"] * budget.kv_bytes_per_token(32, 32, 128, 2) == g["request_bytes_32kv"]
    share = budget.residual_share(g["residual_T"], g["residual_R"], g["bytes_per_elem"])
    assert round(100 * share, 1) == g["residual_share_pct"]
    assert budget.last_page_waste(g["page_T"], 16) == g["waste_16"]
    assert budget.last_page_waste(g["page_T"], 128) == g["waste_128"]
    assert g["waste_16"] * g["bytes_per_token"] / 2 ** 20 == g["waste_16_mib"]
    assert g["waste_128"] * g["bytes_per_token"] / 2 ** 20 == g["waste_128_mib"]


def test_packed_sizes_match_payload():
    """Packed canonical code streams have the bit counts of the payload arithmetic."""
    rng = np.random.default_rng(0)
    for bits in (1, 2, 4):
        c = rng.integers(0, 2 ** bits, size=4096).astype(np.uint8)
        p = codec.pack_codes(c, bits)
        assert p.size == 4096 * bits // 8
        np.testing.assert_array_equal(codec.unpack_codes(p, bits, 4096), c)
    # explicit bit positions: element e at bit 2*(e mod 4) of byte e//4
    p = codec.pack_codes(np.array([1, 2, 3, 0, 3], np.uint8), 2)
    assert p.tolist() == [1 | (2 << 2) | (3 << 4), 3]
    p4 = codec.pack_codes(np.array([0xA, 0x5], np.uint8), 4)
    assert p4.tolist() == [0x5A]


# ---------------------------------------------------------------------------
# HqeKV notes, section 2.3, Eq.(2): the uniform quantizer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
def test_uniform_quantizer_endpoints_and_error_bound(bits):
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal((500, 32)) * rng.uniform(0.1, 20, (500, 1))).astype(np.float32)
    x = bf16_to_f64(np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.float32)
    c, s, z = codec.uniform_quantize(x, bits)
    L = 2 ** bits - 1
    assert c.max() <= L
    # zero = min (Eq.2): the group minimum maps to code 0, the maximum to the top code
    assert np.all(c[np.arange(500), x.argmin(1)] == 0)
    assert np.all(c[np.arange(500), x.argmax(1)] == L)
    xh = codec.uniform_dequantize(c, s, z).astype(np.float64)
    step = (x.max(1) - x.min(1)) / L
    # rounding to the nearest level: error <= step/2, plus the float16 parameter rounding
    slack = np.abs(s.astype(np.float64) - step) * L + np.abs(z.astype(np.float64) - x.min(1)) + 1e-6
    assert np.all(np.abs(xh - x).max(1) <= step / 2 + slack)


def test_uniform_quantizer_degenerate_and_lossless_levels():
    # a constant group: step 0, every code 0, exact reconstruction
    x = np.full((3, 32), 1.5, np.float32)
    c, s, z = codec.uniform_quantize(x, 2)
    assert np.all(c == 0) and np.all(s == 0)
    np.testing.assert_array_equal(codec.uniform_dequantize(c, s, z), x)
    # data on the 4 levels z + k*s (s, z exact in float16): lossless at 2 bits
    rng = np.random.default_rng(1)
    k = rng.integers(0, 4, (64, 32))
    k[:, 0], k[:, 1] = 0, 3
    x = (-0.5 + 0.25 * k).astype(np.float32)
    c, s, z = codec.uniform_quantize(x, 2)
    np.testing.assert_array_equal(c, k)
    np.testing.assert_array_equal(codec.uniform_dequantize(c, s, z), x)


@pytest.mark.parametrize("bad", [2.5e5, -7.0e4, np.nan, np.inf, -np.inf])
def test_quantizers_refuse_parameters_outside_float16(bad):
    """The float16 parameters the pages store cannot hold a step or zero past
    65504, nor a NaN: a 2-bit group of [-1, 1] with 2.5e5 in it (step
    ~83000) or -7e4 (zero -7e4) is refused (ParamRangeError), and so is one
    holding a NaN or an infinity, by the one-bit normalized quantizer too;
    the same group without the value is accepted."""
    x = np.linspace(-1.0, 1.0, 32, dtype=np.float32)[None, :].repeat(2, axis=0)
    codec.uniform_quantize(x, 2)
    codec.int1_normal_quantize(x)
    y = x.copy()
    y[1, 7] = bad
    with np.errstate(invalid="ignore", over="ignore"):
        with pytest.raises(codec.ParamRangeError):
            codec.uniform_quantize(y, 2)
        if not np.isfinite(bad):
            with pytest.raises(codec.ParamRangeError):
                codec.int1_normal_quantize(y)


def test_kivi_groups_keys_per_channel_values_per_token():
    """KV-cache evolution page, section 5: per-channel key groups keep an
    outlier channel from inflating the other channels' steps; values are
    grouped per token."""
    rng = np.random.default_rng(2)
    k = rng.standard_normal((2, 16, 128)).astype(np.float32)
    v = rng.standard_normal((2, 16, 128)).astype(np.float32)
    k[:, :, 7] *= 50.0
    q = codec.kivi_quantize_window(k, v, 2)
    assert q["kscale"].shape == (2, 128, 1) and q["vscale"].shape == (2, 16, 4)
    kh, vh = codec.kivi_dequantize_window(q)
    err = np.abs(kh - k)
    assert err[:, :, 7].max() > 5 * np.delete(err, 7, axis=2).max()
    np.testing.assert_allclose(q["kscale"][:, 7, 0],
                               ((k[:, :, 7].max(1) - k[:, :, 7].min(1)) / 3).astype(np.float16), rtol=1e-3)
    np.testing.assert_allclose(q["vscale"][0, 3, 1],
                               np.float16((v[0, 3, 32:64].max() - v[0, 3, 32:64].min()) / 3), rtol=1e-3)
    # 32-token windows: one key group per channel; 48-token window: two chunks
    q48 = codec.kivi_quantize_window(np.tile(k, (1, 3, 1)), np.tile(v, (1, 3, 1)), 2)
    assert q48["kscale"].shape == (2, 128, 2)


# ---------------------------------------------------------------------------
# HqeKV notes, section 2.3, Eq.(3)-(4) and section 3.4
# ---------------------------------------------------------------------------

def test_normal_quantizer_one_bit_is_sign_test_with_quartile_centres():
    assert abs(0.5 * (1 + math.erf(float(codec.KAPPA1) / math.sqrt(2))) - 0.75) < 1e-7
    rng = np.random.default_rng(3)
    x = bf16_to_f64(np.asarray(rng.standard_normal((200, 128)), np.float32).view(np.uint32) >> 16).astype(np.float32)
    c, m, sd = codec.int1_normal_quantize(x)
    np.testing.assert_array_equal(c, (x > x.astype(np.float64).mean(1, keepdims=True)).astype(np.uint8))
    xh = codec.int1_normal_dequantize(c, m, sd).astype(np.float64)
    lvl = m.astype(np.float64)[:, None] + np.where(c > 0, 1, -1) * 0.6744897501960817 * sd.astype(np.float64)[:, None]
    np.testing.assert_allclose(xh, lvl, rtol=1e-6, atol=1e-6)
    # the general-b quantizer reduces to the same codes at b = 1
    c1, *_ = codec.normal_quantize(x, 1)
    np.testing.assert_array_equal(c1, c)


def test_uniform_vs_normalized_reversal_on_gaussian_vectors():
    """Section 3.4: on Gaussian vectors the normalized quantizer wins at 1 bit
    and the uniform one wins at 4 bits."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2000, 128))
    for bits, uniform_better in ((1, False), (4, True)):
        e_u = np.mean((codec.uniform_roundtrip64(x, bits) - x) ** 2)
        e_n = np.mean((codec.normal_quantize(x, bits)[3] - x) ** 2)
        assert (e_u < e_n) == uniform_better, (bits, e_u, e_n)


# ---------------------------------------------------------------------------
# attention (QEvict 4.1; H2O 1.1)
# ---------------------------------------------------------------------------

def test_attention_matches_bruteforce_and_rows_sum_to_one():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((2, 11, 8))
    v = rng.standard_normal((2, 11, 8))
    mask = rng.random(11) > 0.3
    o, p = attend(q, k, v, mask)
    ob, pb = attend_bruteforce(q, k, v, mask)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(p, pb, atol=1e-12)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
    assert np.all(p[:, ~mask] == 0)
    # removing a position renormalizes the rest (H2O 1.1): masked == gathered subset
    o2, p2 = attend(q, k[:, mask], v[:, mask])
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(p[:, mask], p2, atol=1e-12)


def test_round_to_bf16_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7 + 2 ** -9, -3.0], np.float32)
    np.testing.assert_array_equal(round_to_bf16(x), [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -3.0])


# ---------------------------------------------------------------------------
# HqeKV notes, section 2.3 Eq.(2) with the KIVI grouping of the KV-cache
# evolution page, section 5: per-token quantization in groups of 32
# consecutive channels
# ---------------------------------------------------------------------------

def _grid_token(bits):
    """A 128-channel token whose four 32-channel groups lie on four different
    grids z_j + k * s_j (s_j, z_j exact in float16), each group reaching its
    lowest and highest level, so the expected codes and parameters are known
    without running the quantizer."""
    L = 2 ** bits - 1
    z = np.array([-3.0, 0.5, 10.0, -40.0], np.float32)
    s = np.array([0.25, 1.0, 0.125, 4.0], np.float32)
    rng = np.random.default_rng(7 + bits)
    k = rng.integers(0, L + 1, (4, 32))
    k[:, 3], k[:, 17] = 0, L                       # every group spans its full range
    x = (z[:, None] + k * s[:, None]).astype(np.float32).reshape(128)
    return x, k.reshape(128), s, z


@pytest.mark.parametrize("bits", [2, 4])
def test_per_token_quantize_groups_of_32_channels(bits):
    x, k, s, z = _grid_token(bits)
    c, sc, zc = codec.per_token_quantize(x[None], bits)
    np.testing.assert_array_equal(c[0], k)
    # group j's parameters come from channels [32j, 32j + 32) and nothing else
    np.testing.assert_array_equal(sc[0].astype(np.float32), s)
    np.testing.assert_array_equal(zc[0].astype(np.float32), z)
    np.testing.assert_array_equal(codec.per_token_dequantize(c, sc, zc)[0], x)
    # the pin tells the grouping apart from a strided one (channel c in group c mod 4)
    strided = x.reshape(32, 4).T
    assert not np.array_equal(codec.uniform_quantize(strided, bits)[1].astype(np.float32), s)


def test_per_token_quantize_rows_are_independent():
    """A batch of tokens: each row's parameters depend on that row only."""
    x2, k2, s2, z2 = _grid_token(2)
    x4, k4, s4, z4 = _grid_token(4)
    rows = np.stack([x2, x2 * np.float32(2.0)])
    c, sc, zc = codec.per_token_quantize(rows, 2)
    np.testing.assert_array_equal(c[0], k2)
    np.testing.assert_array_equal(c[1], k2)
    np.testing.assert_array_equal(sc[1].astype(np.float32), 2 * s2)
    np.testing.assert_array_equal(zc[1].astype(np.float32), 2 * z2)


# ---------------------------------------------------------------------------
# HqeKV notes, sections 3.4-3.5: a token moving down re-quantizes its
# current (dequantized) values -- the original is gone once it is quantized
# ---------------------------------------------------------------------------

def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_hqekv_requantize_from_current_values():
    """One 32-channel row [0, 3.0, 2.5, 0, ...] moved to INT4 and then INT2.

    INT4: step fp32(3/15) -> float16 0.199951171875 (= 819/4096), zero 0;
    codes 3/0.19995 = 15.004 -> 15 and 2.5/0.19995 = 12.503 -> 13; values
    15*819/4096 = 2.999267578125 and 13*819/4096 = 2.599365234375.
    INT2 from those: step 2.999267578125/3 = 1 - 2^-12, halfway between the
    float16 neighbours 1 - 2^-11 and 1, rounds to even: 1.0; codes
    rint(2.99927) = 3, rint(2.59937) = 3.
    INT2 of the original row would give rint(2.5/1.0) = 2 (ties to even) at
    channel 2 -- the value this pin rules out."""
    row = np.zeros(32, np.float32)
    row[1], row[2] = 3.0, 2.5
    kb = _bf16(np.stack([row, row]))
    grp = hqekv.HqeKVGroup(kb, kb, G=1, ratios=(1, 0, 0, 0, 0), period=1, group=32)
    grp.tier[:] = hqekv.BF16
    grp._requantize(0, hqekv.INT4)
    tier, kc, ks, kz, vc, vs, vz = grp.codes[0]
    assert tier == hqekv.INT4
    assert kc[:3].tolist() == [0, 15, 13] and float(ks[0]) == 819 / 4096 and float(kz[0]) == 0.0
    assert grp.kcur[0, 1] == 12285 / 4096 and grp.kcur[0, 2] == 10647 / 4096
    grp._requantize(0, hqekv.INT2)
    tier, kc, ks, kz, vc, vs, vz = grp.codes[0]
    assert tier == hqekv.INT2
    assert kc[:3].tolist() == [0, 3, 3] and vc[:3].tolist() == [0, 3, 3]
    assert float(ks[0]) == 1.0 and float(vs[0]) == 1.0
    assert grp.kcur[0, 2] == 3.0 and grp.vcur[0, 2] == 3.0
    # straight from the original the same step gives code 2 at channel 2
    assert codec.per_token_quantize(row, 2)[0][2] == 2
    # a token going straight to INT2 (the other row) does quantize the original
    grp._requantize(1, hqekv.INT2)
    assert grp.codes[1][1][:3].tolist() == [0, 3, 2]


# ---------------------------------------------------------------------------
# FLT_MIN flush (a reading: a head's mass on a unit counts as 0 when the
# unit's sum is below 2^-126; the flush is applied after the sum over the
# unit's tokens, not to each probability)
# ---------------------------------------------------------------------------

def test_qevict_flush_applies_to_unit_sums():
    """One query head, d = 4, q = e_0 (logit = k_0 / 2).  Position 0 holds the
    largest logit 0; window 1 (positions 4..11) holds logits -88.5, each
    probability e^-88.5 = 3.8e-39 below FLT_MIN = 1.18e-38, their sum over the
    window 3.0e-38 above it; window 2 (positions 12..19) holds one token at
    -88.5 (a sum below FLT_MIN).  Per-unit flushing keeps window 1's mass and
    drops window 2's; flushing each probability would drop both."""
    from oracle import qevict as oe
    T, d = 21, 4
    k = np.zeros((1, T, d), np.float32)
    k[0, 1:, 0] = -400.0                       # everything else negligible
    k[0, 4:12, 0] = -177.0                     # logit -88.5
    k[0, 12, 0] = -177.0
    v = np.zeros((1, T, d), np.float32)
    seq = oe.QEvictSequence(_bf16(k), _bf16(v), window=8, omega=100, n_sink=4, n_recent=1,
                            k_full=10, k_quant=10, n_q_heads=1)
    seq.prefill(T - 1)
    q = _bf16(np.array([[1.0, 0, 0, 0]], np.float32))
    _, mass = seq.step(0, q)
    p = math.exp(-88.5) / (1 + 9 * math.exp(-88.5))
    assert p < np.finfo(np.float32).tiny < 8 * p
    assert mass[0, 1] == pytest.approx(8 * p, rel=1e-12)
    assert mass[0, 2] == 0.0
    assert seq.score[1] == pytest.approx(8 * p, rel=1e-12) and seq.score[2] == 0.0


def test_cut_margins_hand_cases():
    """H2O notes section 5.1 (log the cutoff margin of each eviction): the
    relative gap lowest kept minus highest dropped, over the larger of the
    two, at each cut of the (score desc, position desc) ranking; +inf where
    a cut falls outside the list.  Hand cases, including a tie straddling a
    cut (margin 0) and a tie broken by position."""
    from oracle.rank import cut_margins
    m = cut_margins([5.0, 3.0, 3.0, 1.0], [0, 1, 2, 3], [1, 1, 1, 1], [1, 2, 3, 4, 0])
    assert m[0] == 0.4 and m[1] == 0.0 and abs(m[2] - 2.0 / 3.0) < 1e-15
    assert m[3] == float("inf") and m[4] == float("inf")
    # ineligible entries are left out of the ranking
    assert cut_margins([9.0, 4.0, 2.0], [0, 1, 2], [0, 1, 1], [1]) == [0.5]
    # equal scores: the newer position ranks first, the gap is 0
    assert cut_margins([2.0, 2.0, 1.0], [10, 20, 5], [1, 1, 1], [1, 2]) == [0.0, 0.5]


def test_h2o_eviction_margin_hand_case():
    """One sink, two recent, three heavy hitters, seven kept positions after
    the append: positions 1..4 compete, scores 0.5, 0.2, 0.9, 0.3; the best
    three stay (3, 1, 4), position 2 goes, and the gap at the cut is
    (0.3 - 0.2) / 0.3.  With six positions nothing is evicted (+inf)."""
    from oracle import h2o as oh
    pos = np.arange(7)
    sc = np.array([9.0, 0.5, 0.2, 0.9, 0.3, 0.0, 0.0])
    m = oh.eviction_margin(pos, sc, n_heavy=3, n_recent=2, n_sink=1)
    assert abs(m - (0.3 - 0.2) / 0.3) < 1e-15
    new, victim, kept = oh.update_and_evict(pos, sc, np.zeros(7), n_heavy=3, n_recent=2, n_sink=1)
    assert victim == 2 and sorted(kept.tolist()) == [0, 1, 3, 4, 5, 6]
    assert oh.eviction_margin(pos[:6], sc[:6], n_heavy=3, n_recent=2, n_sink=1) == float("inf")
