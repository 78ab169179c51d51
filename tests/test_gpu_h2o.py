"""GPU parity of the H2O token mode with the oracle (through the C ABI).

Per (sequence, KV head): the kept set after the trimmed scored prompt and
after every decode step's eviction must equal the oracle's exactly; the
accumulated scores of the kept tokens must agree to 1e-4 relative; the
attention outputs to 2e-3 max-abs.
"""
import numpy as np
import pytest

import workloads as W
from oracle import h2o as oh

from _harness import gpu_inputs, log

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
SCORE_RTOL = 1e-4
T_SINK, T_RECENT, T_FULL = 1, 2, 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_quantization_eviction_amd  # noqa: F401  (raises if the library is missing)
    return torch


def _run_h2o(cfg, torch, n_splits=0, label=""):
    from tiered_quantization_eviction_amd import Cache, make_config
    wl = W.Workload(cfg)
    B, Hkv, G, d, P = cfg.batch, cfg.n_kv_heads, cfg.group_size, cfg.head_dim, cfg.prefill
    T = cfg.total_tokens
    log(f"[{label}] H2O parity: B={B} Hq={cfg.n_q_heads} Hkv={Hkv} d={d} P={P} steps={cfg.steps} "
        f"sinks={cfg.n_sink} heavy={cfg.k_full} recent={cfg.n_recent} splits={n_splits}")
    K, V, Q = gpu_inputs(cfg, wl)
    qp = np.stack([wl.prefill_queries(b, 0, P) for b in range(B)])          # [B, P, Hq, d]
    cache = Cache(make_config(cfg, n_splits=n_splits))
    out = torch.zeros((B, cfg.n_q_heads, d), dtype=torch.float32, device="cuda")
    cache.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous())
    cache.prefill_score(torch.from_numpy(qp.view(np.int16)).cuda())
    cache.route()

    groups = {}
    for b in range(B):
        k, v = wl.kv(b)
        for g in range(Hkv):
            grp = oh.H2OGroup(k[g], v[g], G=G, n_sink=cfg.n_sink, n_heavy=cfg.k_full, n_recent=cfg.n_recent)
            grp.prefill(P, qp[b][:, g * G:(g + 1) * G])
            groups[b, g] = grp

    def check_sets(tag):
        torch.cuda.synchronize()
        tiers = cache.export("tiers").cpu().numpy().reshape(B, Hkv, T)
        scores = cache.export("scores").cpu().numpy().view(np.float32).reshape(B, Hkv, T)
        for (b, g), grp in groups.items():
            kept = np.flatnonzero((tiers[b, g] == T_SINK) | (tiers[b, g] == T_RECENT) | (tiers[b, g] == T_FULL))
            np.testing.assert_array_equal(kept, np.sort(grp.pos), err_msg=f"{tag}: kept set of (seq {b}, head {g})")
            order = np.argsort(grp.pos)
            np.testing.assert_allclose(scores[b, g, grp.pos[order]], grp.score[order], rtol=SCORE_RTOL, atol=1e-7,
                                       err_msg=f"{tag}: scores of (seq {b}, head {g})")

    def check_log(tag, n_tokens):
        """The eviction record of the step against the oracle's eviction:
        the victim exactly, the margin at the heavy-hitter cut to 2e-4."""
        recs = cache.last_event()
        for (b, g), grp in groups.items():
            r = recs[b * Hkv + g]
            victim = grp.last_victim
            assert r["tokens"] == n_tokens, (tag, r)
            assert r["victims"] == ([] if victim is None else [victim]), f"{tag}: victims of (seq {b}, head {g})"
            m = grp.last_margin
            if np.isinf(m):
                assert np.isinf(r["margin_full"]), (tag, b, g, r)
            else:
                assert abs(r["margin_full"] - m) <= 2 * SCORE_RTOL, f"{tag}: margin {r['margin_full']} vs {m}"

    check_sets("after the trimmed prompt")
    worst = 0.0
    qs = {b: wl.queries(b) for b in range(B)}
    for s in range(cfg.steps):
        t = P + s
        cache.append(K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous())
        cache.decode_attend(Q[:, s].contiguous(), out)
        cache.route()
        torch.cuda.synchronize()
        o_gpu = out.cpu().numpy()
        for (b, g), grp in groups.items():
            o, _, _, _ = grp.step(t, qs[b][s][g * G:(g + 1) * G])
            err = float(np.abs(o_gpu[b, g * G:(g + 1) * G] - o).max())
            worst = max(worst, err)
            assert err <= OUT_TOL, f"step {s} (seq {b}, head {g}): out err {err}"
        check_sets(f"step {s}")
        check_log(f"step {s}", t + 1)
    log(f"[{label}] worst out err {worst:.3e}")


def test_h2o_config_parity(torch_cuda):
    """The H2O workload as specified: one Llama-3.1-8B-shaped layer, 512-token
    scored prompt trimmed to 5 sinks + 48 heavy + 49 recent, 256 steps."""
    _run_h2o(W.H2O, torch_cuda, label="h2o")


@pytest.mark.parametrize("splits", [1, 3])
def test_h2o_small_g8_d64_parity(torch_cuda, splits):
    """G = 8, d = 64, two sequences, ragged tiles, several splits."""
    cfg = W.H2O.replace(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=64, prefill=100, steps=60, n_sink=3,
                        k_full=20, n_recent=17)
    _run_h2o(cfg, torch_cuda, n_splits=splits, label=f"h2o-small-s{splits}")


def test_h2o_no_heavy_hitters_parity(torch_cuda):
    """No heavy-hitter budget: the cache keeps the sinks and the recent
    window only (StreamingLLM)."""
    cfg = W.H2O.replace(batch=1, prefill=200, steps=64, k_full=0)
    _run_h2o(cfg, torch_cuda, label="h2o-kheavy0")


def test_h2o_long_prompt_parity(torch_cuda):
    """A 9000-token scored prompt (one KV head, four query heads; past the
    8192 positions one LDS sort of 8192 keys would hold): the first routing
    call ranks 8867 candidates in one sort of 16384 keys (128 KB of LDS),
    then 12 steps evict one token each; kept sets, scores, outputs and every
    eviction record match the oracle."""
    cfg = W.H2O.replace(batch=1, n_q_heads=4, n_kv_heads=1, prefill=9000, steps=12, n_sink=5, k_full=256,
                        n_recent=128)
    _run_h2o(cfg, torch_cuda, label="h2o-9k")
