"""Seeded random window-policy configurations (drift recipe) for the sweep
parity test: every knob the library accepts for the window policy drawn per
case, at sizes the oracle follows step by step."""
import numpy as np

import workloads as W

N_CASES = 48


def draw(case: int) -> tuple:
    """(workload config, attention splits) of sweep case `case`."""
    return draw_run(case)[:2]


def draw_run(case: int) -> tuple:
    """(workload config, attention splits, runner options) of sweep case
    `case`: the one-call decode step instead of append + attend, and how
    often the per-window masses are asked for."""
    r = np.random.default_rng(7100 + case)
    G = int(r.choice([4, 8]))
    hkv = int(r.choice([1, 2, 4]))
    d = int(r.choice([64, 128]))
    window = int(r.choice([8, 16, 32]))
    bits = int(r.choice([2, 4]))
    # rotary keys: windows of at most one tile, and not at d = 128 with G = 8
    rope = bool(window <= 16 and not (d == 128 and G == 8) and r.random() < 0.4)
    prefill = int(r.integers(150, 1600))
    steps = int(r.integers(40, 97))
    omega = int(r.choice([4, 8, 12, 16, 20, 32]))
    n_sink = int(r.integers(0, 17))
    n_recent = int(r.integers(0, 97))
    batch = int(r.integers(1, 4))
    splits = int(r.choice([0, 1, 2, 5]))
    base = W.DRIFT.replace(name=f"sweep{case}", batch=batch, n_q_heads=G * hkv, n_kv_heads=hkv, head_dim=d,
                           prefill=prefill, steps=steps, window=window, omega=omega, n_sink=n_sink,
                           n_recent=n_recent, quant_bits=bits, rope_base=10000.0 if rope else 0.0,
                           seed=case, switch_step=steps // 2)
    w0 = W.w0(base)
    cfg = base.replace(k_full=int(r.uniform(0.0, 0.4) * w0), k_quant=int(r.uniform(0.0, 0.5) * w0),
                       cluster_a=(w0 // 2, max(1, w0 // 6)), cluster_b=(1, max(1, w0 // 8)))
    opts = dict(fused=bool(r.random() < 0.4), mass_every=int(r.choice([1, 1, 3])))
    return cfg, splits, opts


N_TOKEN_CASES = 20


def draw_hqekv(case: int) -> tuple:
    """(HqeKV config, splits): heads, head size, prompt, routing period,
    tier shares (multiples of 1/20, some of them zero), prompt queries,
    rolling score window and chunk ranking drawn per case."""
    r = np.random.default_rng(7300 + case)
    G = int(r.choice([4, 8]))
    hkv = int(r.choice([1, 2, 4]))
    d = int(r.choice([64, 128]))
    prefill = int(r.integers(200, 2500))
    steps = int(r.integers(40, 131))
    omega = int(r.choice([16, 24, 32, 64]))
    parts = r.multinomial(20, r.dirichlet(np.full(5, 0.7)))
    ratios = tuple(float(k) / 20.0 for k in parts)
    score_window = int(r.choice([0, 0, int(r.integers(1, omega + 1))]))
    chunk = int(r.choice([0, 0, 8, 16, 32, 64]))
    cfg = W.HQEKV.replace(name=f"hq_sweep{case}", batch=int(r.integers(1, 3)), n_q_heads=G * hkv, n_kv_heads=hkv,
                          head_dim=d, prefill=prefill, steps=steps, omega=omega, ratios=ratios,
                          init_queries=int(r.integers(1, 33)), score_window=score_window, chunk=chunk, seed=case)
    return cfg, int(r.choice([0, 1, 3]))


def draw_h2o(case: int) -> tuple:
    """(H2O config, splits): heads, head size, prompt, sinks (also none),
    heavy-hitter and recent budgets drawn per case."""
    r = np.random.default_rng(7500 + case)
    G = int(r.choice([4, 8]))
    hkv = int(r.choice([1, 2]))
    d = int(r.choice([64, 128]))
    cfg = W.H2O.replace(name=f"h2o_sweep{case}", batch=int(r.integers(1, 3)), n_q_heads=G * hkv, n_kv_heads=hkv,
                        head_dim=d, prefill=int(r.integers(60, 600)), steps=int(r.integers(30, 81)),
                        n_sink=int(r.integers(0, 17)), k_full=int(r.integers(0, 65)),
                        n_recent=int(r.integers(0, 65)), seed=case)
    return cfg, int(r.choice([0, 1, 3]))


def head_limit_cases() -> dict:
    """The most query heads a cache takes (128), with eight and with four
    query heads per KV head."""
    drift = W.DRIFT.replace(name="heads128", batch=1, prefill=1500, steps=48, cluster_a=(40, 12), cluster_b=(2, 8),
                            switch_step=24)
    return {
        "qevict-g8": drift.replace(n_q_heads=128, n_kv_heads=16, head_dim=128, window=32, omega=32, k_full=6,
                                   k_quant=18),
        "qevict-g4": drift.replace(n_q_heads=128, n_kv_heads=32, head_dim=64, window=16, omega=16, k_full=12,
                                   k_quant=36),
        "hqekv-g4": W.HQEKV.replace(batch=1, n_q_heads=128, n_kv_heads=32, head_dim=64, prefill=800, steps=70,
                                    omega=32),
        "h2o-g8": W.H2O.replace(batch=1, n_q_heads=128, n_kv_heads=16, head_dim=128, prefill=200, steps=40),
    }
