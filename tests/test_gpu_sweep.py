"""Seeded random configurations on the GPU against the oracle.

QEvict notes, section 4 (Eq. (1)-(6), Algorithm 1): each case draws the
batch, query heads per KV head, head size, window length, routing period
(also one that is not a multiple of the window), sinks, recent tokens,
capacities, code width, rotary keys and attention splits, then runs prefill
and a few routing events with the per-step checks of the parity runner:
outputs within 2e-3, masses and scores within 1e-4 relative, tiers, event
records, ledgers and full-precision contents exactly.  The token policies
get the same treatment with their own knobs (HqeKV notes sections 3.2-3.10:
tier shares, routing period, prompt queries, rolling score window, chunk
ranking; H2O notes section 2: sinks, heavy-hitter and recent budgets) and
the checks of their parity runners.  Each policy also runs at the most
query heads a cache takes (128).
"""
import pytest

import workloads as W

from _sweep import N_CASES, N_TOKEN_CASES, draw_h2o, draw_hqekv, draw_run, head_limit_cases
from test_gpu_h2o import _run_h2o
from test_gpu_hqekv import _run_hqekv
from test_gpu_qevict import _run_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_quantization_eviction_amd  # noqa: F401  (raises if the library is missing)
    return torch


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_config_parity(torch_cuda, case):
    cfg, splits, opts = draw_run(case)
    _run_parity(cfg, torch_cuda, n_splits=splits, check_ledger_every=1, label=f"sweep{case}", **opts)


@pytest.mark.parametrize("case", range(N_TOKEN_CASES))
def test_random_hqekv_config_parity(torch_cuda, case):
    cfg, splits = draw_hqekv(case)
    _run_hqekv(cfg, torch_cuda, n_splits=splits, label=f"hq_sweep{case}")


@pytest.mark.parametrize("case", range(N_TOKEN_CASES))
def test_random_h2o_config_parity(torch_cuda, case):
    cfg, splits = draw_h2o(case)
    _run_h2o(cfg, torch_cuda, n_splits=splits, label=f"h2o_sweep{case}")


SNAP_CASES = 6


@pytest.mark.parametrize("case", range(SNAP_CASES))
def test_random_config_snapshot_restore(torch_cuda, case):
    """A session exported mid-run and restored into a fresh cache (H2O notes
    section 6.2; QEvict notes section 10h): the restored cache continues
    bit-identical to the exported one and stays with the oracle (window
    policy; cases without rotary keys, whose table the snapshot runner does
    not set)."""
    from test_gpu_boundary import _snapshot_run
    plain = [i for i in range(N_CASES) if draw_run(i)[0].rope_base == 0.0]
    cfg = draw_run(plain[case])[0]
    cut = 1 + (cfg.steps - 2) * (case + 1) // (SNAP_CASES + 1)
    _snapshot_run(cfg, torch_cuda, cut, f"sweep{plain[case]}-snapshot", oracle_seq=0)


@pytest.mark.parametrize("case", range(SNAP_CASES))
def test_random_token_config_snapshot_restore(torch_cuda, case):
    """The same for the token policies, alternating HqeKV and H2O cases; an
    HqeKV cut inside a routing period folds the pending masses into the
    exported scores, so the never-exported run agrees to float32 rounding."""
    from test_gpu_boundary import _snapshot_run
    cfg = (draw_hqekv if case % 2 == 0 else draw_h2o)(case // 2)[0]
    cut = 1 + (cfg.steps - 2) * (case + 1) // (SNAP_CASES + 1)
    pending = cfg.policy == W.POLICY_HQEKV and cut % cfg.omega != 0
    _snapshot_run(cfg, torch_cuda, cut, f"{cfg.name}-snapshot", pending=pending)


LAYER_CASES = 4


@pytest.mark.parametrize("case", range(LAYER_CASES))
def test_random_layered_config_parity(torch_cuda, case):
    """Random window-policy cases as caches of 2 to 5 layers over one ledger
    pool (QEvict notes section 4.2: each layer ranked by its own scores):
    every layer and sequence against the oracle, outputs each step, tiers
    and scores after each routing event."""
    import numpy as np
    from oracle import qevict as oe
    from test_gpu_layers import Layered, _layer_inputs
    torch = torch_cuda
    plain = [i for i in range(N_CASES) if draw_run(i)[0].rope_base == 0.0]
    cfg = draw_run(plain[-1 - case])[0]
    L = 2 + case
    run = Layered(cfg, L, _layer_inputs(cfg, L))
    U = run.cache.info("units")
    seqs, qs = {}, {}
    for l in range(L):
        wl = W.Workload(cfg.replace(seed=l))
        for b in range(cfg.batch):
            k, v = wl.kv(b)
            seqs[l, b] = oe.QEvictSequence(k, v, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink,
                                           n_recent=cfg.n_recent, k_full=cfg.k_full, k_quant=cfg.k_quant,
                                           bits=cfg.quant_bits, group=cfg.group, n_q_heads=cfg.n_q_heads)
            seqs[l, b].prefill(cfg.prefill)
            qs[l, b] = wl.queries(b)
    for s in range(cfg.steps):
        routed = run.step(s)
        torch.cuda.synchronize()
        out = run.out.cpu().numpy()
        for (l, b), sq in seqs.items():
            o, _ = sq.step(s, qs[l, b][s])
            err = float(np.abs(out[l, b] - o).max())
            assert err <= 2e-3, f"step {s} layer {l} seq {b}: out err {err}"
        if routed:
            tiers = run.cache.export("tiers").cpu().numpy().reshape(L, cfg.batch, U)
            scores = run.cache.export("scores").cpu().numpy().view(np.float32).reshape(L, cfg.batch, U)
            for (l, b), sq in seqs.items():
                np.testing.assert_array_equal(tiers[l, b], sq.tier, err_msg=f"tiers after step {s}, layer {l} seq {b}")
                np.testing.assert_allclose(scores[l, b], sq.score, rtol=1e-4, atol=1e-7,
                                           err_msg=f"scores after step {s}, layer {l} seq {b}")
    assert run.cache.status() == 0


@pytest.mark.parametrize("name", sorted(head_limit_cases()))
def test_head_count_limit_parity(torch_cuda, name):
    cfg = head_limit_cases()[name]
    if cfg.policy == W.POLICY_QEVICT:
        _run_parity(cfg, torch_cuda, label=name)
    elif cfg.policy == W.POLICY_HQEKV:
        _run_hqekv(cfg, torch_cuda, label=name)
    else:
        _run_h2o(cfg, torch_cuda, label=name)
