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
the checks of their parity runners.
"""
import pytest

import workloads as W

from _sweep import N_CASES, N_TOKEN_CASES, draw_h2o, draw_hqekv, draw_run
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
