"""Multi-layer caches: 32 layers in one cache, one ledger pool for all of them.

QEvict notes section 4.2: one score per layer and window, each layer ranked
by its own scores; sections 4.3 and 4.5 (Eq.(budget), Eq.(3)): the capacities
are what a byte budget over all layers buys, a window costing its bytes in
every layer (qkv_plan_capacities, checked against the oracle's budget
arithmetic in test_abi).  Every layer has its own seeded inputs (the drift
recipe with the layer as the seed).  The oracle follows sampled layers step
by step: outputs within 2e-3, scores within 1e-4 relative, tiers after every
routing event and the ledgers (codes and parameters, through the layered
export) bit for bit.  A 4-layer cache also goes through a snapshot and
restore.
"""
import numpy as np
import pytest

import workloads as W
from oracle import codec as oc
from oracle import qevict as oe

from _harness import gpu_inputs, log

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


def _layered_cfg(L, bits=2):
    from tiered_quantization_eviction_amd import make_config, plan_capacities
    c = W.DRIFT.replace(name="drift_layers", batch=2, n_q_heads=16, n_kv_heads=4, head_dim=128, prefill=2048,
                        steps=96, cluster_a=(60, 24), cluster_b=(4, 12), switch_step=40, quant_bits=bits)
    # a budget of a quarter of the prompt's BF16 bytes over all layers, 70% of
    # the history budget for the quantized tier (the pages' q)
    per_token = L * 2 * c.n_kv_heads * c.head_dim * 2
    budget = 0.25 * c.prefill * per_token
    kf, kq = plan_capacities(make_config(c), budget, 0.7, L)
    return c.replace(k_full=kf, k_quant=kq), budget


class Layered:
    def __init__(self, cfg, L, inputs):
        import torch
        from tiered_quantization_eviction_amd import Cache, make_config
        self.cfg, self.L, self.inputs = cfg, L, inputs
        self.cache = Cache(make_config(cfg, n_layers=L))
        self.out = torch.zeros((L, cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
        P = cfg.prefill
        for l, (K, V, _) in enumerate(inputs):
            self.cache.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous(), layer=l)

    def step(self, s):
        P = self.cfg.prefill
        for l, (K, V, Q) in enumerate(self.inputs):
            self.cache.append(K[:, :, P + s:P + s + 1].contiguous(), V[:, :, P + s:P + s + 1].contiguous(), layer=l)
            self.cache.decode_attend(Q[:, s].contiguous(), self.out[l], layer=l)
        routed = (s + 1) % self.cfg.omega == 0
        if routed:
            self.cache.route()
        return routed


def _layer_inputs(cfg, L):
    ins = []
    for l in range(L):
        c = cfg.replace(seed=l)
        ins.append(gpu_inputs(c, W.Workload(c)))
    return ins


def test_32_layers_share_a_ledger_pool(torch_cuda):
    torch = torch_cuda
    L = 32
    cfg, budget = _layered_cfg(L)
    log(f"[layers] L={L}, budget {budget / 2 ** 20:.1f} MiB -> K_f={cfg.k_full}, K_q={cfg.k_quant} per layer")
    assert cfg.k_full > 0 and cfg.k_quant > cfg.k_full
    inputs = _layer_inputs(cfg, L)
    run = Layered(cfg, L, inputs)
    assert run.cache.info("layers") == L
    U = run.cache.info("units")
    B, H, w, d = cfg.batch, cfg.n_kv_heads, cfg.window, cfg.head_dim
    sampled = [(0, 0), (13, 1), (31, 0), (31, 1)]
    seqs, qs = {}, {}
    for l, b in sampled:
        c = cfg.replace(seed=l)
        wl = W.Workload(c)
        k, v = wl.kv(b)
        seqs[l, b] = oe.QEvictSequence(k, v, window=w, omega=cfg.omega, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                       k_full=cfg.k_full, k_quant=cfg.k_quant, bits=cfg.quant_bits,
                                       group=cfg.group, n_q_heads=cfg.n_q_heads)
        seqs[l, b].prefill(cfg.prefill)
        qs[l, b] = wl.queries(b)
    worst, routes = 0.0, 0
    for s in range(cfg.steps):
        routed = run.step(s)
        torch.cuda.synchronize()
        out = run.out.cpu().numpy()
        for (l, b), sq in seqs.items():
            o, _ = sq.step(s, qs[l, b][s])
            err = float(np.abs(out[l, b] - o).max())
            worst = max(worst, err)
            assert err <= OUT_TOL, f"step {s} layer {l} seq {b}: out err {err}"
        if routed:
            routes += 1
            tiers = run.cache.export("tiers").cpu().numpy().reshape(L, B, U)
            scores = run.cache.export("scores").cpu().numpy().view(np.float32).reshape(L, B, U)
            for (l, b), sq in seqs.items():
                np.testing.assert_array_equal(tiers[l, b], sq.tier, err_msg=f"tiers after step {s}, layer {l} seq {b}")
                np.testing.assert_allclose(scores[l, b], sq.score, rtol=SCORE_RTOL, atol=1e-7,
                                           err_msg=f"scores after step {s}, layer {l} seq {b}")
            if routes in (1, 3, cfg.steps // cfg.omega):
                flags = run.cache.export("ledger").cpu().numpy().reshape(L, B, U)
                kc = run.cache.export("kcodes").cpu().numpy().reshape(L, B, U, H, -1)
                vp = run.cache.export("vparams").cpu().numpy().view(np.uint16).reshape(L, B, U, H, w, d // 32, 2)
                held = int(flags.sum())
                assert held <= L * B * min(cfg.k_full + cfg.k_quant, U), "more ledgers than the pool"
                for (l, b), sq in seqs.items():
                    assert set(np.flatnonzero(flags[l, b])) == set(sq.ledger)
                    for u, Lg in sq.ledger.items():
                        np.testing.assert_array_equal(kc[l, b, u], oc.canonical_k_codes(Lg["kcodes"], cfg.quant_bits))
                        np.testing.assert_array_equal(vp[l, b, u],
                                                      oc.canonical_params(Lg["vscale"], Lg["vzero"]).view(np.uint16))
                log(f"[layers] event {routes}: {held} ledgers held across {L} layers; sampled ledgers bit-exact")
    # layers route on their own scores: their tier vectors differ
    tiers = run.cache.export("tiers").cpu().numpy().reshape(L, B, U)
    assert len({tiers[l, 0].tobytes() for l in range(L)}) > L // 2
    assert run.cache.status() == 0
    log(f"[layers] {routes} events over {cfg.steps} steps; worst out err {worst:.2e}")


def test_layered_snapshot_restore(torch_cuda):
    """A 4-layer cache (INT4 tier) exported mid-run and restored into a fresh
    cache: both continue bit-identically."""
    torch = torch_cuda
    L = 4
    cfg, _ = _layered_cfg(L, bits=4)
    inputs = _layer_inputs(cfg, L)
    A = Layered(cfg, L, inputs)
    for s in range(50):
        A.step(s)
    snap = A.cache.snapshot()
    torch.cuda.synchronize()
    from tiered_quantization_eviction_amd import Cache, make_config
    B = Layered.__new__(Layered)
    B.cfg, B.L, B.inputs = cfg, L, inputs
    B.cache = Cache(make_config(cfg, n_layers=L))
    B.out = torch.zeros_like(A.out)
    B.cache.restore(snap)
    for s in range(50, cfg.steps):
        A.step(s)
        B.step(s)
        assert torch.equal(A.out, B.out), f"step {s}: restored layers differ"
    for what, t in A.cache.snapshot().items():
        assert torch.equal(t, B.cache.export(what)), what
