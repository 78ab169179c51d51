"""The C ABI's session snapshot and failure paths on the GPU.

* Snapshot and restore (H2O notes section 6.2: a session restore needs the
  heavy/recent boundary, scores, positions and step count; QEvict notes
  section 10h: the ledger lives as long as its window): a cache is exported
  mid-run, a fresh cache imports every kind, and both continue; their
  outputs, tiers, scores, ledgers and contents stay bit-identical, and so do
  those of a third cache of the same run that is never exported (the decode
  path's reduction order is fixed, so repeated runs give the same bits).
  The restored QEvict cache is also followed by the oracle.
* Failure paths (H2O notes section 5.2 asks for them): appending past
  max_ctx, attention or routing before any append, prompt scoring on the
  window policy, an import of the wrong size or of another configuration's
  state, and a quantization parameter outside float16 range met by a routing
  pack (latched in the cache's status, other sequences unaffected).
"""
import numpy as np
import pytest

import workloads as W
from oracle import codec as oc
from oracle import qevict as oe
from oracle.numerics import round_to_bf16_bits

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


class CacheRun:
    """One cache driven through the C ABI the way the benchmark drives it."""

    def __init__(self, cfg, K, V, Q, QP=None, prompt=True):
        import torch
        from tiered_quantization_eviction_amd import Cache, make_config
        self.cfg, self.K, self.V, self.Q, self.QP = cfg, K, V, Q, QP
        self.cache = Cache(make_config(cfg))
        self.out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
        if prompt:
            P = cfg.prefill
            self.cache.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous())
            if cfg.policy != W.POLICY_QEVICT:
                self.cache.prefill_score(QP)
                self.cache.route()

    def step(self, s):
        cfg, P = self.cfg, self.cfg.prefill
        self.cache.append(self.K[:, :, P + s:P + s + 1].contiguous(), self.V[:, :, P + s:P + s + 1].contiguous())
        self.cache.decode_attend(self.Q[:, s].contiguous(), self.out)
        routed = cfg.policy == W.POLICY_H2O or (s + 1) % cfg.omega == 0
        if routed:
            self.cache.route()
        return routed


def _prompt_queries(cfg):
    import torch
    if cfg.policy == W.POLICY_QEVICT:
        return None
    wl = W.Workload(cfg)
    P = cfg.prefill
    m = P if cfg.policy == W.POLICY_H2O else cfg.init_queries
    qp = np.stack([wl.prefill_queries(b, P - m, P) for b in range(cfg.batch)])
    return torch.from_numpy(qp.view(np.int16)).cuda()


def _same_state(torch, a, b, tag):
    for what, t in a.cache.snapshot().items():
        u = b.cache.export(what)
        torch.cuda.synchronize()
        if what == "state":
            # the step scalars agree; nothing else of the state record differs either
            assert torch.equal(t, u), f"{tag}: state record"
            continue
        assert torch.equal(t, u), f"{tag}: exported {what} differs"


def _same_state_within(torch, a, b, tag, rtol):
    """Every kind equal, scores within rtol (exporting the scores of a cache
    with masses pending in list order adds them in early, so the last bits of
    its scores can differ from a cache that adds them at its routing call)."""
    for what, t in a.cache.snapshot().items():
        u = b.cache.export(what)
        torch.cuda.synchronize()
        if what == "scores":
            x, y = t.view(torch.float32), u.view(torch.float32)
            assert torch.allclose(x, y, rtol=rtol, atol=1e-12), f"{tag}: scores differ beyond {rtol}"
            continue
        if what == "state":
            continue
        assert torch.equal(t, u), f"{tag}: exported {what} differs"


def _snapshot_run(cfg, torch, cut, label, oracle_seq=None, pending=False):
    wl = W.Workload(cfg)
    K, V, Q = gpu_inputs(cfg, wl)
    QP = _prompt_queries(cfg)
    log(f"[{label}] snapshot at step {cut} of {cfg.steps}: {cfg.policy} B={cfg.batch} P={cfg.prefill}")
    A = CacheRun(cfg, K, V, Q, QP)          # exported mid-run, then continues
    C = CacheRun(cfg, K, V, Q, QP)          # never exported
    seq = qs = None
    if oracle_seq is not None:
        k, v = wl.kv(oracle_seq)
        seq = oe.QEvictSequence(k, v, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                k_full=cfg.k_full, k_quant=cfg.k_quant, bits=cfg.quant_bits, group=cfg.group,
                                n_q_heads=cfg.n_q_heads)
        seq.prefill(cfg.prefill)
        qs = wl.queries(oracle_seq)
    for s in range(cut):
        A.step(s)
        C.step(s)
        assert torch.equal(A.out, C.out), f"[{label}] step {s}: two runs of the same inputs differ"
        if seq is not None:
            seq.step(s, qs[s])
    snap = A.cache.snapshot()
    torch.cuda.synchronize()
    B = CacheRun(cfg, K, V, Q, QP, prompt=False)
    B.cache.restore(snap)
    for what in ("tokens", "steps", "routes"):
        assert B.cache.info(what) == A.cache.info(what), what
    _same_state(torch, A, B, f"[{label}] right after the restore")
    worst = 0.0
    for s in range(cut, cfg.steps):
        routed = A.step(s)
        B.step(s)
        C.step(s)
        assert torch.equal(A.out, B.out), f"[{label}] step {s}: restored cache differs from the exported one"
        if pending:
            assert torch.allclose(A.out, C.out, rtol=0, atol=1e-5), f"[{label}] step {s}: vs the uninterrupted run"
        else:
            assert torch.equal(A.out, C.out), f"[{label}] step {s}: exported cache differs from the uninterrupted one"
        if seq is not None:
            o, _ = seq.step(s, qs[s])
            err = float(np.abs(B.out[oracle_seq].cpu().numpy() - o).max())
            worst = max(worst, err)
            assert err <= OUT_TOL, f"[{label}] step {s}: restored cache vs oracle {err}"
            if routed:
                torch.cuda.synchronize()
                tiers = B.cache.export("tiers").cpu().numpy().reshape(cfg.batch, -1)
                np.testing.assert_array_equal(tiers[oracle_seq], seq.tier, err_msg=f"[{label}] tiers after step {s}")
    _same_state(torch, A, B, f"[{label}] at the end")
    if pending:
        _same_state_within(torch, A, C, f"[{label}] at the end (uninterrupted)", 1e-6)
    else:
        _same_state(torch, A, C, f"[{label}] at the end (uninterrupted)")
    log(f"[{label}] restored run bit-identical over {cfg.steps - cut} steps; oracle worst {worst:.2e}")
    return seq


def _small_drift(bits=2):
    c = W.DRIFT.replace(name="drift_small", batch=3, n_q_heads=16, n_kv_heads=4, head_dim=128, prefill=2048,
                        steps=160, cluster_a=(60, 24), cluster_b=(4, 12), switch_step=64, quant_bits=bits)
    w0 = W.w0(c)
    return c.replace(k_full=int(0.1 * w0), k_quant=int(0.3 * w0))


@pytest.mark.parametrize("bits", [2, 4])
def test_snapshot_restore_qevict(torch_cuda, bits):
    """Exported mid-window after four routing events (step 70), restored, and
    continued through the query switch and the promotions that follow (INT2
    and INT4 recoverable tiers)."""
    seq = _snapshot_run(_small_drift(bits), torch_cuda, 70, f"qevict{bits}-snapshot", oracle_seq=1)
    assert any(e.promoted for e in seq.events[5:]), "no promotion after the restore"


def test_snapshot_restore_h2o(torch_cuda):
    cfg = W.H2O.replace(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=64, prefill=100, steps=60, n_sink=3,
                        k_full=20, n_recent=17)
    _snapshot_run(cfg, torch_cuda, 29, "h2o-snapshot")


@pytest.mark.parametrize("cut", [64, 90])
def test_snapshot_restore_hqekv(torch_cuda, cut):
    """Right after an assignment event, and in the middle of a period: there
    the masses pending in list order are folded into the exported scores (in
    the exported cache too), so the restored cache is bit-identical to the
    exported one and agrees with a never-exported run to float32 rounding."""
    cfg = W.HQEKV.replace(batch=2, n_q_heads=16, n_kv_heads=4, prefill=1024, steps=160)
    _snapshot_run(cfg, torch_cuda, cut, f"hqekv-snapshot-{cut}", pending=cut % cfg.omega != 0)


def test_import_rejects_wrong_size_and_other_state(torch_cuda):
    import torch
    from tiered_quantization_eviction_amd import Cache, QkvError, make_config
    from tiered_quantization_eviction_amd import _lib as L
    cfg = W.TINY
    a = Cache(make_config(cfg))
    b = Cache(make_config(cfg.replace(k_full=5)))
    h = Cache(make_config(W.H2O.replace(batch=1, prefill=64, steps=8)))
    k = torch.zeros((1, 1, 20, 64), dtype=torch.int16, device="cuda")
    a.append(k, k)
    st = a.export("state")
    torch.cuda.synchronize()
    with pytest.raises(QkvError) as e:
        a.import_("tiers", torch.zeros(7, dtype=torch.uint8, device="cuda"))
    assert e.value.code == L.EINVAL
    # same geometry, same policy: the state record fits a cache of other capacities
    b.import_("state", st)
    assert b.info("tokens") == 20
    # another policy or geometry: rejected, the cache unchanged
    with pytest.raises(QkvError) as e:
        h.import_("state", torch.zeros_like(st))
    assert e.value.code == L.EINVAL
    bad = st.clone().view(torch.int64)
    bad[8] = 10 ** 9                                   # N beyond max_ctx
    with pytest.raises(QkvError) as e:
        a.import_("state", bad.view(torch.uint8))
    assert e.value.code == L.EINVAL and a.info("tokens") == 20
    with pytest.raises(QkvError) as e:            # H2O holds no ledger
        h.export("ledger")
    assert e.value.code == L.EINVAL


# ---------------------------------------------------------------------------
# failure paths
# ---------------------------------------------------------------------------

def test_call_order_and_capacity_errors(torch_cuda):
    import torch
    from tiered_quantization_eviction_amd import Cache, QkvError, make_config
    from tiered_quantization_eviction_amd import _lib as L
    cfg = W.TINY
    for policy_cfg in (cfg, W.H2O.replace(batch=1, prefill=64, steps=8)):
        c = Cache(make_config(policy_cfg))
        q = torch.zeros((1, policy_cfg.n_q_heads, policy_cfg.head_dim), dtype=torch.int16, device="cuda")
        out = torch.zeros((1, policy_cfg.n_q_heads, policy_cfg.head_dim), dtype=torch.float32, device="cuda")
        with pytest.raises(QkvError) as e:
            c.decode_attend(q, out)
        assert e.value.code == L.ESTATE
        with pytest.raises(QkvError) as e:
            c.route()
        assert e.value.code == L.ESTATE
        T = policy_cfg.total_tokens
        k = torch.zeros((1, policy_cfg.n_kv_heads, T, policy_cfg.head_dim), dtype=torch.int16, device="cuda")
        c.append(k, k)
        one = k[:, :, :1].contiguous()
        with pytest.raises(QkvError) as e:
            c.append(one, one)
        assert e.value.code == L.ECAPACITY
        assert c.info("tokens") == T
        c.decode_attend(q, out)                 # the cache still works
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
    # the window policy scores no prompt
    c = Cache(make_config(cfg))
    k = torch.zeros((1, 1, 10, 64), dtype=torch.int16, device="cuda")
    c.append(k, k)
    with pytest.raises(QkvError) as e:
        c.prefill_score(torch.zeros((1, 1, 4, 64), dtype=torch.int16, device="cuda"))
    assert e.value.code == L.ESTATE
    # wrong dtype or shape is refused before the C call
    with pytest.raises(ValueError):
        c.append(k.float(), k.float())
    with pytest.raises(ValueError):
        c.decode_attend(torch.zeros((1, 4, 64), dtype=torch.int16, device="cuda"),
                        torch.zeros((1, 4, 32), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("bad", ["-1e5", "nan", "inf"])
def test_range_error_in_a_routing_pack_is_latched(torch_cuda, bad):
    """Sequence 0 holds one bad value in window 2 (positions 20..27): -1e5,
    whose per-token float16 zero (the group minimum) overflows, or a NaN or
    an infinity (non-finite inputs are refused by every quantizer) when the
    first routing event packs the window (every aged window is quantized
    here).  The status reports QKV_ERANGE from then on; sequence 1 keeps
    matching the oracle, and the oracle refuses sequence 0's window the same
    way."""
    import torch
    from tiered_quantization_eviction_amd import _lib as L
    cfg = W.TINY.replace(batch=2, k_full=0, k_quant=100, steps=24)
    wl = W.Workload(cfg)
    K, V, Q = gpu_inputs(cfg, wl)
    # bfloat16 bits: -1e5 rounded, the quiet NaN 0x7fc0, +infinity 0x7f80
    big = {"-1e5": int(round_to_bf16_bits(np.array([-1e5], np.float32))[0]), "nan": 0x7FC0, "inf": 0x7F80}[bad]
    V[0, 0, 22, 5] = big - 65536 if big > 32767 else big
    d = CacheRun(cfg, K, V, Q)
    k1, v1 = wl.kv(1)
    seq = oe.QEvictSequence(k1, v1, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                            k_full=cfg.k_full, k_quant=cfg.k_quant, n_q_heads=cfg.n_q_heads)
    seq.prefill(cfg.prefill)
    q1 = wl.queries(1)
    assert d.cache.status() == L.OK
    for s in range(cfg.steps):
        routed = d.step(s)
        o, _ = seq.step(s, q1[s])
        torch.cuda.synchronize()
        assert float(np.abs(d.out[1].cpu().numpy() - o).max()) <= OUT_TOL, f"step {s}"
        if routed:
            assert d.cache.status() == L.ERANGE, f"step {s}: range error not latched"
            tiers = d.cache.export("tiers").cpu().numpy().reshape(2, -1)
            np.testing.assert_array_equal(tiers[1], seq.tier)
    # the oracle's quantizer refuses the same window
    k0, v0 = wl.kv(0)
    v0 = v0.copy()
    v0[0, 22, 5] = big
    with pytest.raises(oc.ParamRangeError):
        oc.kivi_quantize_window(oe.bf16_to_f64(k0[:, 20:28]).astype(np.float32),
                                oe.bf16_to_f64(v0[:, 20:28]).astype(np.float32), 2)


def test_hqekv_nan_in_a_requantized_token_is_latched(torch_cuda):
    """HqeKV: a NaN in the value row of 24 tokens spread over the prompt.
    The value range that enters the ranking skips it, so the first
    assignment still ranks every token; those of the 24 it moves to INT4,
    INT2 or INT1 are re-quantized, and their groups latch QKV_ERANGE
    (non-finite inputs are refused by every quantizer).  The same cache
    without the NaN leaves the status clear."""
    import torch
    from tiered_quantization_eviction_amd import Cache, make_config
    from tiered_quantization_eviction_amd import _lib as L
    cfg = W.HQEKV.replace(batch=1, n_q_heads=8, n_kv_heads=2, prefill=640, steps=8)
    wl = W.Workload(cfg)
    K, V, _ = gpu_inputs(cfg, wl)
    P, m = cfg.prefill, cfg.init_queries
    qt = torch.from_numpy(np.stack([wl.prefill_queries(0, P - m, P)]).view(np.int16)).cuda()
    planted = np.arange(7, P - 64, 23)[:24]
    quantized = (6, 4, 7)   # tier codes of INT4, INT2, INT1
    for nan in (False, True):
        v = V.clone()
        if nan:
            v[0, 1, torch.as_tensor(planted), 9] = 0x7FC0   # bfloat16 quiet NaN
        c = Cache(make_config(cfg))
        c.append(K[:, :, :P].contiguous(), v[:, :, :P].contiguous())
        c.prefill_score(qt)
        c.route()
        torch.cuda.synchronize()
        tiers = c.export("tiers").cpu().numpy().reshape(1, 2, -1)[0, 1]
        hit = int(np.isin(tiers[planted], quantized).sum())
        log(f"hqekv NaN={nan}: {hit} of {len(planted)} planted tokens quantized, status {c.status()}")
        if nan:
            assert hit > 0, "no planted token was quantized"
            assert c.status() == L.ERANGE
        else:
            assert c.status() == L.OK
