"""qkv_create_static (the entry point for callers that cannot allocate):
a cache in the library's own device array gives the same bits as a cache in
caller memory (qkv_create), on two creations in a row on one device, the
second with a smaller configuration; a configuration beyond the array is
refused."""
import numpy as np
import pytest

import workloads as W

from _harness import gpu_inputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_quantization_eviction_amd  # noqa: F401  (raises if the library is missing)
    return torch


def _run(cfg, torch, static):
    from tiered_quantization_eviction_amd import Cache, make_config
    wl = W.Workload(cfg)
    K, V, Q = gpu_inputs(cfg, wl)
    cache = Cache(make_config(cfg), static=static)
    P = cfg.prefill
    out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    mass = torch.zeros((cfg.batch, cfg.n_kv_heads, cache.info("units")), dtype=torch.float32, device="cuda")
    cache.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous())
    outs, masses = [], []
    for s in range(cfg.steps):
        cache.append(K[:, :, P + s:P + s + 1].contiguous(), V[:, :, P + s:P + s + 1].contiguous())
        cache.decode_attend(Q[:, s].contiguous(), out, mass)
        if (s + 1) % cfg.omega == 0:
            cache.route()
        outs.append(out.clone())
        masses.append(mass.clone())
    state = {w: cache.export(w) for w in ("tiers", "scores", "ledger", "kcodes", "vcodes", "kparams", "vparams",
                                          "keys", "values")}
    torch.cuda.synchronize()
    return cache, outs, masses, state


def _compare(cfg, torch, label):
    log(f"[{label}] static vs caller workspace: B={cfg.batch} P={cfg.prefill} steps={cfg.steps}")
    ref, o1, m1, s1 = _run(cfg, torch, static=False)
    st, o2, m2, s2 = _run(cfg, torch, static=True)
    for s, (a, b) in enumerate(zip(o1, o2)):
        assert torch.equal(a, b), f"[{label}] step {s}: outputs differ"
    for s, (a, b) in enumerate(zip(m1, m2)):
        assert torch.equal(a, b), f"[{label}] step {s}: masses differ"
    for w in s1:
        assert torch.equal(s1[w], s2[w]), f"[{label}] exported {w} differs"
    assert st.status() == 0
    log(f"[{label}] identical over {cfg.steps} steps")
    return st


def test_static_cache_matches_caller_workspace_twice(torch_cuda):
    small = W.TINY.replace(batch=2, n_q_heads=8, n_kv_heads=2, prefill=515, steps=40, k_full=10, k_quant=20)
    first = _compare(small, torch_cuda, "static-1")
    # a second, smaller cache on the same device takes over the array
    second = _compare(W.TINY.replace(steps=24), torch_cuda, "static-2")
    assert first.h.value == second.h.value
    second.close()


def test_static_cache_rejects_what_does_not_fit(torch_cuda):
    from tiered_quantization_eviction_amd import Cache, QkvError, make_config
    from tiered_quantization_eviction_amd import _lib as L
    big = make_config(W.DRIFT)
    assert L.workspace_bytes(big) > L.STATIC_WORKSPACE_BYTES
    with pytest.raises(QkvError) as e:
        Cache(big, static=True)
    assert e.value.code == L.ECAPACITY
