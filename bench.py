"""Decode benchmark of the tiered KV-cache path on one MI355X.

Workload: the QEvict three-tier attention-drift layer -- batch 16, 32K-token
prompt, H_q = 32, H_kv = 8, d = 128, 16-token windows routed every 16 steps,
5 sinks + 64 recent tokens, K_f = 204 full-precision and K_q = 612 INT2 windows,
512 decode steps (synthetic inputs, resident in HBM before timing).

A step is one decode step of the whole path for the batch: append the new
token, attention with fused mass emission and score accumulation, and -- every
Omega steps -- the routing event (rank, pack, promote, evict).

Phases (each timed on its own and reported under "phases"):
* pre_route -- the first Omega steps after the prompt, which end with the
  first routing event: every prompt window is still full precision (2.15 GB
  read per attention step), and the first event packs 612 windows per
  sequence.  A transient of the prompt, measured but not part of `value`.
* steady -- W untimed warm-up steps, then the K timed steps: the routed
  cache, with a routing event every Omega steps.  `value` is its tokens/s and
  `roofline` is taken on its attention launches.
* events -- the routing calls inside the timed steps (rank + pack/promote).

Prints one JSON line.  --gpus N with N > 1 is refused: the benchmark
measures one GPU (how the path would shard is a design, not a measured path).

--workload selects another layer of the same path (the default is the one
above): `stress` (QEvict, batch 32, 128K prompt, G = 8, 32-token windows),
`hqekv` (five-tier per-token assignment, batch 8, 64K prompt), `hqekv_page`
(the same layer with 32-position chunks, scores from the last 20 queries and
an event every 32 tokens), `h2o` (per-token heavy hitters, batch 1,
512-token scored prompt) or `tiny`.  Their lines carry the same fields; their
oracle baseline runs sequence 0 for up to 15 s of decode steps.  The token
policies (H2O, HqeKV) make their first assignment at the end of the prompt,
so their timed steps start routed (no pre_route phase).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# The attention kernel is timed with HIP events on its own stream on every
# PROFILE_STRIDE-th step of the timed region (steps 0, 4, 8, ...): an event
# pair delays the following launch by a few microseconds, so timing every step
# would slow the very loop whose throughput is reported.  The pre-route phase
# is short and reported on its own, so all of its launches are timed.
PROFILE_STRIDE = 4
# The attention kernel is built from these sources; the counter summary is
# only used while their hash matches the one it was taken on.
KERNEL_SRCS = [os.path.join(ROOT, "tiered_quantization_eviction_amd", "csrc", f)
               for f in ("qkv_kernels.hip", "qkv_device.h", "qkv_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_drift_traffic.md")


WORKLOADS = {c.name: c for c in (W.DRIFT, W.DRIFT_INT4, W.DRIFT_L32, W.DRIFT_ROPE, W.DRIFT_G8, W.STRESS,
                                  W.HQEKV, W.HQEKV_PAGE, W.H2O, W.TINY)}
CPU_BUDGET_S = 15.0   # oracle time of the other workloads' bounded samples
DTYPES = {W.POLICY_QEVICT: "bf16+int2 (fp32 accumulate)",
          W.POLICY_H2O: "bf16 (fp32 accumulate)",
          W.POLICY_HQEKV: "bf16+int4+int2+int1 (fp32 accumulate)"}


def describe(cfg, steps, first=0):
    span = f"decode steps {first}..{first + steps - 1} timed" if first else f"{steps} decode steps timed"
    head = (f"batch {cfg.batch}, {cfg.prefill}-token prompt, {span}, "
            f"Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} d={cfg.head_dim}")
    if cfg.name == "drift":
        sw = cfg.switch_step
        inside = ("inside the timed steps" if first <= sw < first + steps else
                  "before the timed steps" if sw < first else "after the timed steps")
        return ("QEvict three-tier attention drift: " + head + ", window=Omega=16, 5 sinks + 64 recent, "
                f"Kf=204 BF16 + Kq=612 INT2 windows (group 32); query switch A->B at step {sw} ({inside})")
    if cfg.policy == W.POLICY_QEVICT and cfg.layers > 1:
        return (f"QEvict three-tier, {cfg.layers} layers in one cache ({cfg.name}): " + head +
                f" per layer, window={cfg.window} Omega={cfg.omega}, {cfg.n_sink} sinks + {cfg.n_recent} recent, "
                f"Kf={cfg.k_full} BF16 + Kq={cfg.k_quant} INT{cfg.quant_bits} windows per layer from a byte budget "
                f"over all layers, one ledger pool; inputs of each layer drawn on the GPU")
    if cfg.policy == W.POLICY_QEVICT:
        rope = (f"; keys before the rotary embedding (table base {cfg.rope_base:g}): pages rotated, ledger packed "
                f"before rotation, quantized tier read rotated" if cfg.rope_base else "")
        return (f"QEvict three-tier ({cfg.name}): " + head + f", window={cfg.window} Omega={cfg.omega}, "
                f"{cfg.n_sink} sinks + {cfg.n_recent} recent, Kf={cfg.k_full} BF16 + Kq={cfg.k_quant} "
                f"INT{cfg.quant_bits} windows" + rope)
    if cfg.policy == W.POLICY_H2O:
        return (f"H2O heavy hitters: " + head + f", scored prompt, {cfg.n_sink} sinks + {cfg.k_full} heavy + "
                f"{cfg.n_recent} recent tokens per KV head, eviction every step")
    rank = (f"chunks of {cfg.chunk} ranked by mean metric (two best BF16)" if cfg.chunk else "per-token ranking")
    scores = (f"scores from the last {cfg.score_window} queries" if cfg.score_window else "accumulated scores")
    return (f"HqeKV five-tier: " + head + f", shares {'/'.join(str(r) for r in cfg.ratios)} "
            f"BF16/INT4/INT2/INT1/evicted by attention x value range, events every {cfg.omega} steps, "
            f"{rank}, {scores}")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def _gen(args):
    cfg, b = args
    wl = W.Workload(cfg)
    k, v = wl.kv(b)
    return k, v, wl.queries(b)


def make_inputs(cfg):
    """K, V [B, Hkv, T, d], Q [B, steps, Hq, d] as bf16 bit patterns."""
    from concurrent.futures import ProcessPoolExecutor
    workers = max(1, min(16, len(os.sched_getaffinity(0)), cfg.batch))
    if workers > 1:
        import multiprocessing as mp
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("fork")) as ex:
            res = list(ex.map(_gen, [(cfg, b) for b in range(cfg.batch)]))
    else:
        res = [_gen((cfg, b)) for b in range(cfg.batch)]
    return (np.stack([r[0] for r in res]), np.stack([r[1] for r in res]), np.stack([r[2] for r in res]))


# ---------------------------------------------------------------------------
# algorithmic bytes of the live cache per step (what one attention launch must read)
# ---------------------------------------------------------------------------

def live_schedule(cfg, steps):
    """Per decode step: (bf16 tokens per KV head, quantized windows per KV
    head) of the live set, following the routing schedule (the counts are the
    same for every sequence)."""
    P, w, ns, nr = cfg.prefill, cfg.window, cfg.n_sink, cfg.n_recent
    unit_of = lambda pos: 0 if pos < ns else 1 + (pos - ns) // w
    start = lambda u: 0 if u == 0 else ns + (u - 1) * w
    N, r0, nF, nQ = P, 1, 0, 0
    out = []
    for s in range(steps):
        N += 1
        r1 = unit_of(N - 1) if N > ns else 0
        recent_tok = max(0, N - start(r0)) if r1 >= r0 else 0
        out.append((min(N, ns) + nF * w + recent_tok, nQ))
        if (s + 1) % cfg.omega == 0:
            limit = N - nr
            aged = (limit - ns) // w if limit > ns else 0
            a1 = max(r0, aged + 1)
            n_cand = nF + nQ + (a1 - r0)
            nF, nQ = min(n_cand, cfg.k_full), min(max(n_cand - cfg.k_full, 0), cfg.k_quant)
            r0 = a1
    return out


def quant_window_bytes(cfg):
    w, d = cfg.window, cfg.head_dim
    return 2 * w * d * cfg.quant_bits // 8 + d * 4 * -(-w // 32) + w * (d // 32) * 4


def attend_bytes(cfg, sched):
    """Algorithmic bytes per attention launch: every live BF16 token (K and V,
    2 bytes each) and every quantized window's codes + parameters, per KV head,
    plus the bf16 queries and the appended token.  With rotary keys, also the table row of each
    quantized window's first position (d/2 float32 (cos, sin) pairs, shared
    by the KV heads of a sequence) and the 16 offset rows."""
    per = []
    rope_row = cfg.head_dim * 4 if cfg.rope_base else 0
    # without rotary keys the step's append is part of the launch: the new
    # token's K and V are read from the input and written to their page
    new_tok = 0 if cfg.rope_base else cfg.batch * cfg.n_kv_heads * cfg.head_dim * 2 * 2 * 2
    for bf_tok, nq in sched:
        kv = cfg.batch * cfg.n_kv_heads * (bf_tok * cfg.head_dim * 4 + nq * quant_window_bytes(cfg))
        kv += cfg.batch * nq * rope_row + (16 * rope_row if nq else 0)
        per.append(kv + cfg.batch * cfg.n_q_heads * cfg.head_dim * 2 + new_tok)
    return per


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------

def run_gpu(cfg, K, V, Q, steps, warmup, n_splits):
    """The pre-route phase (steps 0 .. Omega-1 and the first routing event),
    W warm-up steps, then `steps` timed steps, all on one cache.  Attention
    launches are timed with HIP events attached to the dispatch (every one in
    the pre-route phase, every PROFILE_STRIDE-th in the timed steps); routing
    calls with torch events on the same stream."""
    import torch
    from tiered_quantization_eviction_amd import Cache, make_config
    P, om = cfg.prefill, cfg.omega
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    k_pre = dev(K[:, :, :P])
    v_pre = dev(V[:, :, :P])
    k_dec = dev(np.ascontiguousarray(K[:, :, P:].transpose(2, 0, 1, 3))[:, :, :, None, :])   # [S, B, Hkv, 1, d]
    v_dec = dev(np.ascontiguousarray(V[:, :, P:].transpose(2, 0, 1, 3))[:, :, :, None, :])
    q_dec = dev(np.ascontiguousarray(Q.transpose(1, 0, 2, 3)))                             # [S, B, Hq, d]
    out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    cache = Cache(make_config(cfg, n_splits=n_splits))
    if cfg.rope_base:
        rope = torch.from_numpy(W.Workload(cfg).rope()).cuda()   # the layer's rotary table (a model input)
        cache.set_rope(rope)
    cache.append(k_pre, v_pre)
    ev_route = []

    def loop(s0, n, firsts=None):
        for s in range(s0, s0 + n):
            cache.decode_step(k_dec[s], v_dec[s], q_dec[s], out)   # append + attend (+ merge)
            if firsts is not None and len(firsts) < 4:
                firsts.append(out.clone())
            if (s + 1) % om == 0:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                cache.route()
                e1.record()
                ev_route.append((s, e0, e1))

    # pre-route phase: the all-full-precision steps and the first routing event
    firsts = []
    cache.profile_start(om, 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop(0, om, firsts)
    torch.cuda.synchronize()
    pre_wall = time.perf_counter() - t0
    pre_att = cache.profile_read(om)
    pre_route = [e0.elapsed_time(e1) for _, e0, e1 in ev_route]
    ev_route.clear()
    # warm-up on the routed cache, then the timed steps
    loop(om, warmup)
    s0 = om + warmup
    n_prof = (steps + PROFILE_STRIDE - 1) // PROFILE_STRIDE
    cache.profile_start(n_prof, PROFILE_STRIDE)
    torch.cuda.synchronize()
    ev_route.clear()
    t0 = time.perf_counter()
    loop(s0, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attend_ms = cache.profile_read(n_prof)
    route_ms = [e0.elapsed_time(e1) for _, e0, e1 in ev_route]
    return {"pre_wall": pre_wall, "pre_attend_ms": pre_att, "pre_route_ms": pre_route, "first": s0,
            "wall": wall, "attend_ms": attend_ms, "route_ms": route_ms,
            "firsts": [f[0].cpu().numpy() for f in firsts], "splits": cache.info("splits"),
            "status": cache.status()}


def layered_capacities(cfg):
    """K_f and K_q per layer that a byte budget over all layers buys (the
    library's planner, QEvict notes 4.3 Eq.(3)): the budget is `layers` times
    the bytes one layer of the single-layer workload holds, and q is the share
    its quantized windows take of the history budget."""
    from tiered_quantization_eviction_amd import make_config, plan_capacities
    L, d, w, h = cfg.layers, cfg.head_dim, cfg.window, cfg.n_kv_heads
    per_token = 2 * h * d * 2                                   # one layer, K and V, BF16
    quant = cfg.k_quant * h * quant_window_bytes(cfg)
    hist = cfg.k_full * w * per_token + quant
    budget = L * ((cfg.n_sink + cfg.n_recent) * per_token + hist)
    kf, kq = plan_capacities(make_config(cfg), budget, quant / hist, L)
    return kf, kq, budget, quant / hist


def run_gpu_layers(cfg, steps, warmup, n_splits):
    """The drift layer `cfg.layers` times in one cache, inputs drawn on the GPU
    per layer: per decode step every layer appends its token and attends, and
    every Omega steps one routing call ranks every layer.  Phases as in
    run_gpu; attention launches timed with events every PROFILE_STRIDE-th
    call (calls of all layers counted)."""
    import torch
    from tiered_quantization_eviction_amd import Cache, make_config
    L, P, om = cfg.layers, cfg.prefill, cfg.omega
    cache = Cache(make_config(cfg, n_splits=n_splits, n_layers=L))
    dec = []
    host0 = None
    for l in range(L):
        K, V, Q = W.drift_inputs_torch(cfg, l)
        cache.append(K[:, :, :P].contiguous(), V[:, :, :P].contiguous(), layer=l)
        k_dec = K[:, :, P:].permute(2, 0, 1, 3).contiguous()[:, :, :, None, :]     # [S, B, Hkv, 1, d]
        v_dec = V[:, :, P:].permute(2, 0, 1, 3).contiguous()[:, :, :, None, :]
        q_dec = Q.permute(1, 0, 2, 3).contiguous()                                  # [S, B, Hq, d]
        dec.append((k_dec, v_dec, q_dec))
        if l == 0:   # the oracle leg follows sequence 0 of layer 0
            host0 = (K[:1].cpu().numpy().view(np.uint16), V[:1].cpu().numpy().view(np.uint16),
                     Q[:1].cpu().numpy().view(np.uint16))
        del K, V, Q
        torch.cuda.synchronize()
    out = torch.zeros((L, cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    ev_route = []

    def loop(s0, n, firsts=None):
        for s in range(s0, s0 + n):
            for l, (kd, vd, qd) in enumerate(dec):
                cache.decode_step(kd[s], vd[s], qd[s], out[l], layer=l)
            if firsts is not None and len(firsts) < 4:
                firsts.append(out[0].clone())
            if (s + 1) % om == 0:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                cache.route()
                e1.record()
                ev_route.append((s, e0, e1))

    firsts = []
    cache.profile_start(om * L, 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop(0, om, firsts)
    torch.cuda.synchronize()
    pre_wall = time.perf_counter() - t0
    pre_att = cache.profile_read(om * L)
    pre_route = [e0.elapsed_time(e1) for _, e0, e1 in ev_route]
    ev_route.clear()
    loop(om, warmup)
    s0 = om + warmup
    n_prof = (steps * L + PROFILE_STRIDE - 1) // PROFILE_STRIDE
    cache.profile_start(n_prof, PROFILE_STRIDE)
    torch.cuda.synchronize()
    ev_route.clear()
    t0 = time.perf_counter()
    loop(s0, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attend_ms = cache.profile_read(n_prof)
    route_ms = [e0.elapsed_time(e1) for _, e0, e1 in ev_route]
    return {"pre_wall": pre_wall, "pre_attend_ms": pre_att, "pre_route_ms": pre_route, "first": s0,
            "wall": wall, "attend_ms": attend_ms, "route_ms": route_ms,
            "firsts": [f[0].cpu().numpy() for f in firsts], "splits": cache.info("splits"),
            "status": cache.status(), "host0": host0}


# token modes (H2O, HqeKV): every token is a unit, decisions per (sequence, KV head)
T_SINK, T_RECENT, T_FULL, T_QUANT, T_EVICTED, T_INT4, T_INT1 = 1, 2, 3, 4, 5, 6, 7


def token_bytes_per_token(cfg):
    """Bytes one live token of each tier costs per KV head: bf16 K and V;
    per-token records of codes plus (scale, zero) per 32 channels, or INT1's
    (mean, std), for K and V."""
    d = cfg.head_dim
    return {T_SINK: 4 * d, T_RECENT: 4 * d, T_FULL: 4 * d,
            T_INT4: d + 2 * (d // 32) * 4, T_QUANT: d // 2 + 2 * (d // 32) * 4, T_INT1: d // 4 + 2 * 4}


def prompt_queries(cfg, wl, b):
    """Prompt queries that score the prompt: every position (H2O) or the last
    init_queries positions (HqeKV)."""
    P = cfg.prefill
    m = P if cfg.policy == W.POLICY_H2O else cfg.init_queries
    return wl.prefill_queries(b, P - m, P)


def run_gpu_tok(cfg, K, V, Q, QP, steps, n_splits):
    """Prompt appended, scored and routed before timing; then `steps` decode
    steps (append, attend, route every omega steps) timed.  An untimed pass
    over the same calls on its own cache records the tier histogram after
    every routing call, from which the bytes each attention launch reads are
    counted."""
    import torch
    from tiered_quantization_eviction_amd import Cache, make_config
    P = cfg.prefill
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    k_pre, v_pre = dev(K[:, :, :P]), dev(V[:, :, :P])
    k_dec = dev(np.ascontiguousarray(K[:, :, P:].transpose(2, 0, 1, 3))[:, :, :, None, :])
    v_dec = dev(np.ascontiguousarray(V[:, :, P:].transpose(2, 0, 1, 3))[:, :, :, None, :])
    q_dec = dev(np.ascontiguousarray(Q.transpose(1, 0, 2, 3)))
    qp = dev(QP)
    out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    conf = make_config(cfg, n_splits=n_splits)
    T = cfg.total_tokens

    def start(cache):
        cache.append(k_pre, v_pre)
        cache.prefill_score(qp)
        cache.route()

    route_ev = []
    # routing calls timed with torch events: every one at a period of 16
    # steps or more, every (16 / period)-th below (H2O routes every step, and
    # two event records per step would slow the loop being measured)
    route_stride = max(1, 16 // cfg.omega)
    n_routes = [0]

    def loop(cache, n):
        for s in range(n):
            cache.append(k_dec[s], v_dec[s])
            cache.decode_attend(q_dec[s], out)
            if (s + 1) % cfg.omega == 0:
                if n_routes[0] % route_stride == 0:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    cache.route()
                    e1.record()
                    route_ev.append((e0, e1))
                else:
                    cache.route()
                n_routes[0] += 1

    def hist(cache):
        t = cache.export("tiers").cpu().numpy().reshape(cfg.batch * cfg.n_kv_heads, T)
        return {code: int((t == code).sum()) for code in (T_SINK, T_RECENT, T_FULL, T_INT4, T_QUANT, T_INT1)}

    # counting pass: live tokens per tier before each attention launch
    cc = Cache(conf)
    start(cc)
    per_tok = token_bytes_per_token(cfg)
    state = {"h": hist(cc), "since": 0}
    launch_bytes = []

    def on_route(s):
        state["h"] = hist(cc)
        state["since"] = 0

    for s in range(steps):
        cc.append(k_dec[s], v_dec[s])
        state["since"] += 1
        kv = sum(n * per_tok[code] for code, n in state["h"].items())
        kv += cfg.batch * cfg.n_kv_heads * state["since"] * per_tok[T_RECENT]   # appended since the last route
        launch_bytes.append(kv + cfg.batch * cfg.n_q_heads * cfg.head_dim * 2)
        cc.decode_attend(q_dec[s], out)
        if (s + 1) % cfg.omega == 0:
            cc.route()
            on_route(s)
    torch.cuda.synchronize()
    cc.close()
    del cc

    cache = Cache(conf)
    start(cache)
    n_prof = (steps + PROFILE_STRIDE - 1) // PROFILE_STRIDE
    cache.profile_start(n_prof, PROFILE_STRIDE)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop(cache, steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attend_ms = cache.profile_read(n_prof)
    route_ms = [e0.elapsed_time(e1) for e0, e1 in route_ev]
    return (t1 - t0), attend_ms, launch_bytes, cache.info("splits"), cache.status(), (route_ms, n_routes[0])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def _host_cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def cpu_baseline(cfg, K, V, Q, n_seqs, sample_steps, firsts, budget_s=None):
    """The oracle, as it stands, on the first n_seqs sequences for
    sample_steps decode steps each (prompt handling untimed); with budget_s,
    one sequence for as many steps as fit in that many seconds."""
    from oracle import qevict as oe
    worst = 0.0
    dt = 0.0
    done = 0
    table = W.Workload(cfg).rope() if cfg.rope_base else None
    for b in range(n_seqs):
        seq = oe.QEvictSequence(K[b], V[b], window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink,
                                n_recent=cfg.n_recent, k_full=cfg.k_full, k_quant=cfg.k_quant, bits=cfg.quant_bits,
                                group=cfg.group, n_q_heads=cfg.n_q_heads, rope_table=table)
        seq.prefill(cfg.prefill)
        outs = []
        t0 = time.perf_counter()
        for s in range(sample_steps):
            o, _ = seq.step(s, Q[b, s])
            outs.append(o)
            done += 1
            if budget_s is not None and time.perf_counter() - t0 > budget_s:
                break
        dt += time.perf_counter() - t0
        if b == 0:
            for s, o in enumerate(outs[:len(firsts)]):
                worst = max(worst, float(np.abs(firsts[s] - o).max()))
    per_seq = done // n_seqs
    return {"value": done / dt, "unit": "tokens/s", "cores": _host_cores(), "kind": "oracle",
            "sample": f"sequences 0..{n_seqs - 1} of {cfg.batch}, decode steps 0..{per_seq - 1} each "
                      f"({per_seq // cfg.omega} routing events per sequence), float64 numpy on the host; "
                      f"{dt:.1f} s"}, worst


def cpu_baseline_tok(cfg, K, V, Q, QP, budget_s):
    """The token-mode oracle (one group per KV head) on sequence 0: its
    prompt scored and assigned untimed, then decode steps of all its KV-head
    groups for as many steps as fit in budget_s seconds."""
    G, P = cfg.group_size, cfg.prefill
    groups = []
    for g in range(cfg.n_kv_heads):
        if cfg.policy == W.POLICY_H2O:
            from oracle import h2o as oh
            grp = oh.H2OGroup(K[0, g], V[0, g], G=G, n_sink=cfg.n_sink, n_heavy=cfg.k_full, n_recent=cfg.n_recent)
        else:
            from oracle import hqekv as oq
            ratios32 = tuple(float(np.float32(r)) for r in cfg.ratios)
            grp = oq.HqeKVGroup(K[0, g], V[0, g], G=G, ratios=ratios32, period=cfg.omega, group=cfg.group,
                                window=cfg.score_window, chunk=cfg.chunk)
        grp.prefill(P, QP[0][:, g * G:(g + 1) * G])
        groups.append(grp)
    done = 0
    t0 = time.perf_counter()
    for s in range(cfg.steps):
        for g, grp in enumerate(groups):
            q = Q[0, s][g * G:(g + 1) * G]
            if cfg.policy == W.POLICY_H2O:
                grp.step(P + s, q)
            else:
                grp.step(s, P + s, q)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": _host_cores(), "kind": "oracle",
            "sample": f"sequence 0 of {cfg.batch} ({cfg.n_kv_heads} KV-head groups), decode steps 0..{done - 1} "
                      f"({done // cfg.omega} events), float64 numpy on the host; {dt:.1f} s"}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def read_traffic(src_hash, workload, first, steps):
    """HBM bytes per attention launch from the committed counter summary,
    only if it was taken on the current kernel source, on this workload and
    on the same launches the events time (the routed steps from `first`,
    every PROFILE_STRIDE-th of `steps`).  The summary holds one record per
    launch mix; each record starts at its kernel_source_sha256 field."""
    if workload != "drift":
        return None
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    records = []
    for ln in txt.splitlines():
        if ":" in ln and not ln.startswith(("|", "#", " ")):
            k, v = (x.strip() for x in ln.split(":", 1))
            if k == "kernel_source_sha256":
                records.append({})
            if records:
                records[-1][k] = v
    for f in records:
        try:
            if (f.get("kernel_source_sha256") == src_hash and f.get("launch_mix") == "routed" and
                    int(f.get("first_step", -1)) == first and int(f.get("stride", -1)) == PROFILE_STRIDE and
                    int(f.get("steps", -1)) == steps):
                return float(f["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            continue
    return None


def copy_probe(mib):
    """Five plain device copies of a known size: the HBM byte counters of this
    kernel (read MiB, write MiB per dispatch) calibrate those of the attention
    kernel."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_dispatch": n, "dispatches": 5}), flush=True)


def _phase(bytes_list, ms_list):
    """Average attention launch time (us), its algorithmic bytes and GB/s."""
    if not ms_list:
        return None, None, None
    us = float(np.mean(ms_list)) * 1e3
    b = float(np.mean(bytes_list))
    return us, b, b / (us * 1e-6) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="drift", choices=sorted(WORKLOADS))
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--cpu-steps", type=int, default=512)
    ap.add_argument("--cpu-seqs", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    a = ap.parse_args()
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              f"(how the path would shard across GPUs is a design, not a measured path)", file=sys.stderr)
        sys.exit(2)
    cfg = WORKLOADS[a.workload]
    token_mode = cfg.policy != W.POLICY_QEVICT
    warmup = 0 if token_mode else max(0, min(a.warmup, cfg.steps - cfg.omega - 1))
    lead = 0 if token_mode else cfg.omega + warmup       # decode steps before the timed ones
    steps = max(1, min(a.steps, cfg.steps - lead))
    layered = cfg.layers > 1
    if layered:
        kf, kq, budget, qshare = layered_capacities(cfg)
        cfg = cfg.replace(k_full=kf, k_quant=kq)
        log(f"bench: {cfg.layers} layers; a budget of {budget / 2 ** 30:.2f} GiB per sequence (q = {qshare:.3f}) "
            f"buys K_f = {kf}, K_q = {kq} per layer; inputs drawn on the GPU per layer")
        K = V = Q = None
    else:
        log(f"bench: generating inputs ({cfg.batch} x {cfg.total_tokens} tokens)")
        t = time.perf_counter()
        K, V, Q = make_inputs(cfg)
        log(f"bench: inputs ready in {time.perf_counter() - t:.1f}s; running "
            f"{'a counting pass' if token_mode else f'{cfg.omega} pre-route + {warmup} warm-up'} + "
            f"{steps} timed steps")
    firsts = []
    pre = None
    if token_mode:
        wl = W.Workload(cfg)
        QP = np.stack([prompt_queries(cfg, wl, b) for b in range(cfg.batch)])
        wall, attend_ms, abytes, splits, status, route_ms = run_gpu_tok(cfg, K, V, Q, QP, steps, a.splits)
        first = 0
    else:
        r = (run_gpu_layers(cfg, steps, warmup, a.splits) if layered else
             run_gpu(cfg, K, V, Q, steps, warmup, a.splits))
        if layered:
            K, V, Q = r["host0"]
        wall, attend_ms, firsts, splits, status, route_ms = (r["wall"], r["attend_ms"], r["firsts"], r["splits"],
                                                             r["status"], r["route_ms"])
        first = r["first"]
        # per attention launch (one layer); a decode step holds `layers` of them
        sched_bytes = attend_bytes(cfg, live_schedule(cfg, first + steps))
        launch_bytes = [b for b in sched_bytes for _ in range(cfg.layers)]
        abytes = launch_bytes[first * cfg.layers:]
        pre_us, pre_b, pre_gbps = _phase(launch_bytes[:cfg.omega * cfg.layers], r["pre_attend_ms"])
        pre = {"steps": cfg.omega, "ms_per_step": r["pre_wall"] * 1e3 / cfg.omega,
               "tokens_per_s": cfg.batch * cfg.omega / r["pre_wall"],
               "attention_us": pre_us, "algorithmic_bytes_per_launch": pre_b, "attention_GBps": pre_gbps,
               "attention_frac_of_peak": pre_gbps / HBM_PEAK_GBPS,
               "first_event_us": r["pre_route_ms"][0] * 1e3 if r["pre_route_ms"] else None,
               "timed_launches": f"all {len(r['pre_attend_ms'])}"}
    if status != 0:
        log(f"bench: device status {status}")
    kv_bytes = sum(abytes)
    tok_s = cfg.batch * steps / wall
    sampled = abytes[::PROFILE_STRIDE][:len(attend_ms)]          # the launches that were timed
    att_us, bytes_per_launch, achieved = _phase(sampled, attend_ms)
    src_hash = kernel_source_hash()
    traffic = read_traffic(src_hash, a.workload, first, steps)
    log(f"bench: {wall * 1e3:.1f} ms for {steps} timed steps; attention avg {att_us:.1f} us, "
        f"{achieved:.0f} GB/s algorithmic")
    cpu = None
    worst = None
    if not a.no_cpu and a.workload == "drift":
        n_cpu = min(a.cpu_steps, cfg.steps)
        log(f"bench: oracle baseline on {n_cpu} steps of {a.cpu_seqs} sequences")
        cpu, worst = cpu_baseline(cfg, K, V, Q, a.cpu_seqs, n_cpu, firsts)
    elif not a.no_cpu and layered:
        log(f"bench: oracle baseline on layer 0, sequence 0, up to {CPU_BUDGET_S:.0f} s of decode steps")
        cpu, worst = cpu_baseline(cfg, K, V, Q, 1, cfg.steps, firsts, budget_s=CPU_BUDGET_S)
        cpu["value"] /= cfg.layers     # a decode step of the model is every layer's
        cpu["sample"] = "layer 0 of " + str(cfg.layers) + ", " + cpu["sample"] + "; tokens/s divided by the layers"
    elif not a.no_cpu and token_mode:
        log(f"bench: oracle baseline on sequence 0, up to {CPU_BUDGET_S:.0f} s of decode steps")
        cpu = cpu_baseline_tok(cfg, K, V, Q, QP, CPU_BUDGET_S)
    elif not a.no_cpu:
        log(f"bench: oracle baseline on sequence 0, up to {CPU_BUDGET_S:.0f} s of decode steps")
        cpu, worst = cpu_baseline(cfg, K, V, Q, 1, cfg.steps, firsts, budget_s=CPU_BUDGET_S)
    kernel = ("tok_attend_kernel<%d>" % cfg.head_dim if token_mode else
              "attend_qevict_kernel<%d, %d, %d, %s>" % (cfg.head_dim, 2 if cfg.group_size == 4 else 1,
                                                       cfg.quant_bits, "true" if cfg.rope_base else "false"))
    n_routes = len(route_ms)
    if isinstance(route_ms, tuple):   # token modes: (the timed routing calls, all routing calls)
        route_ms, n_routes = route_ms
    events = {"count": n_routes, "timed": len(route_ms),
              "avg_us": float(np.mean(route_ms)) * 1e3 if route_ms else None,
              "max_us": float(np.max(route_ms)) * 1e3 if route_ms else None,
              "share_of_timed_wall": float(np.mean(route_ms)) * n_routes / 1e3 / wall if route_ms else 0.0}
    steady = {"first_step": first, "steps": steps, "ms_per_step": wall * 1e3 / steps, "tokens_per_s": tok_s,
              "attention_us": att_us, "algorithmic_bytes_per_launch": bytes_per_launch, "attention_GBps": achieved,
              "attention_frac_of_peak": achieved / HBM_PEAK_GBPS,
              "whole_loop_kv_GBps": kv_bytes / wall / 1e9}
    res = {
        "metric": "decode tokens/s + KV-read GB/s (% of HBM peak), 32K ctx, batch 16, 1 layer"
                  if a.workload == "drift" else
                  f"decode tokens/s + KV-read GB/s (% of HBM peak), {cfg.layers} layer{'s' if cfg.layers > 1 else ''}",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[cfg.policy].replace("int2", f"int{cfg.quant_bits}"),
        "data": "synthetic",
        "config": {"workload": describe(cfg, steps, first), "global_batch": cfg.batch,
                   "seq_len": cfg.total_tokens, "parallelism": "single GPU", "attention_splits": splits},
        "kv_read_GBps": kv_bytes / wall / 1e9,
        "kv_read_pct_hbm_peak": 100.0 * kv_bytes / wall / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": att_us,
                     "timed_launches": f"{len(attend_ms)} of the {steps * cfg.layers} attention launches of the "
                                       f"timed steps (every {PROFILE_STRIDE}th, from decode step {first})"},
        "phases": {"pre_route": pre, "steady": steady, "events": events},
        "cpu_baseline": cpu,
        "parity_spot_check_max_abs": worst,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
