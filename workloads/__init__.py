"""Seeded synthetic inputs for the tiered decode-attention path.

This module only *produces inputs*: key/value streams and query streams with
the shapes, value distributions and attention structure of the workloads the
pages describe (Llama-3.1-8B-shaped single layers; sink/recent/window
geometry; outlier key channels; drifting attention targets).  It holds none
of the method's arithmetic -- no attention, scoring, quantization or routing
-- so that both the fp64 oracle (``oracle/``) and the HIP path can consume it
without sharing any method code.

Every tensor is drawn from its own PCG64 stream keyed by (seed, recipe id,
sequence, tensor id), so one sequence can be regenerated on its own (the
oracle checks sampled sequences of the large workloads).  Draws are made in
float32 and rounded to bfloat16 (round to nearest even); bfloat16 tensors are
carried as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 carriage (input encoding only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:                                    # fast multithreaded path for large streams
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    except ImportError:                     # pragma: no cover - numpy-only hosts
        u = x.copy().view(np.uint32)
        lsb = np.right_shift(u, 16)
        np.bitwise_and(lsb, 1, out=lsb)
        np.add(lsb, 0x7FFF, out=lsb)
        np.add(u, lsb, out=u)
        np.right_shift(u, 16, out=u)
        return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------

POLICY_QEVICT = "qevict"
POLICY_H2O = "h2o"
POLICY_HQEKV = "hqekv"


@dataclass(frozen=True)
class Config:
    """One workload: model-layer geometry, method parameters, input recipe."""

    name: str
    policy: str
    recipe: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prefill: int
    steps: int
    # QEvict geometry (window = tokens per window, omega = routing period)
    window: int = 1
    omega: int = 1
    n_sink: int = 0
    n_recent: int = 0
    k_full: int = 0          # QEvict: windows kept BF16; H2O: heavy-hitter slots B_h
    k_quant: int = 0         # QEvict: windows kept quantized
    quant_bits: int = 2
    group: int = 32
    # HqeKV: BF16 / INT4 / INT2 / INT1-normal / evict shares
    ratios: tuple = (0.0, 0.0, 0.0, 0.0, 0.0)
    init_queries: int = 0    # HqeKV: prompt queries scored before the first assignment
    score_window: int = 0    # HqeKV: 0 = scores accumulate every step; m = only the last m steps before an event
    chunk: int = 0           # HqeKV: 0 = per-token ranking; c = chunks of c positions ranked by their mean metric
    seed: int = 0
    # recipe knobs
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    cluster_a: tuple = (0, 0)     # drift: (first window, window count)
    cluster_b: tuple = (0, 0)
    switch_step: int = 0
    key_gain: float = 9.5
    side_gain: float = 4.7
    n_clusters: int = 64
    switch_period: int = 200
    layers: int = 1          # layers of one cache (each with its own inputs)
    rope_base: float = 0.0   # rotary embedding of the keys (0: none): table base, queries rotated

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def total_tokens(self) -> int:
        return self.prefill + self.steps

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _w0(prefill: int, n_sink: int, n_recent: int, window: int) -> int:
    """Windows whose last position is older than the protected recent region
    at the end of prefill (the count the tier shares are taken of)."""
    limit = prefill - n_recent          # aged iff last position < limit
    # window j covers [n_sink + j*w, n_sink + (j+1)*w); last = n_sink + (j+1)*w - 1
    return max(0, (limit - n_sink) // window)


CONFIGS: dict[str, Config] = {}


def _reg(c: Config) -> Config:
    CONFIGS[c.name] = c
    return c


# 1: tiny single-layer decode, QEvict, parity config.
TINY = _reg(Config(
    name="tiny", policy=POLICY_QEVICT, recipe="aimed",
    batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, prefill=128, steps=32,
    window=8, omega=8, n_sink=4, n_recent=16, k_full=4, k_quant=4, quant_bits=2,
    outlier_channels=2, outlier_scale=10.0, seed=0))

# 2: H2O per-token heavy-hitter eviction on one Llama-3.1-8B-shaped layer.
#    Budget 20% of 512 = 102 slots = 5 sinks + 48 heavy + 49 recent.
H2O = _reg(Config(
    name="h2o", policy=POLICY_H2O, recipe="aimed",
    batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, prefill=512, steps=256,
    window=1, omega=1, n_sink=5, n_recent=49, k_full=48, k_quant=0,
    outlier_channels=4, outlier_scale=8.0, seed=0))

# 3: QEvict three-tier with attention drift (the measured workload).
_W0_DRIFT = _w0(32768, 5, 64, 16)
DRIFT = _reg(Config(
    name="drift", policy=POLICY_QEVICT, recipe="drift",
    batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, prefill=32768, steps=512,
    window=16, omega=16, n_sink=5, n_recent=64,
    k_full=int(0.10 * _W0_DRIFT), k_quant=int(0.30 * _W0_DRIFT), quant_bits=2,
    cluster_a=(1024, 256), cluster_b=(8, 128), switch_step=100, seed=0))

# 3b: the same layer with a 4-bit recoverable tier at the same bytes: one
#     window and KV head costs 2816 B in INT4 against 1792 B in INT2, so the
#     bytes of 612 INT2 windows hold 389 INT4 windows.
DRIFT_INT4 = _reg(DRIFT.replace(name="drift_int4", quant_bits=4, k_quant=389))

# 3c: 32 layers of the drift layer in one cache (Llama-3.1-8B depth), the
#     per-layer capacities those of a byte budget of 32 times the layer's.
DRIFT_L32 = _reg(DRIFT.replace(name="drift_l32", layers=32))

# 3d: the drift layer with keys before the rotary embedding (Llama-3 table
#     base 500000): pages hold rotated keys, the ledger packs the keys before
#     rotation and the quantized tier is read rotated at its positions.
DRIFT_ROPE = _reg(DRIFT.replace(name="drift_rope", rope_base=500000.0))

# 3e: the drift layer with eight query heads per KV head (Hq = 64, the
#     Llama-70B head geometry) at the same 16-token windows.
DRIFT_G8 = _reg(DRIFT.replace(name="drift_g8", n_q_heads=64))

# 4: HqeKV five-tier per-token assignment.
HQEKV = _reg(Config(
    name="hqekv", policy=POLICY_HQEKV, recipe="hqekv",
    batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, prefill=65536, steps=256,
    window=1, omega=64, ratios=(0.20, 0.30, 0.30, 0.10, 0.10), init_queries=20,
    outlier_channels=4, outlier_scale=8.0, seed=0))

# 4b: HqeKV's page variant: chunks of 32 positions ranked by their mean
#     metric (the two best kept BF16), a rolling window of the last 20
#     queries, an event every 32 tokens.
HQEKV_PAGE = _reg(HQEKV.replace(name="hqekv_page", omega=32, score_window=20, chunk=32))

# 5: long-context stress, G = 8, 32-token windows.
_W0_STRESS = _w0(131072, 5, 32, 32)
STRESS = _reg(Config(
    name="stress", policy=POLICY_QEVICT, recipe="clusters",
    batch=32, n_q_heads=64, n_kv_heads=8, head_dim=128, prefill=131072, steps=1024,
    window=32, omega=32, n_sink=5, n_recent=32,
    k_full=int(0.25 * _W0_STRESS), k_quant=int(0.50 * _W0_STRESS), quant_bits=2,
    n_clusters=64, switch_period=200, seed=0))


def w0(cfg: Config) -> int:
    return _w0(cfg.prefill, cfg.n_sink, cfg.n_recent, cfg.window)


# ---------------------------------------------------------------------------
# rotary embedding table (a model input): frequency i of d/2 is base^(-2i/d),
# the angle of position p is p times it, cos and sin taken in float64 and
# rounded to float32; [n_pos, d/2, 2]
# ---------------------------------------------------------------------------

def rope_table(n_pos: int, d: int, base: float) -> np.ndarray:
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def low_frequency_channels(d: int, base: float, span: int, max_angle: float = 0.3) -> np.ndarray:
    """Channels (i and i + d/2) of the pairs whose angle over `span`
    positions stays below max_angle radians (at least the four slowest pairs)."""
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    pairs = np.flatnonzero(inv * span <= max_angle)
    if len(pairs) < 4:
        pairs = np.argsort(inv)[:4]
    return np.sort(np.concatenate([pairs, pairs + d // 2]))


def _rope_rows_f32(rows: np.ndarray, table: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Model-side rotation of query targets (float32; rotate-half pairing)."""
    h = rows.shape[-1] // 2
    c, s = table[pos, :, 0], table[pos, :, 1]
    lo, hi = rows[..., :h], rows[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1).astype(np.float32)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

_RECIPE_ID = {"aimed": 1, "drift": 3, "hqekv": 4, "clusters": 5}
_T_K, _T_V, _T_Q, _T_PQ, _T_AUX = 1, 2, 3, 4, 5


def _rng(cfg: Config, b: int, tensor) -> np.random.Generator:
    key = (tensor,) if isinstance(tensor, int) else tuple(tensor)
    ss = np.random.SeedSequence(entropy=cfg.seed, spawn_key=(_RECIPE_ID[cfg.recipe], b) + key)
    return np.random.Generator(np.random.PCG64(ss))


def _unit_vectors(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    u = rng.standard_normal((n, d)).astype(np.float64)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    return u.astype(np.float32)


class Workload:
    """Per-sequence synthetic K/V/Q streams for one :class:`Config`."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._kv_cache: dict[int, tuple[np.ndarray, np.ndarray]] = {}

    # -- keys / values ------------------------------------------------------
    def _aux(self, b: int):
        cfg = self.cfg
        rng = _rng(cfg, b, _T_AUX)
        hkv, d = cfg.n_kv_heads, cfg.head_dim
        aux = {}
        if cfg.outlier_channels:
            aux["outliers"] = np.stack([rng.choice(d, cfg.outlier_channels, replace=False) for _ in range(hkv)])
        if cfg.recipe == "drift":
            aux["u_a"] = _unit_vectors(rng, hkv, d)
            aux["u_b"] = _unit_vectors(rng, hkv, d)
            if cfg.rope_base:
                # with rotary keys the clusters live in the channel pairs whose
                # rotation over the whole context stays small (the
                # lowest-frequency pairs): there a cluster direction lines up
                # across all its positions, as without the rotation
                m = np.zeros(d, np.float32)
                m[low_frequency_channels(d, cfg.rope_base, cfg.total_tokens)] = 1.0
                for key in ("u_a", "u_b"):
                    u = aux[key] * m
                    aux[key] = (u / np.linalg.norm(u, axis=-1, keepdims=True)).astype(np.float32)
        if cfg.recipe == "clusters":
            aux["mu"] = np.stack([_unit_vectors(rng, cfg.n_clusters, d) for _ in range(hkv)])   # [hkv, C, d]
            n_win = (cfg.total_tokens - cfg.n_sink + cfg.window - 1) // cfg.window
            p = 1.0 / (np.arange(cfg.n_clusters) + 1.0)
            aux["win_cluster"] = rng.choice(cfg.n_clusters, size=(hkv, n_win), p=p / p.sum())
            n_per = (cfg.steps + cfg.switch_period - 1) // cfg.switch_period
            aux["target"] = rng.integers(0, cfg.n_clusters, size=(n_per,))
        return aux

    def kv(self, b: int) -> tuple[np.ndarray, np.ndarray]:
        """bf16 bits of K and V for every position: two uint16 [Hkv, T, d]."""
        if b in self._kv_cache:
            return self._kv_cache[b]
        cfg = self.cfg
        hkv, T, d = cfg.n_kv_heads, cfg.total_tokens, cfg.head_dim
        aux = self._aux(b)
        k = _rng(cfg, b, _T_K).standard_normal((hkv, T, d), dtype=np.float32)
        v = _rng(cfg, b, _T_V).standard_normal((hkv, T, d), dtype=np.float32)
        if cfg.outlier_channels:
            for g in range(hkv):
                k[g][:, aux["outliers"][g]] *= np.float32(cfg.outlier_scale)
        if cfg.recipe == "drift":
            for (w0_, nw), u in ((cfg.cluster_a, aux["u_a"]), (cfg.cluster_b, aux["u_b"])):
                lo = cfg.n_sink + w0_ * cfg.window
                hi = min(cfg.n_sink + (w0_ + nw) * cfg.window, cfg.prefill)
                if hi > lo:
                    k[:, lo:hi, :] += np.float32(cfg.key_gain) * u[:, None, :]
        if cfg.recipe == "clusters":
            pos = np.arange(cfg.n_sink, T)
            win = (pos - cfg.n_sink) // cfg.window
            for g in range(hkv):
                k[g, cfg.n_sink:, :] += np.float32(cfg.key_gain) * aux["mu"][g][aux["win_cluster"][g][win]]
        if cfg.recipe == "hqekv":
            sig = np.exp(0.5 * _rng(cfg, b, _T_AUX + 10).standard_normal((hkv, T, 1))).astype(np.float32)
            v *= sig
        out = (f32_to_bf16_bits(k), f32_to_bf16_bits(v))
        self._kv_cache.clear()          # keep at most one sequence resident
        self._kv_cache[b] = out
        return out

    # -- queries ------------------------------------------------------------
    def _aimed(self, b: int, positions: np.ndarray, tensor, lo=None, hi=None) -> np.ndarray:
        """q_h = 2 k_j + N(0,1), j uniform over positions <= the query's own
        (or over [lo, hi) when given).  With a rotary table the target is the
        rotated key k_j at its position: queries are given already rotated."""
        cfg = self.cfg
        kb, _ = self.kv(b)
        rng = _rng(cfg, b, tensor)
        n = len(positions)
        hq, d, G = cfg.n_q_heads, cfg.head_dim, cfg.group_size
        if lo is None:
            j = np.floor(rng.random((n, hq)) * (positions[:, None] + 1)).astype(np.int64)
        else:
            j = (lo[:, None] + np.floor(rng.random((n, hq)) * (hi - lo)[:, None])).astype(np.int64)
        noise = rng.standard_normal((n, hq, d), dtype=np.float32)
        g = np.arange(hq) // G
        tgt = bf16_bits_to_f32(kb[g[None, :], j, :])                            # only the target keys
        if cfg.rope_base:
            tgt = _rope_rows_f32(tgt, self.rope(), j)
        return f32_to_bf16_bits(np.float32(2.0) * tgt + noise)

    def rope(self) -> np.ndarray:
        """The rotary table of this workload ([total_tokens, d/2, 2] float32)."""
        return rope_table(self.cfg.total_tokens, self.cfg.head_dim, self.cfg.rope_base)

    def queries(self, b: int) -> np.ndarray:
        """bf16 bits of the decode-step queries: uint16 [steps, Hq, d]."""
        cfg = self.cfg
        hq, d, G = cfg.n_q_heads, cfg.head_dim, cfg.group_size
        if cfg.recipe in ("aimed", "hqekv"):
            return self._aimed(b, cfg.prefill + np.arange(cfg.steps), _T_Q)
        aux = self._aux(b)
        rng = _rng(cfg, b, _T_Q)
        noise = rng.standard_normal((cfg.steps, hq, d), dtype=np.float32)
        g = np.arange(hq) // G
        if cfg.recipe == "drift":
            s = np.arange(cfg.steps)[:, None, None]
            ua, ub = aux["u_a"][g][None], aux["u_b"][g][None]
            hi_, lo_ = np.float32(cfg.key_gain), np.float32(cfg.side_gain)
            tgt = np.where(s < cfg.switch_step, hi_ * ua + lo_ * ub, hi_ * ub + lo_ * ua)
            if cfg.rope_base:
                # queries are given rotated at their own positions
                pos = cfg.prefill + np.arange(cfg.steps)
                tgt = _rope_rows_f32(np.broadcast_to(tgt, (cfg.steps, hq, d)),
                                     self.rope(), np.broadcast_to(pos[:, None], (cfg.steps, hq)))
            q = tgt + noise
            return f32_to_bf16_bits(q.astype(np.float32))
        if cfg.recipe == "clusters":
            tgt = aux["target"][np.arange(cfg.steps) // cfg.switch_period]       # [steps]
            mu = aux["mu"][g[None, :], tgt[:, None]]                              # [steps, hq, d]
            return f32_to_bf16_bits(np.float32(cfg.key_gain) * mu + noise)
        raise ValueError(cfg.recipe)

    def prefill_queries(self, b: int, t0: int, t1: int) -> np.ndarray:
        """Queries for prompt positions t0..t1-1 (scored prefill): [t1-t0, Hq, d].

        Each prompt position has its own stream, so any slice is reproducible
        without drawing the whole prompt's queries."""
        if self.cfg.recipe not in ("aimed", "hqekv"):
            raise ValueError("scored prefill is defined for the aimed-query recipes")
        out = [self._aimed(b, np.array([t]), (_T_PQ, t))[0] for t in range(t0, t1)]
        return np.stack(out) if out else np.zeros((0, self.cfg.n_q_heads, self.cfg.head_dim), np.uint16)

    # -- whole batch --------------------------------------------------------
    def kv_all(self) -> tuple[np.ndarray, np.ndarray]:
        ks, vs = zip(*(self.kv(b) for b in range(self.cfg.batch)))
        return np.stack(ks), np.stack(vs)

    def queries_all(self) -> np.ndarray:
        return np.stack([self.queries(b) for b in range(self.cfg.batch)])


# ---------------------------------------------------------------------------
# the drift recipe drawn on the GPU (for many-layer runs, where drawing every
# layer on the host would take minutes): the same structure -- N(0,1) keys and
# values, two key clusters along per-(sequence, KV head) unit vectors, queries
# aimed at one cluster with the other as a side target, roles swapped at the
# switch step -- from torch's generator seeded by (seed, layer); not the same
# numbers as the host recipe
# ---------------------------------------------------------------------------

def drift_inputs_torch(cfg: Config, layer: int, device="cuda"):
    """K, V [B, Hkv, T, d] and Q [B, steps, Hq, d] as int16 (bf16 bits) on `device`."""
    import torch
    if cfg.recipe != "drift":
        raise ValueError("drift_inputs_torch draws the drift recipe")
    B, Hkv, T, d, S, Hq, G = (cfg.batch, cfg.n_kv_heads, cfg.total_tokens, cfg.head_dim, cfg.steps,
                              cfg.n_q_heads, cfg.group_size)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000003 * cfg.seed + 7919 * layer + 17)
    unit = lambda: torch.nn.functional.normalize(torch.randn((B, Hkv, d), generator=gen, device=device), dim=-1)
    u_a, u_b = unit(), unit()
    K = torch.empty((B, Hkv, T, d), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    for b in range(B):                       # one sequence at a time (float32 draws)
        k = torch.randn((Hkv, T, d), generator=gen, device=device)
        for (w0_, nw), u in ((cfg.cluster_a, u_a[b]), (cfg.cluster_b, u_b[b])):
            lo = cfg.n_sink + w0_ * cfg.window
            hi = min(cfg.n_sink + (w0_ + nw) * cfg.window, cfg.prefill)
            if hi > lo:
                k[:, lo:hi, :] += cfg.key_gain * u[:, None, :]
        K[b] = k.to(torch.bfloat16)
        V[b] = torch.randn((Hkv, T, d), generator=gen, device=device).to(torch.bfloat16)
    g = torch.arange(Hq, device=device) // G
    ua, ub = u_a[:, g], u_b[:, g]                       # [B, Hq, d]
    before = cfg.key_gain * ua + cfg.side_gain * ub
    after = cfg.key_gain * ub + cfg.side_gain * ua
    s = torch.arange(S, device=device)[None, :, None, None]
    noise = torch.randn((B, S, Hq, d), generator=gen, device=device)
    Q = (torch.where(s < cfg.switch_step, before[:, None], after[:, None]) + noise).to(torch.bfloat16)
    return K.view(torch.int16), V.view(torch.int16), Q.view(torch.int16)
