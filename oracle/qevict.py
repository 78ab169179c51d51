"""QEvict recoverable three-tier routing, one sequence (oracle side).

Follows the QEvict notes:

* section 4.1 -- sinks and a recent region are protected and stay in full
  precision; the rest of the history is cut into consecutive windows; each
  window is Full, Quantized or Evicted; attention reads Full windows and
  dequantized Quantized windows (Eq. attention / state).
* section 4.2, Eq.(1) -- the window score is additive over decode steps,
  never decays, one score per layer and window, summed over query heads and
  the window's tokens (the 1/H_q factor is a positive constant for a layer
  and does not change any ranking; scores here are kept without it).
* section 4.3, Eq.(3) -- capacities K_f and K_q (given directly as counts).
* section 4.4, Eq.(4)-(6) and Algorithm 1 -- every Omega generated tokens the
  candidates (previous Full, previous Quantized, windows that just aged out of
  the recent region) are ranked by score; the top K_f are Full, the next K_q
  Quantized, the rest Evicted.  A window is quantized once, on its first
  demotion, keys per channel / values per token, and the codes are kept in a
  persistent ledger that later demotions reuse; a promoted window is rebuilt
  from the ledger.
* Fig.1 -- all windows start in full precision (and unranked).

Readings where the pages are silent (each also listed in the design notes):

* Steps are 0-based; the routing event follows step s when (s+1) % Omega == 0,
  after that step's attention and score update.
* A window ages out of the recent region when its last position is older than
  the newest n_recent positions (last < N - n_recent, N = tokens so far);
  aged windows join the candidates at the next event.
* Mass accumulates from a token's own step, also while its window is recent
  and also while it is quantized ("not yet scored" = not yet ranked).
* Mass of one head on one window is flushed to 0 when below FLT_MIN (2^-126),
  so that scores that a float32 accumulation cannot distinguish from zero tie
  exactly and fall to the position tie-break.
* Ranking uses the total order of ``oracle.rank``.
* A promoted window's full-precision content is the bfloat16 rounding of its
  dequantized ledger (the original is gone after the first demotion); the
  ledger is kept while the window is Full again.
* Routing is per sequence (one score per window, summed over KV heads), so
  all KV heads of a window share its tier.
* Rotary embedding (``rope``, a table given with the inputs): keys arrive
  before the rotation; the full-precision content read by attention is the
  rotated key (``oracle.rope``), a window's ledger quantizes its original
  unrotated keys, the quantized tier is read as the rotation of the
  dequantized keys at their positions, and a promoted window's content is
  that rotation rounded like a stored key.  Without a table no rotation is
  applied (the synthetic keys of the other workloads carry none).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import rope as rp
from .attention import attend
from .codec import kivi_dequantize_window, kivi_quantize_window
from .numerics import FLT_MIN, bf16_to_f64, round_to_bf16
from .rank import cut_margins, order

EMPTY, SINK, RECENT, FULL, QUANT, EVICTED = 0, 1, 2, 3, 4, 5


@dataclass
class RouteEvent:
    step: int
    n_tokens: int
    candidates: int
    full: list
    quant: list
    evicted: list
    promoted: list
    first_packed: list
    reused: list
    margins: list = field(default_factory=list)


class QEvictSequence:
    """State of one sequence under QEvict routing (float64 arithmetic)."""

    def __init__(self, k_bits: np.ndarray, v_bits: np.ndarray, *, window: int, omega: int,
                 n_sink: int, n_recent: int, k_full: int, k_quant: int, bits: int = 2,
                 group: int = 32, n_q_heads: int, rope_table=None):
        self.korig = bf16_to_f64(k_bits)              # [Hkv, T, d] (before any rotation)
        self.vorig = bf16_to_f64(v_bits)
        self.rope = None if rope_table is None else np.asarray(rope_table, np.float32)
        self.hkv, self.T, self.d = self.korig.shape
        self.hq = n_q_heads
        self.G = n_q_heads // self.hkv
        self.w, self.omega = window, omega
        self.n_sink, self.n_recent = n_sink, n_recent
        self.k_full, self.k_quant = k_full, k_quant
        self.bits, self.group = bits, group
        self.n_units = 1 + math.ceil((self.T - n_sink) / window)
        self.tier = np.full(self.n_units, EMPTY, np.uint8)
        self.score = np.zeros(self.n_units, np.float64)
        self.ledger: dict[int, dict] = {}
        # content currently read by attention, per position (float64 values)
        if self.rope is None:
            self.kcur = self.korig.copy()
        else:
            pos = np.arange(self.korig.shape[1])
            self.kcur = np.stack([rp.rotate_stored(self.korig[g], self.rope, pos) for g in range(self.korig.shape[0])])
        self.vcur = self.vorig.copy()
        self.N = 0
        self.P = 0
        self.events: list[RouteEvent] = []
        pos = np.arange(self.T)
        self.unit_of_pos = np.where(pos < n_sink, 0, 1 + (pos - n_sink) // window)

    # -- geometry -----------------------------------------------------------
    def span(self, u: int) -> tuple[int, int]:
        if u == 0:
            return 0, self.n_sink
        s = self.n_sink + (u - 1) * self.w
        return s, s + self.w

    def start(self, u: int) -> int:
        return self.span(u)[0]

    def last(self, u: int) -> int:
        return self.span(u)[1] - 1

    # -- prefill ------------------------------------------------------------
    def prefill(self, P: int) -> None:
        """All prompt windows start in full precision and unranked (Recent);
        scores are 0.  The first event's candidate pool is then every window
        that has aged out of the recent region, which is the pool Eq.(4) gives
        when the aged prompt windows are counted as the previous Full set."""
        self.P = self.N = P
        # a unit takes a tier once it holds a position: with no sink tokens
        # the sink unit stays empty
        if self.n_sink > 0:
            self.tier[0] = SINK
        for u in range(1, self.unit_of_pos[P - 1] + 1):
            self.tier[u] = RECENT

    # -- one decode step ----------------------------------------------------
    def accessible_mask(self) -> np.ndarray:
        acc_unit = np.isin(self.tier, (SINK, RECENT, FULL, QUANT))
        m = acc_unit[self.unit_of_pos]
        m[self.N:] = False
        return m

    def step(self, s: int, q_bits: np.ndarray):
        """Append the token at position P+s, attend, accumulate, maybe route.

        Returns (out [Hq, d] float64, mass [Hkv, n_units] float64)."""
        pos = self.P + s
        self.N = pos + 1
        u = self.unit_of_pos[pos]
        if self.tier[u] == EMPTY:
            self.tier[u] = SINK if u == 0 else RECENT
        q = bf16_to_f64(q_bits)
        mask = self.accessible_mask()
        n = self.N
        out, p = attend(q, self.kcur[:, :n], self.vcur[:, :n], mask[:n])
        # mass of each head on each unit, flushed below FLT_MIN, summed per KV head
        units = self.unit_of_pos[:n]
        per_head = np.zeros((self.hq, self.n_units))
        for h in range(self.hq):
            per_head[h] = np.bincount(units, weights=p[h], minlength=self.n_units)
        per_head[per_head < FLT_MIN] = 0.0
        mass = per_head.reshape(self.hkv, self.G, self.n_units).sum(axis=1)
        self.score += mass.sum(axis=0)
        if (s + 1) % self.omega == 0:
            self.route(s)
        return out, mass

    # -- routing event (Eq. 4-6, Algorithm 1) ------------------------------
    def _quantize_unit(self, u: int) -> dict:
        # a window is packed on its first demotion only, so its content is
        # still the original (keys before the rotation)
        a, b = self.span(u)
        keys = self.korig if self.rope is not None else self.kcur
        return kivi_quantize_window(keys[:, a:b].astype(np.float32),
                                    self.vcur[:, a:b].astype(np.float32), self.bits, self.group)

    def _rotated(self, kh: np.ndarray, a: int, b: int, stored: bool) -> np.ndarray:
        """Dequantized keys [Hkv, w, d] of positions a..b-1 as attention reads
        them: rotated at their positions when there is a table."""
        if self.rope is None:
            return round_to_bf16(kh) if stored else kh
        pos = np.arange(a, b)
        f = rp.rotate_stored if stored else rp.rotate
        return np.stack([f(kh[g], self.rope, pos) for g in range(kh.shape[0])])

    def route(self, s: int) -> RouteEvent:
        N = self.N
        cand = [u for u in range(1, self.n_units)
                if self.tier[u] in (FULL, QUANT)
                or (self.tier[u] == RECENT and self.last(u) < N - self.n_recent)]
        cand = np.array(cand, np.int64)
        starts = np.array([self.start(u) for u in cand], np.int64)
        ranked = cand[order(self.score[cand], starts)] if len(cand) else cand
        F = ranked[: self.k_full]
        Q = ranked[self.k_full: self.k_full + self.k_quant]
        E = ranked[self.k_full + self.k_quant:]
        ev = RouteEvent(step=s, n_tokens=N, candidates=len(cand), full=sorted(F.tolist()),
                        quant=sorted(Q.tolist()), evicted=sorted(E.tolist()), promoted=[],
                        first_packed=[], reused=[],
                        margins=cut_margins(self.score[cand], starts, np.ones(len(cand), bool),
                                            [self.k_full, self.k_full + self.k_quant]))
        for u in Q.tolist():
            if u not in self.ledger:
                self.ledger[u] = self._quantize_unit(u)
                ev.first_packed.append(u)
            elif self.tier[u] != QUANT:
                ev.reused.append(u)
            a, b = self.span(u)
            kh, vh = kivi_dequantize_window(self.ledger[u])
            self.kcur[:, a:b] = self._rotated(kh, a, b, stored=False)
            self.vcur[:, a:b] = vh
            self.tier[u] = QUANT
        for u in F.tolist():
            if self.tier[u] == QUANT:
                kh, vh = kivi_dequantize_window(self.ledger[u])
                a, b = self.span(u)
                self.kcur[:, a:b] = self._rotated(kh, a, b, stored=True)   # rotated again at its positions
                self.vcur[:, a:b] = round_to_bf16(vh)
                ev.promoted.append(u)
            self.tier[u] = FULL
        for u in E.tolist():
            self.tier[u] = EVICTED
            self.ledger.pop(u, None)
        self.events.append(ev)
        return ev


def run_sequence(cfg, k_bits, v_bits, q_bits, steps: int | None = None, record=False, rope_table=None):
    """Drive one sequence through prefill and ``steps`` decode steps.

    Returns (seq, outs [steps, Hq, d], masses list) -- masses only when
    ``record`` is true."""
    seq = QEvictSequence(k_bits, v_bits, window=cfg.window, omega=cfg.omega, n_sink=cfg.n_sink,
                         n_recent=cfg.n_recent, k_full=cfg.k_full, k_quant=cfg.k_quant,
                         bits=cfg.quant_bits, group=cfg.group, n_q_heads=cfg.n_q_heads, rope_table=rope_table)
    seq.prefill(cfg.prefill)
    steps = cfg.steps if steps is None else steps
    outs = np.zeros((steps, cfg.n_q_heads, cfg.head_dim))
    masses = []
    for s in range(steps):
        o, m = seq.step(s, q_bits[s])
        outs[s] = o
        if record:
            masses.append(m)
    return seq, outs, masses
