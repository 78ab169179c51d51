"""H2O heavy-hitter eviction (oracle side).

H2O page:

* section 1.1 -- the new position is appended to form D_t = C_{t-1} + {t};
  attention is normalized over D_t.
* section 1.2 -- the cumulative score of a kept position is the sum of the
  weights it received from its own step on; evicted positions stop
  accumulating; budget B = B_h + B_r, the recent set is the newest B_r
  positions, the heavy set the best B_h older positions.
* section 2.1 -- update order: append, attend on D_t, add the weights to the
  scores, slide the recent window, then evict (at most one per step in the
  online form) the lowest-scored position outside the recent window; the
  step's output uses the pre-eviction set.
* "multi-head and GQA" paragraph and section 5 kernel notes -- with grouped
  query attention the weights of the query heads of one KV group are summed
  into one score per KV head; victims are chosen per (request, KV head).
* prefill: the page leaves open how the prompt enters the budget; from
  section 1.2 (a position accumulates from its own causal row on) the reading
  here is that the prompt is scored token by token (query t attends to
  positions <= t, no eviction), then trimmed once to sinks + newest B_r +
  best B_h.

Sinks (a protected prefix, as in StreamingLLM and the QEvict setup) are never
evicted.  Victim order: lowest score, ties to the oldest position (the
reverse of the shared best-first order of ``oracle.rank``).
"""
from __future__ import annotations

import numpy as np

from .attention import attend
from .numerics import FLT_MIN, bf16_to_f64
from .rank import cut_margins, order


def update_and_evict(positions, scores, weights, *, n_heavy: int, n_recent: int, n_sink: int = 0,
                     budget: int | None = None):
    """One H2O step on given weights (one scoring unit).

    positions/scores: the kept set *including* the newly appended position
    (its score is its weight from this step only); weights: this step's
    attention weights over that set.  Returns (new_scores, victim_position or
    None, kept_positions)."""
    positions = np.asarray(positions, np.int64)
    new = np.asarray(scores, np.float64) + np.asarray(weights, np.float64)
    budget = (n_sink + n_heavy + n_recent) if budget is None else budget
    if len(positions) <= budget:
        return new, None, positions.copy()
    newest = np.sort(positions)[-n_recent:] if n_recent else np.array([], np.int64)
    protected = np.isin(positions, newest) | (positions < n_sink)
    cand = np.flatnonzero(~protected)
    ranked = cand[order(new[cand], positions[cand])]          # best first
    victim = int(ranked[-1])
    keep = np.ones(len(positions), bool)
    keep[victim] = False
    return new, int(positions[victim]), positions[keep]


def eviction_margin(positions, scores, *, n_heavy: int, n_recent: int, n_sink: int = 0) -> float:
    """The relative score gap at the heavy-hitter cut of one H2O step (the
    H2O notes, section 5.1: log how close each eviction was), on the
    updated scores of the kept set including the new position: the same
    candidates update_and_evict ranks, the cut after the best n_heavy;
    +inf when nothing is evicted."""
    positions = np.asarray(positions, np.int64)
    scores = np.asarray(scores, np.float64)
    if len(positions) <= n_sink + n_heavy + n_recent:
        return float("inf")
    newest = np.sort(positions)[-n_recent:] if n_recent else np.array([], np.int64)
    protected = np.isin(positions, newest) | (positions < n_sink)
    cand = np.flatnonzero(~protected)
    return cut_margins(scores[cand], positions[cand], np.ones(len(cand), bool), [n_heavy])[0]


class H2OGroup:
    """H2O state of one (sequence, KV head) scoring unit, G query heads."""

    def __init__(self, k_rows: np.ndarray, v_rows: np.ndarray, *, G: int, n_sink: int,
                 n_heavy: int, n_recent: int):
        self.k = bf16_to_f64(k_rows)          # [T, d] all positions (originals)
        self.v = bf16_to_f64(v_rows)
        self.G = G
        self.n_sink, self.n_heavy, self.n_recent = n_sink, n_heavy, n_recent
        self.budget = n_sink + n_heavy + n_recent
        self.pos = np.zeros(0, np.int64)       # kept positions, in append order
        self.score = np.zeros(0, np.float64)

    def _attend(self, q_bits):
        q = bf16_to_f64(q_bits)                # [G, d]
        out, p = attend(q, self.k[self.pos][None], self.v[self.pos][None])
        w = p.copy()
        w[w < FLT_MIN] = 0.0
        return out, w.sum(axis=0)              # group weight per kept position

    def append(self, t: int):
        self.pos = np.append(self.pos, t)
        self.score = np.append(self.score, 0.0)

    def prefill(self, P: int, q_prompt_bits):
        """Score the prompt token by token with no eviction, then trim."""
        for t in range(P):
            self.append(t)
            _, w = self._attend(q_prompt_bits[t])
            self.score += w
        self.trim()

    def trim(self):
        if len(self.pos) <= self.budget:
            return
        newest = np.sort(self.pos)[-self.n_recent:] if self.n_recent else np.array([], np.int64)
        protected = np.isin(self.pos, newest) | (self.pos < self.n_sink)
        cand = np.flatnonzero(~protected)
        ranked = cand[order(self.score[cand], self.pos[cand])]
        keep = protected.copy()
        keep[ranked[: self.n_heavy]] = True
        self.pos, self.score = self.pos[keep], self.score[keep]

    def step(self, t: int, q_bits):
        """Append position t, attend over D_t, accumulate, evict at most one.

        Returns (out [G, d], weights over D_t, positions of D_t, victim)."""
        self.append(t)
        out, w = self._attend(q_bits)
        d_pos = self.pos.copy()
        new, victim, kept = update_and_evict(self.pos, self.score, w, n_heavy=self.n_heavy,
                                             n_recent=self.n_recent, n_sink=self.n_sink,
                                             budget=self.budget)
        self.last_margin = eviction_margin(self.pos, new, n_heavy=self.n_heavy, n_recent=self.n_recent,
                                           n_sink=self.n_sink)
        self.last_victim = victim
        keep = np.isin(self.pos, kept)
        self.pos, self.score = self.pos[keep], new[keep]
        return out, w, d_pos, victim
