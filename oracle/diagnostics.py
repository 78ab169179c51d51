"""Routing diagnostics against full-cache attention (oracle side).

TEST INFRASTRUCTURE: like the rest of ``oracle``, only the tests, the smoke
entry point and the benchmark's CPU-baseline leg may use this module.

The QEvict notes, section 3 (the diagnostic runs made before the mechanism is
proposed), define what is measured here:

* future missed mass (FMM): at a decode step, run attention over the whole
  uncompressed cache (every token so far, full precision); FMM is the part of
  that distribution which falls on tokens the policy has already dropped for
  good;
* observation two splits the same full-cache attention over the tiers a
  policy holds the tokens in (full precision, INT2, evicted);
* selection churn: the Jaccard distance between the sets kept at two
  consecutive routing events;
* global long-term importance recovery (LIR): how often a window that has
  been out of the full-precision set comes back into it.

Readings where the pages leave a choice open (also listed in the design
notes):

* the full-cache attention is taken per query head (GQA: query head h reads
  KV head h // G) and every share is the mean over the query heads;
* dropped means evicted: sinks, recent windows, full-precision and quantized
  windows are all still held (a quantized window is read dequantized);
* churn is reported for the full-precision set and for the kept set (full
  precision together with quantized);
* LIR over a run is re-entries / exits: an exit is a window that is in the
  full-precision set at one event and not at the next; a re-entry is a window
  that enters the set at an event after an exit of its own.  An evicted window
  never returns, so under two tiers every exit is final and LIR is 0.
"""
from __future__ import annotations

import numpy as np

from .attention import attend


def full_attention(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Attention probabilities of q [Hq, d] over every key k [Hkv, N, d]
    (float64, no mask): [Hq, N]."""
    k = np.asarray(k, np.float64)
    _, p = attend(q, k, k)   # (the values play no part in the probabilities)
    return p


def future_missed_mass(p: np.ndarray, held: np.ndarray) -> float:
    """Mean over query heads of the full-cache attention on positions that
    are not held (held [N] bool)."""
    held = np.asarray(held, bool)
    return float(np.mean(p[:, ~held].sum(axis=1)))


def tier_shares(p: np.ndarray, tier_of_pos: np.ndarray, tiers) -> dict:
    """Mean over query heads of the full-cache attention on the positions of
    each tier code in ``tiers`` (tier_of_pos [N])."""
    tier_of_pos = np.asarray(tier_of_pos)
    return {t: float(np.mean(p[:, tier_of_pos == t].sum(axis=1))) for t in tiers}


def jaccard_distance(a, b) -> float:
    """1 - |a & b| / |a | b|; two empty sets are at distance 0."""
    a, b = set(a), set(b)
    union = a | b
    if not union:
        return 0.0
    return 1.0 - len(a & b) / len(union)


def churn(sets) -> list[float]:
    """Jaccard distance of each pair of consecutive sets."""
    sets = [set(s) for s in sets]
    return [jaccard_distance(x, y) for x, y in zip(sets, sets[1:])]


def recovery_counts(full_sets) -> tuple[int, int]:
    """(re-entries, exits) of a sequence of full-precision sets, one per
    routing event."""
    full_sets = [set(s) for s in full_sets]
    exited: set = set()
    exits = re_entries = 0
    for prev, cur in zip(full_sets, full_sets[1:]):
        left = prev - cur
        entered = cur - prev
        re_entries += len(entered & exited)
        exits += len(left)
        exited |= left
    return re_entries, exits


def lir(full_sets) -> float:
    re_entries, exits = recovery_counts(full_sets)
    return re_entries / exits if exits else 0.0
