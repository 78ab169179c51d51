"""The ranking order shared by every router (oracle side).

QEvict Eq.(5) ranks candidates by accumulated score, highest first; the H2O
page (section 5.1, small-shape correctness) asks for a fixed tie rule keyed
on the original position.  Reading (the pages give the
key but not its direction): one total order everywhere -- score descending,
then start position descending, so among equal scores the newer unit ranks
higher.  When scores carry no information this degenerates to recency.
"""
from __future__ import annotations

import numpy as np


def order(score: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Indices sorted best-first by (score desc, pos desc)."""
    score = np.asarray(score, np.float64)
    pos = np.asarray(pos, np.int64)
    return np.lexsort((-pos, -score))


def rank_tiers(score, pos, eligible, counts) -> np.ndarray:
    """Assign tiers by rank: the first counts[0] eligible entries (best-first)
    get tier 0, the next counts[1] tier 1, ...; the rest of the eligible
    entries get tier len(counts); ineligible entries get 255."""
    score = np.asarray(score, np.float64)
    pos = np.asarray(pos, np.int64)
    eligible = np.asarray(eligible, bool)
    out = np.full(score.shape, 255, np.uint8)
    idx = np.flatnonzero(eligible)
    ranked = idx[order(score[idx], pos[idx])]
    start = 0
    for t, c in enumerate(counts):
        out[ranked[start:start + c]] = t
        start += c
    out[ranked[start:]] = len(counts)
    return out


def cut_margins(score, pos, eligible, cuts) -> list[float]:
    """Relative score gap across each cut position of the ranking (the
    'margin' the H2O page suggests logging: lowest kept minus highest
    dropped).  Returns +inf where a cut falls outside the candidate list."""
    score = np.asarray(score, np.float64)
    idx = np.flatnonzero(np.asarray(eligible, bool))
    ranked = idx[order(score[idx], np.asarray(pos)[idx])]
    s = score[ranked]
    out = []
    for c in cuts:
        if c <= 0 or c >= len(s):
            out.append(float("inf"))
            continue
        hi, lo = s[c - 1], s[c]
        den = max(abs(hi), abs(lo), 1e-300)
        out.append(float((hi - lo) / den))
    return out
