"""HqeKV five-tier assignment (oracle side).

HqeKV notes:

* section 3.2 -- key importance is the accumulated attention weight; value
  importance multiplies it by the token's value range (max - min over the
  channels).  Section 3.7's worked example ranks tokens by this joint product
  and cuts the ranking by the tier shares; reading: one joint ranking per
  token, keys and values share the tier.
* section 3.3, Eq.(6) -- shares of FP16 / 4-bit / 2-bit / 1-bit / evicted;
  the configuration fixes them (the TPE search that would choose them needs a
  calibration model and dataset).
* section 3.4 -- 4- and 2-bit use the uniform quantizer, 1-bit the normalized
  one (``oracle.codec``).
* section 3.5 -- every T generated tokens the cache is re-assigned, and a
  token may only move to a lower precision (never back up).
* section 3.8 / 3.10 -- prefill: importance from the last m = 20 prompt
  queries, then the first assignment.

Readings: granularity is per token (keys too: groups of 32 channels of one
token); scores accumulate over every scoring query (prompt tail and all decode
steps), or, with a rolling window of m queries (sections 3.8 and 3.10: the
metric is kept over the most recent m = 20 queries), over the prompt tail
for the first assignment and then over the last m decode steps before each
event only, the scores starting again from 0 after every event; with chunks
of c tokens (section 3.3's implementation note: the cache is cut into groups
of G = 32 tokens, a group's importance is the mean of its tokens', and the two
most important groups always stay FP16) the eligible live tokens of each run
of c positions form a chunk ranked by the mean of their joint metrics, share
counts are floor(r_k * ceil(N / c)) chunks, the two best chunks get FP16
whatever the shares say, and every token takes its chunk's target; at an event the tokens appended since the previous event keep full
precision and are not ranked; share counts are floor(r_k * N) with N the
number of tokens ever appended, cut in the order FP16, 4-bit, 2-bit, 1-bit,
the rest evicted; a downgraded token is re-quantized from its current
dequantized float32 values.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attend
from .codec import (int1_normal_dequantize, int1_normal_quantize, per_token_dequantize,
                    per_token_quantize)
from .numerics import FLT_MIN, bf16_to_f64
from .rank import cut_margins, order, rank_tiers

BF16, INT4, INT2, INT1, EVICT = 0, 1, 2, 3, 4


def joint_metric(acc_attention, value_range):
    return np.asarray(acc_attention, np.float64) * np.asarray(value_range, np.float64)


def share_counts(ratios, n_total: int):
    return [int(math.floor(r * n_total)) for r in ratios[:4]]


def assign(metric, pos, eligible, counts):
    """Target tier per token by rank of the joint metric (ties: newer first)."""
    return rank_tiers(metric, pos, eligible, counts)


class HqeKVGroup:
    """HqeKV state of one (sequence, KV head): per-token tiers and contents."""

    def __init__(self, k_rows, v_rows, *, G: int, ratios, period: int, group: int = 32, window: int = 0,
                 chunk: int = 0):
        self.korig = bf16_to_f64(k_rows)          # [T, d]
        self.vorig = bf16_to_f64(v_rows)
        self.T, self.d = self.korig.shape
        self.G, self.ratios, self.period, self.group = G, tuple(ratios), period, group
        self.window = window                       # 0: accumulate every step; m: the last m before an event
        self.chunk = chunk                         # 0: rank tokens; c: rank chunks of c positions
        self.kcur = self.korig.copy()
        self.vcur = self.vorig.copy()
        self.tier = np.full(self.T, 255, np.uint8)   # 255: not appended yet
        self.score = np.zeros(self.T)
        vr = self.vorig
        self.range = vr.max(axis=1) - vr.min(axis=1)
        self.N = 0
        self.last_event_N = 0
        self.codes: dict[int, tuple] = {}

    def live(self):
        return np.flatnonzero((self.tier != 255) & (self.tier != EVICT))

    def _attend(self, q_bits, upto: int):
        idx = self.live()
        idx = idx[idx < upto]
        q = bf16_to_f64(q_bits)
        out, p = attend(q, self.kcur[idx][None], self.vcur[idx][None])
        w = p.copy()
        w[w < FLT_MIN] = 0.0
        return out, idx, w.sum(axis=0)

    def prefill(self, P: int, q_tail_bits):
        """Prompt in full precision; the last m prompt queries (m = len of
        q_tail_bits) are scored causally; then the first assignment."""
        self.tier[:P] = BF16
        self.N = P
        m = len(q_tail_bits)
        for i in range(m):
            t = P - m + i
            _, idx, w = self._attend(q_tail_bits[i], t + 1)
            self.score[idx] += w
        self.last_event_N = 0
        self.event()

    def step(self, s: int, t: int, q_bits):
        self.tier[t] = BF16
        self.N = t + 1
        out, idx, w = self._attend(q_bits, self.N)
        if self.window == 0 or s % self.period >= self.period - self.window:
            self.score[idx] += w
        if (s + 1) % self.period == 0:
            self.event()
        return out, idx, w

    def event(self):
        N = self.N
        live = self.live()
        eligible = np.zeros(self.T, bool)
        if self.last_event_N == 0:                 # first assignment: the whole prompt
            eligible[live] = True
        else:                                      # tokens appended before the previous event
            eligible[live[live < self.last_event_N]] = True
        metric = joint_metric(self.score, self.range)
        counts = share_counts(self.ratios, N)
        if self.chunk:
            target = self._chunk_targets(metric, eligible, N)
        else:
            target = assign(metric, np.arange(self.T), eligible, counts)
        end = N if self.last_event_N == 0 else self.last_event_N   # the ranked range of positions
        moved, gone = 0, []
        for t in np.flatnonzero(eligible):
            new = max(int(self.tier[t]), int(target[t]))
            if new > self.tier[t]:
                self._requantize(t, new)
                moved += 1
                if new == EVICT:
                    gone.append(int(t))
        # the event's record (H2O notes section 5.1: what each eviction
        # decided and how close its cuts were): tokens per tier of the
        # ranked range after it, tokens moved down and evicted, and the
        # relative metric gap at each of the four cuts of the token ranking
        cum = np.cumsum(counts).tolist()
        tiers = self.tier[:end]
        self.last_record = {
            "tokens": N, "candidates": int(eligible.sum()),
            "full": int((tiers == BF16).sum()), "int4": int((tiers == INT4).sum()),
            "int2": int((tiers == INT2).sum()), "int1": int((tiers == INT1).sum()),
            "moved": moved, "evicted": len(gone), "requantized": moved - len(gone), "victims": sorted(gone),
            "margins": [float("inf")] * 4 if self.chunk else cut_margins(metric, np.arange(self.T), eligible, cum),
        }
        self.last_event_N = N
        self.last_metric = metric
        if self.window:
            self.score[:] = 0.0

    def _chunk_targets(self, metric, eligible, N):
        """Target tier per token from the rank of its chunk's mean metric."""
        c = self.chunk
        n_chunks = -(-self.T // c)
        cid = np.arange(self.T) // c
        cnt = np.bincount(cid[eligible], minlength=n_chunks)
        tot = np.bincount(cid[eligible], weights=metric[eligible], minlength=n_chunks)
        ranked = cnt > 0
        mean = np.zeros(n_chunks)
        mean[ranked] = tot[ranked] / cnt[ranked]
        self.chunk_mean = np.where(ranked, mean, np.nan)
        tc = assign(mean, np.arange(n_chunks), ranked, share_counts(self.ratios, -(-N // c)))
        idx = np.flatnonzero(ranked)
        best = idx[order(mean[idx], idx)][:2]
        tc[best] = BF16                             # the two most important chunks stay FP16
        target = np.full(self.T, 255, np.uint8)
        target[eligible] = tc[cid[eligible]]
        return target

    def _requantize(self, t: int, new: int):
        if new == EVICT:
            self.tier[t] = EVICT
            self.codes.pop(t, None)
            return
        k32 = self.kcur[t].astype(np.float32)
        v32 = self.vcur[t].astype(np.float32)
        if new in (INT4, INT2):
            bits = 4 if new == INT4 else 2
            kc, ks, kz = per_token_quantize(k32, bits, self.group)
            vc, vs, vz = per_token_quantize(v32, bits, self.group)
            self.kcur[t] = per_token_dequantize(kc, ks, kz, self.group)
            self.vcur[t] = per_token_dequantize(vc, vs, vz, self.group)
            self.codes[t] = (new, kc, ks, kz, vc, vs, vz)
        else:
            kc, km, ksd = int1_normal_quantize(k32)
            vc, vm, vsd = int1_normal_quantize(v32)
            self.kcur[t] = int1_normal_dequantize(kc, km, ksd)
            self.vcur[t] = int1_normal_dequantize(vc, vm, vsd)
            self.codes[t] = (new, kc, km, ksd, vc, vm, vsd)
        self.tier[t] = new
