"""Capacity and payload arithmetic (oracle side).

* QEvict notes section 4.3, Eq.(3): K_f = floor((1-q) B_hist / M_f),
  K_q = floor(q B_hist / M_q); section 4.5 works it for Llama-3.1-8B geometry.
* KV-cache evolution page section 2: per-token KV payload 2 * L * H_kv * d * b.
* section 5 (KIVI): average payload w/8 + s/g bytes per element for w-bit
  codes, groups of g elements and s parameter bytes per group.
* section 10.3: share of BF16 payload for a quantized body plus an R-token
  high-precision residual.
* section 10.7: slots wasted in the last page of a T-token request.
"""
from __future__ import annotations

import math


def tier_capacities(b_hist: float, q: float, m_full: float, m_quant: float) -> tuple[int, int]:
    return int(math.floor((1.0 - q) * b_hist / m_full)), int(math.floor(q * b_hist / m_quant))


def kv_bytes_per_token(layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * n_kv_heads * head_dim * elem_bytes


def payload_bytes_per_elem(bits: int, group: int, param_bytes: int) -> float:
    return bits / 8.0 + param_bytes / group


def residual_share(tokens: int, residual: int, avg_bytes: float, full_bytes: float = 2.0) -> float:
    return ((tokens - residual) * avg_bytes + residual * full_bytes) / (tokens * full_bytes)


def last_page_waste(tokens: int, page: int) -> int:
    return (-tokens) % page


def window_ledger_bytes(window: int, head_dim: int, bits: int, group: int = 32, param_bytes: int = 4) -> int:
    """Bytes of one window of one KV head in the quantized tier: K and V codes,
    K parameters per channel per (up to group-token) chunk, V parameters per
    token per channel group."""
    codes = 2 * window * head_dim * bits // 8
    k_params = head_dim * math.ceil(window / group) * param_bytes
    v_params = window * (head_dim // group) * param_bytes
    return codes + k_params + v_params
