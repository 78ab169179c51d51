"""Rotary position embedding around the quantized tier (oracle side).

QEvict notes, section 4.4 (Algorithm 1, the promotion step, and the paragraph
on promoted keys' positions): keys are quantized in the domain before the
rotary embedding, each window keeping its tokens' original absolute
positions; a window promoted back to full precision is dequantized and
rotated again at those positions.  The H2O page (section 3.3, positions) and
the KV-cache evolution page (section 10.3) add that a kept key must keep its
original position's rotation.

Readings (the pages fix neither the pairing nor the precision):

* The rotation pairs channel i with channel i + d/2 (the rotate-half form of
  Llama-family models): for a table row (c_i, s_i) of position p,
  r_i = x_i c_i - x_{i+d/2} s_i and r_{i+d/2} = x_{i+d/2} c_i + x_i s_i.
* The table (cos, sin per position and frequency, float32) is an input of the
  layer, as the model supplies it.
* A key stored in full precision is rotated once: float64 products and
  difference of its bfloat16 value and the float32 table, rounded to float32
  and then to bfloat16 (round to nearest even).  A promoted key is the same
  rotation of its float32 dequantized value.  The quantized tier is read as
  the rotation of the dequantized values, unrounded.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to_bf16


def rotate(x: np.ndarray, table: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotate rows x[..., t, d] at positions[t] with table [n_pos, d/2, 2]
    (cos, sin); float64 result (products exact, one rounding per output)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    tb = np.asarray(table, np.float32)[np.asarray(positions)].astype(np.float64)   # [t, h, 2]
    c, s = tb[..., 0], tb[..., 1]
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rotate_stored(x: np.ndarray, table: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """The full-precision copy of rotated keys: float32, then bfloat16."""
    return round_to_bf16(rotate(x, table, positions).astype(np.float32))
