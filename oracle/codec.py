"""Quantizers of the KV tiers (oracle side).

Uniform quantizer -- HqeKV notes, section 2.3, Eq.(2): per group, the offset
is the group minimum and the step is (max - min) / (2^b - 1); a value maps to
round((x - z) / s) and back to q*s + z.  The KV-cache evolution page
(section 5, KIVI) fixes the group axes and the payload: keys are grouped per
channel along tokens, values per token along channels, groups of 32, a scale
and a zero per group (4 bytes), giving 0.375 B/element at 2 bits.

Precision (a reading; the pages do not fix it): min and max are exact; the
step is the float32 quotient of the float32 difference; scale and zero are
stored as float16 (round to nearest even) -- two float16 values are the 4-byte
parameter pair of the payload arithmetic; the code is round-half-even of the
float32 quotient (x - z16) / s16, clamped to [0, 2^b - 1], and 0 for a group
whose stored step is 0; dequantization is a single-rounding float32
multiply-add code*s16 + z16.

Normalized quantizer -- HqeKV notes, section 2.3, Eq.(3)-(4): standardize by
the vector's mean and standard deviation, put centres at standard-normal
quantiles, assign each value to the centre with the least probability mass
between them.  Reading of the garbled centre list and index range of Eq.(4):
centres c_j = Phi^-1((j + 1/2) / 2^b), j = 0 .. 2^b - 1, ties to the lower j.
At one bit this is a sign test about the mean, with centres -/+ Phi^-1(3/4).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.stats import norm

from .numerics import fma32

KAPPA1 = np.float32(norm.ppf(0.75))      # Phi^-1(3/4) = 0.6744897501960817


class ParamRangeError(OverflowError):
    """A scale or zero does not fit float16."""


# ---------------------------------------------------------------------------
# uniform (affine) quantizer, groups along the last axis
# ---------------------------------------------------------------------------

def uniform_quantize(x: np.ndarray, bits: int):
    """Quantize groups laid along the last axis of ``x`` (float32 values).

    Returns (codes uint8, scale float16, zero float16); scale/zero have the
    shape of ``x`` without its last axis."""
    x32 = np.asarray(x, dtype=np.float32)
    levels = np.float32(2 ** bits - 1)
    mn = x32.min(axis=-1)
    mx = x32.max(axis=-1)
    with np.errstate(over="ignore"):
        s32 = (mx - mn) / levels                      # float32 subtract, float32 divide
        s16 = s32.astype(np.float16)
        z16 = mn.astype(np.float16)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(z16))):
        raise ParamRangeError("quantization parameter exceeds float16 range")
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (x32 - z) / s                             # float32 subtract, float32 divide
    code = np.clip(np.rint(r), 0, levels)            # rint: round half to even
    code = np.where(s == 0, 0, code)
    return code.astype(np.uint8), s16, z16


def uniform_dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x_hat = float32 fma(code, s, z); scale/zero broadcast over the last axis."""
    return fma32(codes, np.asarray(s16)[..., None], np.asarray(z16)[..., None])


# ---------------------------------------------------------------------------
# normalized quantizer
# ---------------------------------------------------------------------------

def int1_normal_quantize(x: np.ndarray):
    """One-bit normalized quantizer over the last axis (a token's d channels).

    mean m = float32(exact sum / d) (sum in float64, exact for bfloat16 inputs
    of ordinary range), sigma = float32(sqrt(sum((x - m)^2) / d)) (population
    deviation), code = 1 iff x > m.  Returns (codes, m16, sigma16)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    d = x64.shape[-1]
    m32 = (x64.sum(axis=-1) / d).astype(np.float32)
    dev = x64 - m32.astype(np.float64)[..., None]
    sd32 = np.sqrt((dev * dev).sum(axis=-1) / d).astype(np.float32)
    with np.errstate(over="ignore"):
        m16 = m32.astype(np.float16)
        sd16 = sd32.astype(np.float16)
    if not (np.all(np.isfinite(m16)) and np.all(np.isfinite(sd16))):
        raise ParamRangeError("normalized-quantizer parameter exceeds float16 range")
    codes = (x64 > m32.astype(np.float64)[..., None]).astype(np.uint8)
    return codes, m16, sd16


def int1_normal_dequantize(codes: np.ndarray, m16: np.ndarray, sd16: np.ndarray) -> np.ndarray:
    """x_hat = float32(m + sigma * c_code), c = -/+ Phi^-1(3/4), one rounding."""
    c = np.where(np.asarray(codes) != 0, KAPPA1, -KAPPA1).astype(np.float32)
    return fma32(c, np.asarray(sd16)[..., None], np.asarray(m16)[..., None])


def normal_centres(bits: int) -> np.ndarray:
    j = np.arange(2 ** bits)
    return norm.ppf((j + 0.5) / 2 ** bits)


def normal_quantize(x: np.ndarray, bits: int):
    """General-b normalized quantizer (float64), Eq.(3)-(4) under the reading
    above.  Returns (codes, mean, std, x_hat)."""
    x64 = np.asarray(x, dtype=np.float64)
    m = x64.mean(axis=-1, keepdims=True)
    sd = x64.std(axis=-1, keepdims=True)
    xs = np.where(sd > 0, (x64 - m) / np.where(sd > 0, sd, 1.0), 0.0)
    c = normal_centres(bits)
    # probability mass between value and centre = |Phi(x') - Phi(c_j)|
    dist = np.abs(norm.cdf(xs)[..., None] - norm.cdf(c))
    codes = np.argmin(dist, axis=-1)                  # first minimum -> lower j on ties
    xhat = m + sd * c[codes]
    return codes.astype(np.uint8), m[..., 0], sd[..., 0], xhat


def uniform_roundtrip64(x: np.ndarray, bits: int) -> np.ndarray:
    """Uniform quantize/dequantize in float64 over the last axis (analysis use)."""
    x64 = np.asarray(x, dtype=np.float64)
    mn = x64.min(axis=-1, keepdims=True)
    mx = x64.max(axis=-1, keepdims=True)
    s = (mx - mn) / (2 ** bits - 1)
    q = np.where(s > 0, np.clip(np.rint((x64 - mn) / np.where(s > 0, s, 1.0)), 0, 2 ** bits - 1), 0)
    return q * s + mn


# ---------------------------------------------------------------------------
# KIVI grouping of one window block
# ---------------------------------------------------------------------------

def kivi_quantize_window(k: np.ndarray, v: np.ndarray, bits: int, group: int = 32):
    """Quantize one window of keys and values, K per channel, V per token.

    k, v: float32 [H, w, d].  Keys are grouped per channel along the window's
    tokens, in chunks of ``group`` tokens when the window is longer (groups
    never span windows, which are routed independently); values per token in
    groups of ``group`` consecutive channels.

    Returns a dict with codes indexed [H, w, d] and parameter arrays
    kscale/kzero [H, d, n_chunks], vscale/vzero [H, w, d // group]."""
    H, w, d = k.shape
    if d % group:
        raise ValueError("head_dim must be a multiple of the group")
    n_chunks = math.ceil(w / group)
    kcodes = np.zeros((H, w, d), np.uint8)
    ks = np.zeros((H, d, n_chunks), np.float16)
    kz = np.zeros((H, d, n_chunks), np.float16)
    kt = np.asarray(k, np.float32).transpose(0, 2, 1)          # [H, d, w]
    for ci in range(n_chunks):
        t0, t1 = ci * group, min(w, (ci + 1) * group)
        c, s, z = uniform_quantize(kt[:, :, t0:t1], bits)        # groups: [H, d] over tokens
        kcodes[:, t0:t1, :] = c.transpose(0, 2, 1)
        ks[:, :, ci], kz[:, :, ci] = s, z
    vg = np.asarray(v, np.float32).reshape(H, w, d // group, group)
    vc, vs, vz = uniform_quantize(vg, bits)
    return dict(kcodes=kcodes, kscale=ks, kzero=kz,
                vcodes=vc.reshape(H, w, d), vscale=vs, vzero=vz, bits=bits, group=group)


def kivi_dequantize_window(q: dict):
    """Inverse of :func:`kivi_quantize_window` -> (k_hat, v_hat) float32 [H, w, d]."""
    kc, vc = q["kcodes"], q["vcodes"]
    H, w, d = kc.shape
    g = q["group"]
    n_chunks = q["kscale"].shape[-1]
    khat = np.zeros((H, w, d), np.float32)
    for ci in range(n_chunks):
        t0, t1 = ci * g, min(w, (ci + 1) * g)
        khat[:, t0:t1, :] = uniform_dequantize(kc[:, t0:t1, :].transpose(0, 2, 1),
                                               q["kscale"][:, :, ci], q["kzero"][:, :, ci]).transpose(0, 2, 1)
    vhat = uniform_dequantize(vc.reshape(H, w, d // g, g), q["vscale"], q["vzero"]).reshape(H, w, d)
    return khat, vhat


def per_token_quantize(x: np.ndarray, bits: int, group: int = 32):
    """Per-token uniform quantization over ``group`` channels: x [..., d]."""
    d = x.shape[-1]
    c, s, z = uniform_quantize(np.asarray(x, np.float32).reshape(*x.shape[:-1], d // group, group), bits)
    return c.reshape(x.shape), s, z


def per_token_dequantize(codes, s16, z16, group: int = 32):
    d = codes.shape[-1]
    return uniform_dequantize(codes.reshape(*codes.shape[:-1], d // group, group), s16, z16).reshape(codes.shape)


# ---------------------------------------------------------------------------
# canonical packed layout (byte-level exchange format)
# ---------------------------------------------------------------------------

def pack_codes(flat: np.ndarray, bits: int) -> np.ndarray:
    """Pack a 1-D code stream: element e sits at bit bits*(e mod (8/bits)) of
    byte floor(e*bits/8) (2-bit: four per byte; 4-bit: low nibble first;
    1-bit: bit e mod 8)."""
    flat = np.asarray(flat, np.uint8).reshape(-1)
    per = 8 // bits
    if flat.size % per:
        flat = np.concatenate([flat, np.zeros(per - flat.size % per, np.uint8)])
    lanes = flat.reshape(-1, per).astype(np.uint16)
    shifts = (np.arange(per) * bits).astype(np.uint16)
    return (lanes << shifts).sum(axis=1).astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    per = 8 // bits
    p = np.asarray(packed, np.uint8).astype(np.uint16)
    shifts = (np.arange(per) * bits).astype(np.uint16)
    return ((p[:, None] >> shifts) & ((1 << bits) - 1)).reshape(-1)[:n].astype(np.uint8)


def canonical_k_codes(kcodes: np.ndarray, bits: int) -> np.ndarray:
    """Keys: per head, element (channel c, token t) has index e = c*w + t."""
    H, w, d = kcodes.shape
    return np.stack([pack_codes(kcodes[h].T.reshape(-1), bits) for h in range(H)])


def canonical_v_codes(vcodes: np.ndarray, bits: int) -> np.ndarray:
    """Values (and per-token keys): per head, e = t*d + c."""
    H = vcodes.shape[0]
    return np.stack([pack_codes(vcodes[h].reshape(-1), bits) for h in range(H)])


def canonical_params(scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """(scale, zero) float16 pairs in the parameter arrays' own index order
    ([head][channel][token-group] for keys, [head][token][channel-group] for
    values)."""
    return np.stack([scale, zero], axis=-1).astype(np.float16)
