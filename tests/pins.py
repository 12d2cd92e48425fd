"""Independent second implementations used to pin the CPU oracle.

None of this calls the oracle: each function reaches the same result by a
different route (bit-field formulas instead of tables, threshold counting
instead of nearest search, torch's own float8 conversions, a dense
all-experts evaluation instead of routed pairs), so a slip in either side
shows up as a disagreement.
"""
from __future__ import annotations

import numpy as np
import torch


# ---------------------------------------------------------------- decode --

def e2m1_value_bitfield(code: int) -> float:
    """E2M1 from its fields: sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e8m0_values_torch() -> np.ndarray:
    """All 256 E8M0 bytes decoded by torch's float8_e8m0fnu."""
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu)
    return b.double().numpy()


def e4m3_values_torch() -> np.ndarray:
    """All 256 E4M3 codes decoded by torch's float8_e4m3fn."""
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return b.double().numpy()


def dequant_mxfp4_np(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[rows, K/2] + [rows, K/32] -> float64 [rows, K] via bit fields."""
    lut = np.array([e2m1_value_bitfield(c) for c in range(16)])
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return lut[codes] * np.repeat(sc, 32, axis=1)


# -------------------------------------------------------------- quantise --

# E2M1 tie points between neighbouring magnitudes 0,.5,1,1.5,2,3,4,6; at
# threshold i an exact tie goes up when the upper code i+1 is even.
_E2M1_THRESH = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_round_np(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, np.float64)
    a = np.abs(q)
    idx = np.zeros(q.shape, np.int64)
    for i, t in enumerate(_E2M1_THRESH):
        up_on_tie = (i + 1) % 2 == 0
        idx += (a > t) | ((a == t) & up_on_tie)
    return (idx | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def scale_exp_np(amax: np.ndarray, emax: int) -> np.ndarray:
    """floor(log2(amax)) - emax from numpy's frexp, clamped to [-127, 127]."""
    _, ex = np.frexp(amax)
    se = ex.astype(np.int64) - 1 - emax
    se = np.where(amax == 0, -127, se)
    return np.clip(se, -127, 127)


def quant_mxfp4_np(w: np.ndarray):
    w = np.asarray(w, np.float32).astype(np.float64)
    rows, K = w.shape
    blocks = w.reshape(rows, K // 32, 32)
    se = scale_exp_np(np.abs(blocks).max(axis=2), 2)
    q = blocks / np.ldexp(1.0, se)[..., None]
    codes = e2m1_round_np(q).reshape(rows, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (se + 127).astype(np.uint8)


def _f64_to_f32_round_to_odd(q: np.ndarray) -> np.ndarray:
    """float64 -> float32 rounding to odd: truncate, then set the last bit if
    anything was dropped.  A later nearest-even rounding to a format with far
    fewer bits then gives the same result as rounding the float64 directly
    (torch converts float64 to float8 through float32, which would otherwise
    round twice)."""
    f = q.astype(np.float32)
    inexact = f.astype(np.float64) != q
    over = inexact & (np.abs(f.astype(np.float64)) > np.abs(q))
    f = np.where(over, np.nextafter(f, np.float32(0)), f)
    bits = f.view(np.uint32) | np.where(inexact, np.uint32(1), np.uint32(0))
    return bits.astype(np.uint32).view(np.float32)


def e4m3_round_torch(q: np.ndarray) -> np.ndarray:
    """Nearest-even E4M3 code via torch, after the saturating clamp to 448."""
    q = np.clip(np.asarray(q, np.float64), -448.0, 448.0)
    t = torch.from_numpy(_f64_to_f32_round_to_odd(q)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quant_mxfp8_np(v: np.ndarray):
    v = np.asarray(v, np.float64)
    rows, K = v.shape
    blocks = v.reshape(rows, K // 32, 32)
    se = scale_exp_np(np.abs(blocks).max(axis=2), 8)
    q = blocks / np.ldexp(1.0, se)[..., None]
    return e4m3_round_torch(q).reshape(rows, K), (se + 127).astype(np.uint8)


def dequant_mxfp8_np(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = e4m3_values_torch()[codes]
    return vals * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def mxfp8_round_trip_np(v: np.ndarray) -> np.ndarray:
    c, s = quant_mxfp8_np(v)
    return dequant_mxfp8_np(c, s)


# ---------------------------------------------------------------- routing --

def route_bruteforce(logits: np.ndarray, k: int):
    """Python sort on (-logit, index); weights = softmax over all experts,
    restricted to the selected ones and renormalised."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        ids[t] = order
        z = np.asarray(row, np.float64)
        p = np.exp(z - z.max())
        p /= p.sum()
        sel = p[order]
        w[t] = sel / sel.sum()
    return ids, w


# ------------------------------------------------------------ dense FFN --

def dense_moe_np(x: np.ndarray, logits: np.ndarray, weights: dict, k: int,
                 act_mxfp8: bool = False) -> np.ndarray:
    """Evaluate EVERY expert on every token and mix with a dense [T, E] gate
    that is zero off the top-k (brute-force routing above)."""
    a = np.asarray(x, np.float64)
    if act_mxfp8:
        a = mxfp8_round_trip_np(a)
    T = a.shape[0]
    E = logits.shape[1]
    ids, w = route_bruteforce(logits, k)
    G = np.zeros((T, E))
    for t in range(T):
        G[t, ids[t]] = w[t]
    y = np.zeros((T, a.shape[1]))
    for e in range(E):
        Wg = dequant_mxfp4_np(weights["w_gate"][e], weights["w_gate_scale"][e])
        Wu = dequant_mxfp4_np(weights["w_up"][e], weights["w_up_scale"][e])
        Wd = dequant_mxfp4_np(weights["w_down"][e], weights["w_down_scale"][e])
        g = a @ Wg.T
        u = a @ Wu.T
        h = g * (1.0 / (1.0 + np.exp(-g))) * u
        if act_mxfp8:
            h = mxfp8_round_trip_np(h)
        y += G[:, e:e + 1] * (h @ Wd.T)
    return y
