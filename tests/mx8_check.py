"""Parity of the MXFP8-activation mode where its integer decisions are taken
on floating-point values that the two sides round differently.

In that mode h = silu(W_gate a) * (W_up a) is re-quantised to E4M3 codes
with one E8M0 scale per 32 (both sides, the reading that mirrors the MX
format on the down projection's input).  The oracle computes h in float64;
the GPU accumulates g and u in float32 (any order) and evaluates silu in
float32, so its h differs from the exact one by up to the float32 error
bound below.  Where the exact h lies closer than that bound to a rounding
boundary of E4M3 (or its block's largest magnitude to a power of two, which
decides the scale), both codes are correct roundings of an admissible value,
and the two sides may legitimately disagree by one step -- enough, on a large
element, to move a token's output by a few percent of RMS.

So the check is: (1) every code and scale the GPU chose is a correct rounding
of some value within the error bound of the exact h (bit-exact wherever that
interval holds one code); (2) the layer output equals the oracle's down
projection and combine evaluated on the GPU's own h, within the tolerance.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from tests import pins

U32 = 2.0 ** -24            # float32 unit roundoff


def exact_h(acts, wts, ids, tokens):
    """float64 h (before its MXFP8 round trip) of every pair (t, j), t in
    `tokens`, and a bound of |h32 - h| for any float32 evaluation: the sums
    of d exact products g, u carry at most (d + 16) u |a|.|w| each (any
    summation order), propagated through h = silu(g) u, plus 16 ulps of h
    for silu's exp and reciprocal and the product."""
    k = ids.shape[1]
    x = synth.bf16_bits_to_f32(acts["x_bf16"][tokens]).astype(np.float64)
    codes, scales = oracle.quant_mxfp8(x)
    a = oracle.dequant_mxfp8(codes, scales)
    d = a.shape[1]
    f = wts["w_gate"].shape[1]
    h = np.zeros((len(tokens), k, f))
    dh = np.zeros_like(h)
    for e in np.unique(ids[tokens]):
        rows, slots = np.nonzero(ids[tokens] == e)
        Wg = oracle.dequant_mxfp4(wts["w_gate"][e], wts["w_gate_scale"][e])
        Wu = oracle.dequant_mxfp4(wts["w_up"][e], wts["w_up_scale"][e])
        ar = a[rows]
        g, u = ar @ Wg.T, ar @ Wu.T
        G, Ua = np.abs(ar) @ np.abs(Wg).T, np.abs(ar) @ np.abs(Wu).T
        sig = 1.0 / (1.0 + np.exp(-g))
        silu = g * sig
        hv = silu * u
        dg, du = (d + 16) * U32 * G, (d + 16) * U32 * Ua
        h[rows, slots] = hv
        dh[rows, slots] = (np.abs(u * sig * (1 + g * (1 - sig))) * dg + np.abs(silu) * du + 16 * U32 * np.abs(hv))
    return h, dh


def check_h(h, dh, codes, scales):
    """Every GPU scale and code is a correct MXFP8 rounding of some value
    within [h - dh, h + dh]; returns (elements whose interval straddles a
    rounding boundary, those where the GPU's code differs from the exact
    value's code)."""
    n, f = h.shape
    hb, db = h.reshape(n, f // 32, 32), dh.reshape(n, f // 32, 32)
    amax, damax = np.abs(hb).max(axis=2), db.max(axis=2)
    se_gpu = scales.astype(np.int64) - 127
    se_lo = pins.scale_exp_np(np.maximum(amax - damax, 0.0), 8)
    se_hi = pins.scale_exp_np(amax + damax, 8)
    assert np.all((se_gpu >= se_lo) & (se_gpu <= se_hi)), "a block scale no admissible value gives"
    step = np.ldexp(1.0, -se_gpu)[..., None]
    table = pins.e4m3_values_torch()
    v_lo = table[pins.e4m3_round_torch((hb - db) * step)]
    v_hi = table[pins.e4m3_round_torch((hb + db) * step)]
    v_gpu = table[codes.reshape(n, f // 32, 32)]
    assert np.all((v_gpu >= v_lo) & (v_gpu <= v_hi)), "an h code no admissible value rounds to"
    v_exact = table[pins.e4m3_round_torch(hb * np.ldexp(1.0, -pins.scale_exp_np(amax, 8))[..., None])]
    v_exact_scaled = v_exact * np.ldexp(1.0, pins.scale_exp_np(amax, 8))[..., None]
    differ = int((v_gpu / step != v_exact_scaled).sum())
    return int((v_lo != v_hi).sum()), differ


def down_combine(hdec, ids, w, wts, tokens):
    """y[t] = sum_j w[t][j] * W_down,e(t,j) h(t,j) in float64, for the given
    (decoded) h of the tokens' pairs."""
    k = ids.shape[1]
    d = wts["w_down"].shape[1]
    y = np.zeros((len(tokens), d))
    for e in np.unique(ids[tokens]):
        rows, slots = np.nonzero(ids[tokens] == e)
        Wd = oracle.dequant_mxfp4(wts["w_down"][e], wts["w_down_scale"][e])
        y[rows] += w[tokens][rows, slots][:, None] * (hdec[rows, slots] @ Wd.T)
    return y


def gpu_h_by_pair(codes_sorted, scales_sorted, sorted_pairs, k, tokens):
    """The GPU's h rows (expert-sorted) regrouped as [len(tokens), k, ...]."""
    row_of_pair = np.empty_like(sorted_pairs)
    row_of_pair[sorted_pairs] = np.arange(len(sorted_pairs))
    pairs = (np.asarray(tokens)[:, None] * k + np.arange(k)[None, :]).ravel()
    rows = row_of_pair[pairs]
    c = codes_sorted[rows].reshape(len(tokens), k, -1)
    s = scales_sorted[rows].reshape(len(tokens), k, -1)
    return c, s
