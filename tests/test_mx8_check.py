"""The MXFP8-mode checker (tests/mx8_check.py) on the CPU: h evaluated in
float32 (numpy, another summation order than float64) must pass it, and
planted mistakes -- a code two steps off, a block scale one step off where no
admissible value gives it -- must fail it."""
import numpy as np
import pytest

import oracle
import synth
from tests import mx8_check, pins, problems


@pytest.fixture(scope="module")
def case():
    w = synth.Workload("mx8c", 48, 256, 512, 4, 2, "mxfp8", "none", 321)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    ids, wt = oracle.route(acts["logits"], w.k)
    tokens = np.arange(w.T)
    h, dh = mx8_check.exact_h(acts, wts, ids, tokens)
    # the same h evaluated in float32
    x = synth.bf16_bits_to_f32(acts["x_bf16"]).astype(np.float64)
    a = oracle.dequant_mxfp8(*oracle.quant_mxfp8(x)).astype(np.float32)
    h32 = np.zeros_like(h)
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        Wg = oracle.dequant_mxfp4(wts["w_gate"][e], wts["w_gate_scale"][e]).astype(np.float32)
        Wu = oracle.dequant_mxfp4(wts["w_up"][e], wts["w_up_scale"][e]).astype(np.float32)
        g, u = a[rows] @ Wg.T, a[rows] @ Wu.T
        h32[rows, slots] = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float64)
    return w, acts, wts, ids, wt, h, dh, h32


def test_float32_h_is_within_the_bound_and_passes(case):
    w, acts, wts, ids, wt, h, dh, h32 = case
    assert np.all(np.abs(h32 - h) <= dh)
    codes, scales = pins.quant_mxfp8_np(h32.reshape(-1, w.f))
    amb, differ = mx8_check.check_h(h.reshape(-1, w.f), dh.reshape(-1, w.f), codes, scales)
    assert differ <= amb
    # the output from the float32 codes, and from the exact ones (the oracle)
    hdec = pins.dequant_mxfp8_np(codes, scales).reshape(h.shape)
    y = mx8_check.down_combine(hdec, ids, wt, wts, np.arange(w.T))
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k, act_mode=oracle.ACT_MXFP8)["y"]
    exact_dec = pins.mxfp8_round_trip_np(h.reshape(-1, w.f)).reshape(h.shape)
    assert np.allclose(mx8_check.down_combine(exact_dec, ids, wt, wts, np.arange(w.T)), ref, rtol=0, atol=1e-12)
    if differ == 0:
        assert np.allclose(y, ref, rtol=0, atol=1e-12)


def test_planted_code_two_steps_off_fails(case):
    w, acts, wts, ids, wt, h, dh, h32 = case
    codes, scales = pins.quant_mxfp8_np(h32.reshape(-1, w.f))
    bad = codes.copy()
    i = np.argmax(np.abs(h32.reshape(-1, w.f)))          # a large element, far from saturation ties
    r, c = np.unravel_index(i, bad.shape)
    bad[r, c] = (bad[r, c] & 0x80) | max(0, (bad[r, c] & 0x7F) - 2)
    with pytest.raises(AssertionError):
        mx8_check.check_h(h.reshape(-1, w.f), dh.reshape(-1, w.f), bad, scales)


def test_planted_scale_off_fails(case):
    w, acts, wts, ids, wt, h, dh, h32 = case
    codes, scales = pins.quant_mxfp8_np(h32.reshape(-1, w.f))
    bad = scales.copy()
    bad[3, 5] += 1
    with pytest.raises(AssertionError):
        mx8_check.check_h(h.reshape(-1, w.f), dh.reshape(-1, w.f), codes, bad)


def test_gpu_rows_regroup_by_pair():
    # rows in expert-sorted order map back to (token, slot) through sorted_pairs
    k, T = 2, 5
    sorted_pairs = np.array([3, 0, 7, 1, 9, 2, 4, 5, 6, 8], np.int32)
    codes = np.arange(10)[:, None] * np.ones((1, 4), np.int64)
    scales = codes[:, :1]
    c, s = mx8_check.gpu_h_by_pair(codes, scales, sorted_pairs, k, [1, 4])
    # pair p = t*k + j sits at the row r with sorted_pairs[r] == p
    assert c[0, 0, 0] == 5 and c[0, 1, 0] == 0 and c[1, 0, 0] == 9 and c[1, 1, 0] == 4
