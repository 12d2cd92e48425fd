"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks one oracle function against a closed form, a library
routine (torch's float8 codecs), brute force, or an independent second
implementation (tests/pins.py), chosen so that a dropped term, a wrong sign,
index or nibble order, or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs

def test_e2m1_decode_matches_bitfield_closed_form():
    for c in range(16):
        got = oracle.e2m1_value(c)
        want = pins.e2m1_value_bitfield(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_e8m0_decode_matches_torch_all_bytes():
    ref = pins.e8m0_values_torch()
    for b in range(255):
        assert oracle.e8m0_value(b) == ref[b], b
    assert math.isnan(oracle.e8m0_value(255)) and math.isnan(ref[255])


def test_e4m3_decode_matches_torch_all_codes():
    ref = pins.e4m3_values_torch()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c


def _e2m1_probe_values():
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 6.5, 7.999, 8.0, 100.0]
    for t in ties:
        vals += [t, np.nextafter(t, 0.0), np.nextafter(t, 10.0)]
    rng = np.random.default_rng(5)
    vals += list(rng.uniform(0.0, 8.0, 4000))
    vals += list(np.float32(rng.uniform(0.0, 8.0, 4000)).astype(np.float64))
    v = np.array(vals, np.float64)
    return np.concatenate([v, -v])


def test_e2m1_round_matches_threshold_table():
    q = _e2m1_probe_values()
    want = pins.e2m1_round_np(q)
    got = np.array([oracle.e2m1_round(float(v)) for v in q], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(q[i], got[i], want[i]) for i in bad[:10]]


def test_e2m1_round_tie_table():
    # nearest-even: ties go to the code whose mantissa bit is 0
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for q, v in expect.items():
        assert oracle.e2m1_value(oracle.e2m1_round(q)) == v
        assert oracle.e2m1_value(oracle.e2m1_round(-q)) == -v
    assert oracle.e2m1_round(-0.1) == 8          # negative underflow keeps its sign
    assert oracle.e2m1_round(7.5) == 7           # saturates to 6


def test_e4m3_round_matches_torch():
    rng = np.random.default_rng(6)
    q = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-0.02, 0.02, 5000),                       # subnormal range
        np.float32(rng.standard_normal(5000) * 50).astype(np.float64),
        np.arange(-448, 449, 0.125),                           # many exact ties
    ])
    got = np.array([oracle.e4m3_round(float(v)) for v in q], np.uint8)
    want = pins.e4m3_round_torch(q)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(q[i], got[i], want[i]) for i in bad[:10]]
    # saturation, never the NaN code
    for v in (448.5, 463.9, 464.0, 500.0, 511.99):
        assert oracle.e4m3_round(v) == 0x7E and oracle.e4m3_round(-v) == 0xFE


def test_e4m3_round_all_bf16_inputs():
    b = np.arange(65536, dtype=np.uint32)
    v32 = (b << 16).astype(np.uint32).view(np.float32)
    v32 = v32[np.isfinite(v32)]
    vals = v32[np.abs(v32) <= 1024.0].astype(np.float64)
    got = np.array([oracle.e4m3_round(float(v)) for v in vals], np.uint8)
    want = pins.e4m3_round_torch(vals)
    assert np.array_equal(got, want)


# -------------------------------------------------------------- MX tensors

def test_mx_block_size_is_the_pages_32():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    blk = facts["mx_block_size"]
    w = np.full((1, 4 * blk), 0.01, np.float32)
    _, s0 = oracle.quant_mxfp4(w)
    w2 = w.copy()
    w2[0, blk - 1] = 1.0          # last element of block 0
    _, s1 = oracle.quant_mxfp4(w2)
    w3 = w.copy()
    w3[0, blk] = 1.0              # first element of block 1
    _, s2 = oracle.quant_mxfp4(w3)
    assert s0.shape == (1, 4)
    assert s1[0, 0] != s0[0, 0] and np.array_equal(s1[0, 1:], s0[0, 1:])
    assert s2[0, 1] != s0[0, 1] and s2[0, 0] == s0[0, 0]


@pytest.mark.parametrize("e", [-127, -100, -20, -7, -1, 0, 1, 9, 60, 125])
def test_mxfp4_codebook_times_pow2_round_trips_exactly(e):
    rng = np.random.default_rng(1000 + e)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rows = []
    for top in (4.0, 6.0):
        for _ in range(8):
            v = rng.choice(mags, 32) * rng.choice([-1.0, 1.0], 32)
            v[rng.integers(32)] = top * rng.choice([-1.0, 1.0])
            rows.append(v)
    blk = np.ldexp(np.array(rows), e).astype(np.float32)
    assert np.array_equal(blk.astype(np.float64), np.ldexp(np.array(rows), e))
    packed, scales = oracle.quant_mxfp4(blk)
    assert np.all(scales == e + 127)
    back = oracle.dequant_mxfp4(packed, scales)
    assert np.array_equal(back, blk.astype(np.float64))


def test_mxfp4_nibble_order_low_nibble_is_even_element():
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 4.0          # amax 4 -> scale 2^0, code 6 (value 4)
    w[0, 1] = -1.0         # code 0b1010
    packed, scales = oracle.quant_mxfp4(w)
    assert scales[0, 0] == 127
    assert packed[0, 0] == (6 | (10 << 4))


def test_mxfp4_quantizer_matches_second_quantizer():
    rng = np.random.default_rng(7)
    mats = [rng.standard_normal((64, 256)).astype(np.float32) * 0.02,
            rng.standard_normal((16, 512)).astype(np.float32) * 3e4,
            (rng.standard_normal((8, 128)) * 1e-30).astype(np.float32),
            np.zeros((2, 64), np.float32)]
    t = np.array(_e2m1_probe_values()[:4096], np.float32).reshape(32, 128)
    mats.append(t)
    for m in mats:
        p1, s1 = oracle.quant_mxfp4(m)
        p2, s2 = pins.quant_mxfp4_np(m)
        assert np.array_equal(s1, s2)
        assert np.array_equal(p1, p2)


@pytest.mark.parametrize("name", ["tiny", "verify_1seq", "verify_32seq"])
def test_quantizers_agree_on_every_weight_of_the_workload(name):
    """The oracle's quantiser and the independent NumPy one give the same
    bytes on every expert matrix of the workload (all 3 x E matrices)."""
    from concurrent.futures import ThreadPoolExecutor
    w = synth.workload(name)

    def one(e):
        for m in synth.expert_weights_f32(w, e):
            p1, s1 = oracle.quant_mxfp4(m)
            p2, s2 = pins.quant_mxfp4_np(m)
            if not (np.array_equal(p1, p2) and np.array_equal(s1, s2)):
                return e
        return None

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        bad = [e for e in ex.map(one, range(w.E)) if e is not None]
    assert bad == []


def test_mxfp4_dequant_matches_bitfield_decoder():
    rng = np.random.default_rng(8)
    packed = rng.integers(0, 256, (16, 64), dtype=np.uint8)
    scales = rng.integers(0, 255, (16, 4), dtype=np.uint8)
    assert np.array_equal(oracle.dequant_mxfp4(packed, scales),
                          pins.dequant_mxfp4_np(packed, scales))


def test_mxfp8_quantizer_matches_torch_based_quantizer():
    rng = np.random.default_rng(9)
    for v in (rng.standard_normal((32, 256)),
              np.float32(rng.standard_normal((8, 512)) * 1e-3).astype(np.float64),
              rng.standard_normal((4, 64)) * 1e6):
        c1, s1 = oracle.quant_mxfp8(v)
        c2, s2 = pins.quant_mxfp8_np(v)
        assert np.array_equal(s1, s2)
        assert np.array_equal(c1, c2)
        assert np.array_equal(oracle.dequant_mxfp8(c1, s1), pins.dequant_mxfp8_np(c2, s2))


def test_mxfp8_e4m3_grid_times_pow2_round_trips():
    grid = pins.e4m3_values_torch()[:127]
    rng = np.random.default_rng(10)
    for e in (-120, -3, 0, 5, 100):
        v = rng.choice(grid, (4, 64)) * rng.choice([-1.0, 1.0], (4, 64))
        v[:, 0] = 448.0
        v[:, 32] = -256.0
        v = np.ldexp(v, e)
        c, s = oracle.quant_mxfp8(v)
        assert np.all(s == e + 127)
        assert np.array_equal(oracle.dequant_mxfp8(c, s), v)


# ----------------------------------------------------------------- routing

def _route_cases():
    rng = np.random.default_rng(11)
    yield rng.standard_normal((64, 16)).astype(np.float32), 4
    yield rng.integers(-2, 3, (64, 16)).astype(np.float32), 5          # many exact ties
    yield np.zeros((4, 8), np.float32), 8                                # all equal, k = E
    base = rng.standard_normal((32, 12)).astype(np.float32)
    # k-th and (k+1)-th logits one ulp apart
    srt = np.sort(base, axis=1)[:, ::-1]
    for t in range(32):
        j = int(np.argwhere(base[t] == srt[t, 3])[0, 0])
        i = int(np.argwhere(base[t] == srt[t, 2])[0, 0])
        base[t, j] = np.nextafter(base[t, i], np.float32(-np.inf))
    yield base, 3
    yield rng.standard_normal((16, 128)).astype(np.float32), 8


# ---------------------------------------------------------- router logits

def _bf16(a):
    return synth.bf16_bits_from_f32(np.asarray(a, np.float32))


def test_router_logits_match_pure_python_bruteforce():
    rng = np.random.default_rng(41)
    for T, d, E in ((3, 64, 5), (1, 32, 1), (4, 96, 3)):
        x = _bf16(rng.standard_normal((T, d)))
        w = _bf16(rng.standard_normal((E, d)) * 0.02)
        got, absdot = oracle.router_logits(x, w)
        xv = synth.bf16_bits_to_f32(x).astype(np.float64).tolist()
        wv = synth.bf16_bits_to_f32(w).astype(np.float64).tolist()
        for t in range(T):
            for e in range(E):
                s = a = 0.0
                for i in range(d):
                    s += xv[t][i] * wv[e][i]
                    a += abs(xv[t][i] * wv[e][i])
                assert got[t, e] == s and absdot[t, e] == a, (t, e)


def test_router_one_hot_rows_pick_weight_entries():
    rng = np.random.default_rng(42)
    d, E = 256, 7
    w = _bf16(rng.standard_normal((E, d)))
    picks = [0, 1, 31, 32, 200, 255]
    x = np.zeros((len(picks), d), np.float32)
    for t, i in enumerate(picks):
        x[t, i] = 1.0 if t % 2 == 0 else -2.0
    logits, _ = oracle.router_logits(_bf16(x), w)
    wv = synth.bf16_bits_to_f32(w).astype(np.float64)
    for t, i in enumerate(picks):
        assert np.array_equal(logits[t], (1.0 if t % 2 == 0 else -2.0) * wv[:, i])


def test_router_sign_flip_and_split_support_additivity():
    rng = np.random.default_rng(43)
    T, d, E = 5, 512, 9
    x = _bf16(rng.standard_normal((T, d)))
    w = rng.standard_normal((E, d)).astype(np.float32)
    w_lo, w_hi = w.copy(), w.copy()
    w_lo[:, d // 2:] = 0.0                            # disjoint supports: w = w_lo + w_hi exactly
    w_hi[:, :d // 2] = 0.0
    full, absdot = oracle.router_logits(x, _bf16(w))
    lo, a_lo = oracle.router_logits(x, _bf16(w_lo))
    hi, a_hi = oracle.router_logits(x, _bf16(w_hi))
    np.testing.assert_allclose(full, lo + hi, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(absdot, a_lo + a_hi, rtol=1e-12)
    neg, _ = oracle.router_logits(x ^ np.uint16(0x8000), _bf16(w))
    assert np.array_equal(neg, -full)
    assert np.all(absdot >= np.abs(full))


# ------------------------------------------------------- dflash acceptance

def _dirichlet(rng, shape, V, alpha=0.5):
    p = rng.gamma(alpha, size=shape + (V,))
    return (p / p.sum(axis=-1, keepdims=True)).astype(np.float32)


def _draw_searchsorted(w, r):
    """Independent integer inverse CDF: numpy cumulative sum and searchsorted."""
    q = np.rint(np.asarray(w, np.float64) * 2.0 ** 32).astype(np.uint64)
    cum = np.cumsum(q, dtype=np.uint64)
    S = int(cum[-1])
    thr = (S * int(np.floor(np.float64(r) * 2.0 ** 24))) >> 24
    return int(np.searchsorted(cum, np.uint64(thr), side="right"))


def test_dflash_first_token_is_distributed_as_the_target():
    # losslessness: whatever the drafter proposes, the first emitted token
    # (the accepted draft, or the draw after a rejection) follows p_target
    rng = np.random.default_rng(51)
    V, G, N = 6, 3, 200000
    pt1 = _dirichlet(rng, (G + 1,), V)
    pd1 = _dirichlet(rng, (G,), V)
    p64 = pd1.astype(np.float64)
    p64 /= p64.sum(axis=1, keepdims=True)
    draft = np.stack([rng.choice(V, size=N, p=p64[j]) for j in range(G)], 1)
    u = rng.random((N, G), dtype=np.float32)
    r = rng.random(N, dtype=np.float32)
    n_acc, tok = oracle.dflash_accept(draft, np.broadcast_to(pd1, (N, G, V)), np.broadcast_to(pt1, (N, G + 1, V)), u, r)
    first = np.where(n_acc >= 1, draft[:, 0], tok)
    counts = np.bincount(first, minlength=V)
    expect = pt1[0].astype(np.float64) / pt1[0].sum() * N
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 35.0, chi2                        # 5 degrees of freedom: p < 2e-6 to fail
    # acceptance rate of position 0: sum_x min(p_draft(x), p_target(x))
    acc = float(np.minimum(pd1[0], pt1[0]).sum())
    sd = math.sqrt(acc * (1 - acc) / N)
    assert abs((n_acc >= 1).mean() - acc) < 6 * sd


def test_dflash_identical_distributions_accept_the_whole_block():
    rng = np.random.default_rng(52)
    B, G, V = 20, 8, 50
    pt = _dirichlet(rng, (B, G + 1), V)
    draft = rng.integers(0, V, size=(B, G)).astype(np.int32)
    pt[np.arange(B)[:, None], np.arange(G)[None, :], draft] += 0.01   # every draft token has p > 0
    u = rng.random((B, G), dtype=np.float32)
    r = rng.random(B, dtype=np.float32)
    n_acc, tok = oracle.dflash_accept(draft, pt[:, :G], pt, u, r)
    assert np.all(n_acc == G)
    for b in range(B):
        assert tok[b] == _draw_searchsorted(pt[b, G], r[b]), b


def test_dflash_one_hot_target_rejects_and_draws_its_token():
    rng = np.random.default_rng(53)
    B, G, V = 16, 4, 32
    pd = _dirichlet(rng, (B, G), V)
    pt = np.zeros((B, G + 1, V), np.float32)
    want = rng.integers(0, V, size=B)
    draft = (want[:, None] + 1 + rng.integers(0, V - 1, size=(B, G))) % V   # never the target's token
    pt[np.arange(B), 0, want] = 1.0
    u = rng.random((B, G), dtype=np.float32)
    r = rng.random(B, dtype=np.float32)
    n_acc, tok = oracle.dflash_accept(draft.astype(np.int32), pd, pt, u, r)
    assert np.all(n_acc == 0)
    assert np.array_equal(tok, want)


def test_dflash_draw_skips_zero_weights():
    # a draw never lands on a zero-weight token, at either end of r's range
    G, V = 2, 8
    pt = np.zeros((4, G + 1, V), np.float32)
    pt[:, :G, 1] = 1.0                               # the drafts (token 1) are accepted
    pt[:, G, 2:4] = 0.5                              # the bonus draw: tokens 2 and 3 only
    draft = np.ones((4, G), np.int32)
    u = np.zeros((4, G), np.float32)
    r = np.array([0.0, 0.4999, 0.5, np.float32(1.0) - np.float32(2.0 ** -24)], np.float32)
    n_acc, tok = oracle.dflash_accept(draft, pt[:, :G], pt, u, r)
    assert np.all(n_acc == G)
    assert tok.tolist() == [2, 2, 3, 3]


def test_dflash_draws_match_independent_searchsorted():
    rng = np.random.default_rng(54)
    B, G, V = 64, 2, 1000
    pt = _dirichlet(rng, (B, G + 1), V, alpha=0.2)
    pd = _dirichlet(rng, (B, G), V, alpha=0.2)
    draft = rng.integers(0, V, size=(B, G)).astype(np.int32)
    u = rng.random((B, G), dtype=np.float32)
    r = rng.random(B, dtype=np.float32)
    r[:4] = [0.0, np.float32(1.0) - np.float32(2.0 ** -24), 0.5, 2.0 ** -20]
    n_acc, tok = oracle.dflash_accept(draft, pd, pt, u, r)
    for b in range(B):
        j = n_acc[b]
        if j < G:
            w = np.maximum(pt[b, j] - pd[b, j], np.float32(0.0))
            assert not (u[b, j] * pd[b, j, draft[b, j]] < pt[b, j, draft[b, j]]), b
        else:
            w = pt[b, G]
        assert tok[b] == _draw_searchsorted(w, r[b]), b
        assert all(u[b, i] * pd[b, i, draft[b, i]] < pt[b, i, draft[b, i]] for i in range(j)), b


def test_dflash_zero_residual_falls_back_to_the_target_row():
    # p_target = p_draft / 2 (not normalised): max(0, p_target - p_draft) is
    # zero everywhere, so a rejection draws from p_target itself
    rng = np.random.default_rng(55)
    B, G, V = 24, 3, 40
    pd = _dirichlet(rng, (B, G), V)
    pt = np.concatenate([pd * np.float32(0.5), _dirichlet(rng, (B, 1), V)], axis=1)
    draft = rng.integers(0, V, size=(B, G)).astype(np.int32)
    u = np.full((B, G), 0.75, np.float32)           # 0.75 p_draft >= p_draft / 2: rejected at once
    r = rng.random(B, dtype=np.float32)
    n_acc, tok = oracle.dflash_accept(draft, pd, pt, u, r)
    assert np.all(n_acc == 0)
    for b in range(B):
        assert tok[b] == _draw_searchsorted(pt[b, 0], r[b]), b


def test_dflash_out_of_range_draft_is_rejected():
    # a token outside [0, V) ends the block like one the target gives no mass
    rng = np.random.default_rng(56)
    B, G, V = 12, 4, 30
    pd = _dirichlet(rng, (B, G), V)
    pt = _dirichlet(rng, (B, G + 1), V)
    draft = rng.integers(1, V, size=(B, G)).astype(np.int32)
    pt[np.arange(B)[:, None], np.arange(G)[None, :], draft] += 0.05   # the in-range drafts are likely kept
    u = np.zeros((B, G), np.float32)                # u = 0: every token with p_target > 0 is accepted
    r = rng.random(B, dtype=np.float32)
    jbad = np.arange(B) % G
    bad = draft.copy()
    bad[np.arange(B), jbad] = np.where(np.arange(B) % 2 == 0, -1, V)
    zero = draft.copy()
    zero[np.arange(B), jbad] = 0
    pt0 = pt.copy()
    pt0[np.arange(B), jbad, 0] = 0.0                 # token 0 has no target mass at the bad position
    n_bad, tok_bad = oracle.dflash_accept(bad, pd, pt0, u, r)
    n_zero, tok_zero = oracle.dflash_accept(zero, pd, pt0, u, r)
    assert np.array_equal(n_bad, jbad)
    assert np.array_equal(n_bad, n_zero) and np.array_equal(tok_bad, tok_zero)


def test_dflash_non_positive_weights_count_as_zero():
    # negative and NaN entries of the row drawn from carry no mass
    rng = np.random.default_rng(57)
    B, V = 16, 64
    pt = _dirichlet(rng, (B, 1), V)
    junk = pt.copy()
    mask = rng.random((B, 1, V)) < 0.3
    vals = np.where(rng.random((B, 1, V)) < 0.5, np.float32(-0.25), np.float32(np.nan))
    junk[mask] = vals[mask]
    clean = np.where(mask, np.float32(0.0), pt)
    draft = np.zeros((B, 0), np.int32)
    pd = np.zeros((B, 0, V), np.float32)
    r = rng.random(B, dtype=np.float32)
    _, tok_junk = oracle.dflash_accept(draft, pd, junk, np.zeros((B, 0), np.float32), r)
    _, tok_clean = oracle.dflash_accept(draft, pd, clean, np.zeros((B, 0), np.float32), r)
    assert np.array_equal(tok_junk, tok_clean)
    assert not np.any(mask[np.arange(B), 0, tok_junk])


def test_dflash_r_outside_the_unit_interval_is_clamped():
    rng = np.random.default_rng(58)
    V = 20
    pt = _dirichlet(rng, (1, 1), V)
    pt[0, 0, [0, 1, V - 1]] = 0.0                    # first and last positive weights at 2 and V - 2
    one_minus = np.float32(1.0) - np.float32(2.0 ** -24)
    rs = np.array([-0.5, np.nan, 0.0, 1.0, 2.0, np.inf, one_minus], np.float32)
    n = rs.size
    _, tok = oracle.dflash_accept(np.zeros((n, 0), np.int32), np.zeros((n, 0, V), np.float32),
                                  np.broadcast_to(pt, (n, 1, V)), np.zeros((n, 0), np.float32), rs)
    assert tok[:3].tolist() == [2, 2, 2]            # at or below 0: the first positive weight
    assert tok[3:].tolist() == [V - 2] * 4           # at or above 1: as the largest float below 1


def test_route_matches_bruteforce():
    for logits, k in _route_cases():
        ids, w = oracle.route(logits, k)
        ids2, w2 = pins.route_bruteforce(logits, k)
        assert np.array_equal(ids, ids2)
        np.testing.assert_allclose(w, w2, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_route_equal_logits_give_uniform_weights():
    for k in (1, 2, 3, 8):
        ids, w = oracle.route(np.full((3, 9), 0.7, np.float32), k)
        assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))
        np.testing.assert_allclose(w, 1.0 / k, rtol=1e-15)


def test_permute_is_stable_sort_by_expert():
    rng = np.random.default_rng(12)
    for T, k, E in ((8, 2, 4), (256, 8, 64), (100, 3, 7), (1, 1, 1), (0, 4, 8)):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = oracle.route(logits, k) if T else (np.zeros((0, k), np.int32), None)
        r = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(r["counts"], np.bincount(flat, minlength=E))
        assert r["offsets"][0] == 0 and r["offsets"][-1] == T * k
        assert np.all(np.diff(r["offsets"]) >= 0)
        assert np.array_equal(r["sorted_pairs"], np.argsort(flat, kind="stable"))
        assert np.array_equal(r["sorted_pairs"][r["inverse"]], np.arange(T * k))


# --------------------------------------------------------------- forward

def _problem(T, d, f, E, k, seed, act="bf16", bias="none"):
    w = synth.Workload("t", T, d, f, E, k, act, bias, seed)
    acts = synth.make_activations(w)
    g, u, dn = zip(*[synth.expert_weights_f32(w, e) for e in range(E)])
    return w, acts, oracle.quantize_experts(g, u, dn)


@pytest.mark.parametrize("shape", [(8, 256, 512, 4, 2), (8, 128, 64, 8, 2), (5, 64, 96, 3, 3)])
def test_forward_equals_dense_evaluation(shape):
    T, d, f, E, k = shape
    w, acts, wts = _problem(T, d, f, E, k, seed=21)
    r = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)
    ref = pins.dense_moe_np(acts["x"], acts["logits"], wts, k)
    np.testing.assert_allclose(r["y"], ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_forward_mxfp8_equals_dense_evaluation():
    T, d, f, E, k = 8, 128, 96, 4, 2
    w, acts, wts = _problem(T, d, f, E, k, seed=22, act="mxfp8")
    r = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k, act_mode=oracle.ACT_MXFP8)
    ref = pins.dense_moe_np(acts["x"], acts["logits"], wts, k, act_mxfp8=True)
    # h is re-quantised on both sides; the dense path's different summation
    # order can flip an E4M3 rounding only on an exact-tie knife edge
    np.testing.assert_allclose(r["y"], ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())


def test_forward_single_expert_reduces_to_matmuls():
    w, acts, wts = _problem(6, 64, 64, 1, 1, seed=23)
    r = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, 1)
    Wg = pins.dequant_mxfp4_np(wts["w_gate"][0], wts["w_gate_scale"][0])
    Wu = pins.dequant_mxfp4_np(wts["w_up"][0], wts["w_up_scale"][0])
    Wd = pins.dequant_mxfp4_np(wts["w_down"][0], wts["w_down_scale"][0])
    g = acts["x"].astype(np.float64) @ Wg.T
    u = acts["x"].astype(np.float64) @ Wu.T
    y = (g / (1 + np.exp(-g)) * u) @ Wd.T
    assert np.all(r["w"] == 1.0)
    np.testing.assert_allclose(r["y"], y, rtol=1e-12, atol=1e-14)


def test_forward_one_hot_activation_picks_weight_columns():
    T, d, f, E, k = 4, 64, 32, 2, 1
    w, acts, wts = _problem(T, d, f, E, k, seed=24)
    x = np.zeros((T, d), np.uint16)
    cols = [0, 31, 32, 63]
    for t, c in enumerate(cols):
        x[t, c] = 0x3F80                                  # bf16 1.0
    r = oracle.moe_forward(x, acts["logits"], wts, k, want_h=True)
    for t, c in enumerate(cols):
        e = r["ids"][t, 0]
        Wg = pins.dequant_mxfp4_np(wts["w_gate"][e], wts["w_gate_scale"][e])
        Wu = pins.dequant_mxfp4_np(wts["w_up"][e], wts["w_up_scale"][e])
        g, u = Wg[:, c], Wu[:, c]
        np.testing.assert_allclose(r["h"][t, 0], g / (1 + np.exp(-g)) * u, rtol=1e-15, atol=0)


def test_forward_zero_weights_give_exact_zero():
    T, d, f, E, k = 8, 64, 64, 4, 2
    w, acts, wts = _problem(T, d, f, E, k, seed=25)
    for n in ("w_gate", "w_up", "w_down"):
        wts[n][:] = 0
    r = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)
    assert np.all(r["y"] == 0.0)


def test_forward_dominant_logit_selects_one_expert():
    T, d, f, E, k = 4, 64, 64, 4, 2
    w, acts, wts = _problem(T, d, f, E, k, seed=26)
    logits = acts["logits"].copy()
    logits[:, 2] = 80.0
    r = oracle.moe_forward(acts["x_bf16"], logits, wts, k)
    r1 = oracle.moe_forward(acts["x_bf16"], np.zeros((T, 1), np.float32),
                            {n: v[2:3] for n, v in wts.items()}, 1)
    assert np.all(r["ids"][:, 0] == 2)
    np.testing.assert_allclose(r["y"], r1["y"], rtol=1e-25 + 1e-12, atol=1e-30)


def test_forward_token_subset_equals_rows_of_full_batch():
    T, d, f, E, k = 16, 128, 64, 8, 3
    w, acts, wts = _problem(T, d, f, E, k, seed=27, bias="normal")
    full = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)
    rows = [0, 5, 15]
    sub = oracle.moe_forward(acts["x_bf16"][rows], acts["logits"][rows], wts, k)
    assert np.array_equal(sub["y"], full["y"][rows])
    assert np.array_equal(sub["ids"], full["ids"][rows])


def test_forward_threads_do_not_change_result():
    T, d, f, E, k = 12, 64, 64, 4, 2
    w, acts, wts = _problem(T, d, f, E, k, seed=28)
    a = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k, nthreads=1)
    b = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k, nthreads=4)
    assert np.array_equal(a["y"], b["y"])


def test_forward_rejects_bad_shapes():
    w, acts, wts = _problem(2, 64, 64, 2, 1, seed=29)
    with pytest.raises(ValueError):
        oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, 3)      # k > E
