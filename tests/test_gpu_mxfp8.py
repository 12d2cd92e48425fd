"""GPU parity of the MXFP8-activation path (the 8192-token chunk's mode).

The activation quantiser must match the oracle's MXFP8 quantiser bit for bit
(every rounding decision is taken on a bf16 value scaled by a power of two).
h is re-quantised on both sides from differently rounded values (float32
sums on the GPU, float64 in the oracle), so where the exact h sits within
float32 error of an E4M3 rounding boundary either code is correct; the
checks (tests/mx8_check.py) are that every h code and scale the GPU chose is
a correct rounding of an admissible value, and that the layer output equals
the oracle's down projection and combine of the GPU's own h within
max|y - y_ref| <= 2e-2 * RMS(y_ref).  The error against the oracle's own h is
printed beside it.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import mx8_check, pins, problems

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def test_quantize_act_mxfp8_bit_exact():
    moe = _moe()
    rng = np.random.default_rng(80)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2] *= 1e-30                                            # tiny blocks
    x[3] *= 1e30                                             # huge blocks
    x[4, ::32] = 448.0                                       # ties and saturation near the top
    x[4, 1::32] = 464.0
    x[5] = np.resize(np.array([0.0137, -0.0146, 1.0625, 3.3e-3, 5e-4, -7e-4], np.float32), 512)
    xb = synth.bf16_bits_from_f32(x)
    codes, scales = moe.quantize_act_mxfp8(_bf16(xb))
    torch.cuda.synchronize()
    c2, s2 = oracle.quant_mxfp8(synth.bf16_bits_to_f32(xb).astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), s2)
    assert np.array_equal(codes.cpu().numpy(), c2)


def _run(w, acts, dev, out_dtype, T=None):
    moe = _moe()
    T = w.T if T is None else T
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=T, act_mode=moe.ACT_MXFP8_E4M3,
                         out_dtype=out_dtype)
    P = T * w.k
    r = {"topk_ids": torch.empty(P, dtype=torch.int32, device="cuda"),
         "expert_offsets": torch.empty(w.E + 1, dtype=torch.int32, device="cuda"),
         "sorted_pairs": torch.empty(P, dtype=torch.int32, device="cuda")}
    y = layer(_bf16(acts["x_bf16"][:T]), torch.from_numpy(acts["logits"][:T]).cuda(), routing=r)
    codes, scales = layer.debug_hidden(T)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in r.items()}
    out["h_codes"], out["h_scales"] = codes.cpu().numpy(), scales.cpu().numpy()
    return y.float().cpu().numpy(), out


def _check(w, acts, wts, y, r, tokens, ref):
    """(error against the down + combine of the GPU's own h, error against
    the oracle, h elements within float32 error of a rounding boundary, h
    codes that differ from the exact h's), after checking every GPU h code."""
    ids, wt = oracle.route(acts["logits"][: len(r["topk_ids"]) // w.k], w.k)
    c, s = mx8_check.gpu_h_by_pair(r["h_codes"], r["h_scales"], r["sorted_pairs"], w.k, tokens)
    h, dh = mx8_check.exact_h(acts, wts, ids, tokens)
    amb, differ = mx8_check.check_h(h.reshape(-1, w.f), dh.reshape(-1, w.f), c.reshape(-1, w.f),
                                    s.reshape(-1, w.f // 32))
    hdec = pins.dequant_mxfp8_np(c.reshape(-1, w.f), s.reshape(-1, w.f // 32)).reshape(h.shape)
    y_own = mx8_check.down_combine(hdec, ids, wt, wts, tokens)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return (float(np.abs(y[tokens] - y_own).max()) / rms, float(np.abs(y[tokens] - ref).max()) / rms,
            amb, differ)


@pytest.mark.parametrize("T,E,k", [
    (40, 4, 2), (100, 2, 2), (13, 8, 3),
    (300, 2, 2),              # 300 pairs per expert: two full 128-pair chunks and a 44-pair tail
    (64, 1, 1),               # one expert, exactly half a chunk
])
def test_mxfp8_small_forward(T, E, k):
    """Eight seeds per shape; every one within the tolerance.  The error comes
    from single-step disagreements of h's E4M3 codes, whose rate is printed."""
    moe = _moe()
    own, strict, amb, differ = [], [], 0, 0
    for seed in range(8):
        w = synth.Workload("mx8", T, 256, 512, E, k, "mxfp8", "none", 90 + T + 1000 * seed)
        acts = synth.make_activations(w)
        wts = problems.pack_experts(w)
        dev = problems.to_device(wts)
        ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k, act_mode=oracle.ACT_MXFP8)
        y32, r = _run(w, acts, dev, moe.OUT_F32)
        ids, _ = oracle.route(acts["logits"], k)
        assert np.array_equal(r["topk_ids"], ids.reshape(-1))
        e_own, e_ref, a, dfr = _check(w, acts, wts, y32, r, np.arange(T), ref["y"])
        own.append(e_own)
        strict.append(e_ref)
        amb += a
        differ += dfr
    print(f"mxfp8 T={T} E={E} k={k}, 8 seeds: f32-out rel max err vs the GPU's own h: max {max(own):.3e}; "
          f"vs the oracle: max {max(strict):.3e}, mean {np.mean(strict):.3e}; h codes within float32 error of "
          f"a tie: {amb}, of which the GPU rounded the other way: {differ}")
    assert max(own) <= TOL, own


@pytest.mark.parametrize("d,f", [(8704, 512), (512, 8704), (256, 1024)])
def test_mxfp8_k_extents(d, f):
    moe = _moe()
    w = synth.Workload("mx8", 24, d, f, 4, 2, "mxfp8", "none", d + f)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k, act_mode=oracle.ACT_MXFP8)
    y32, r = _run(w, acts, problems.to_device(wts), moe.OUT_F32)
    e_own, e_ref, amb, differ = _check(w, acts, wts, y32, r, np.arange(w.T), ref["y"])
    print(f"mxfp8 d={d} f={f}: f32-out rel max err vs own h {e_own:.3e}, vs the oracle {e_ref:.3e} "
          f"({differ} of {amb} tie codes the other way)")
    assert e_own <= TOL


def test_chunk_8192_sampled_parity():
    moe = _moe()
    w = synth.workload("chunk_8192")
    acts, wts = problems.problem(w)
    dev = problems.to_device(wts)
    y16, r = _run(w, acts, dev, moe.OUT_BF16)
    ids, _ = oracle.route(acts["logits"], w.k)
    assert np.array_equal(r["topk_ids"], ids.reshape(-1))
    perm = oracle.permute(ids, w.E)
    assert np.array_equal(r["expert_offsets"], perm["offsets"])
    assert np.array_equal(r["sorted_pairs"], perm["sorted_pairs"])
    rng = np.random.default_rng(8)
    sample = np.sort(rng.choice(w.T, size=12, replace=False))
    ref = oracle.moe_forward(acts["x_bf16"][sample], acts["logits"][sample], wts, w.k,
                             act_mode=oracle.ACT_MXFP8, nthreads=problems.THREADS)["y"]
    e_own, e_ref, amb, differ = _check(w, acts, wts, y16, r, sample, ref)
    floor = problems.rel_max_err(torch.from_numpy(ref).bfloat16().double().numpy(), ref)
    print(f"chunk_8192: bf16-out rel max err over {len(sample)} tokens vs own h {e_own:.3e}, vs the oracle "
          f"{e_ref:.3e} (bf16 rounding of the reference alone: {floor:.3e}; {differ} of {amb} tie codes "
          f"the other way)")
    assert e_own <= TOL


@pytest.mark.parametrize("shifts", [(40, 40, 40, 40), (-60, -60, -60, -60), (40, -40, 0, 0)])
def test_mxfp8_outputs_outside_the_fp16_range(shifts):
    # the dense path stores each pair's outputs as fp16 codes with a
    # power-of-two scale per 128 columns: outputs near 1e10 (past fp16's
    # largest value), near 1e-20 (below its smallest), and experts of both
    # kinds inside one token must come back within the tolerance
    moe = _moe()
    w = synth.Workload("mx8", 24, 256, 512, 4, 2, "mxfp8", "none", 95)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    s = wts["w_down_scale"].astype(np.int32) + np.array(shifts, np.int32)[:, None, None]
    assert s.min() >= 0 and s.max() <= 254                   # stays a finite E8M0 byte
    wts["w_down_scale"] = s.astype(np.uint8)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k, act_mode=oracle.ACT_MXFP8)["y"]
    assert np.isfinite(ref).all()
    amax = np.abs(ref).max()
    assert amax > 1e6 or amax < 1e-8 or shifts[0] != shifts[1]
    y32, _ = _run(w, acts, problems.to_device(wts), moe.OUT_F32)
    err = problems.rel_max_err(y32, ref)
    print(f"mxfp8 down-scale shifts {shifts}: max |y| {amax:.3e}, f32-out rel max err {err:.3e}")
    assert err <= TOL
