"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: routing ids, expert offsets, the permutation, the FP4 decode and the
weight quantiser are bit-exact; routing weights within 1e-6; the layer
output within max|y - y_ref| <= 2e-2 * RMS(y_ref) (y_ref in double).  Full
sizes run the GPU on the whole batch, in the launch configuration the
benchmark times, and check a sample of tokens against the oracle (tokens are
independent given their routing) plus the routing of every token.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import problems, tiling

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


def _run(w: synth.Workload, acts, wts_dev, out_dtype=None, T=None, routing=True):
    moe = _moe()
    T = w.T if T is None else T
    layer = moe.MoeMxfp4(wts_dev, w.E, w.d, w.f, w.k, max_tokens=max(T, 1),
                         out_dtype=moe.OUT_F32 if out_dtype is None else out_dtype)
    x = torch.from_numpy(acts["x_bf16"][:T].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"][:T]).cuda()
    r = None
    if routing:
        P = T * w.k
        r = {"topk_ids": torch.empty(P, dtype=torch.int32, device="cuda"),
             "topk_w": torch.empty(P, dtype=torch.float32, device="cuda"),
             "expert_offsets": torch.empty(w.E + 1, dtype=torch.int32, device="cuda"),
             "sorted_pairs": torch.empty(P, dtype=torch.int32, device="cuda")}
    y = layer(x, lg, routing=r)
    torch.cuda.synchronize()
    out = {"y": y.float().cpu().numpy()}
    if r:
        out.update({k: v.cpu().numpy() for k, v in r.items()})
    return out, layer


def _check_routing(w, acts, got, T=None):
    T = w.T if T is None else T
    ids, wts = oracle.route(acts["logits"][:T], w.k)
    perm = oracle.permute(ids, w.E)
    assert np.array_equal(got["topk_ids"], ids.reshape(-1))
    assert np.abs(got["topk_w"] - wts.reshape(-1)).max() <= 1e-6
    assert np.array_equal(got["expert_offsets"], perm["offsets"])
    assert np.array_equal(got["sorted_pairs"], perm["sorted_pairs"])


# ------------------------------------------------------------- decode ---

def test_debug_dequant_bit_exact_all_bytes_and_scales():
    moe = _moe()
    E, d, f = 1, 256, 256
    rng = np.random.default_rng(40)
    wts = {}
    for name, (rows, K) in (("w_gate", (f, d)), ("w_up", (f, d)), ("w_down", (d, f))):
        packed = ((np.arange(rows * K // 2) * 7 + rng.integers(0, 256)) % 256).astype(np.uint8)
        scales = (np.arange(rows * K // 32) % 255).astype(np.uint8)     # every finite byte
        wts[name] = packed.reshape(1, rows, K // 2)
        wts[name + "_scale"] = rng.permutation(scales).reshape(1, rows, K // 32)
    dev = problems.to_device(wts)
    layer = moe.MoeMxfp4(dev, E, d, f, 1, max_tokens=1)
    for m, name in enumerate(("w_gate", "w_up", "w_down")):
        rows = wts[name].shape[1]
        got = layer.debug_dequant(0, m, 0, rows).cpu().numpy()
        with np.errstate(over="ignore"):
            ref = oracle.dequant_mxfp4(wts[name][0], wts[name + "_scale"][0]).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
    # a row window
    got = layer.debug_dequant(0, 2, 100, 7).cpu().numpy()
    with np.errstate(over="ignore"):
        ref = oracle.dequant_mxfp4(wts["w_down"][0, 100:107], wts["w_down_scale"][0, 100:107])
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_quantize_weights_bit_exact():
    moe = _moe()
    rng = np.random.default_rng(41)
    rows = [rng.standard_normal((64, 512)) * 0.02,
            rng.standard_normal((8, 512)) * 3e4,
            rng.standard_normal((8, 512)) * 1e-39,                      # subnormal floats
            np.zeros((2, 512)), -np.zeros((2, 512))]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.9])
    base = np.concatenate([ties, -ties, np.nextafter(ties, 0), np.nextafter(ties, 9)])
    t = np.resize(base, 16 * 512).reshape(16, 512)
    t[:, ::32] = 4.0                                                   # pin each block's scale
    rows += [t, t * 2.0 ** -20]
    w = np.concatenate(rows).astype(np.float32)
    p, s = moe.quantize_weights(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    p2, s2 = oracle.quant_mxfp4(w)
    assert np.array_equal(s.cpu().numpy(), s2)
    assert np.array_equal(p.cpu().numpy(), p2)


# ------------------------------------------------------- small / full ---

def test_tiny_workload_full_parity():
    w = synth.workload("tiny")
    acts, wts = problems.problem(w)
    dev = problems.to_device(wts)
    got, _ = _run(w, acts, dev)
    _check_routing(w, acts, got)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    err = problems.rel_max_err(got["y"], ref)
    print(f"tiny f32-out rel max err {err:.3e}")
    assert err <= TOL
    got16, _ = _run(w, acts, dev, out_dtype=0, routing=False)
    err16 = problems.rel_max_err(got16["y"], ref)
    print(f"tiny bf16-out rel max err {err16:.3e}")
    assert err16 <= TOL
    # the bf16 output is the float32 result rounded once to nearest even
    assert np.array_equal(got16["y"].astype(np.float32),
                          torch.from_numpy(got["y"]).bfloat16().float().numpy())


@pytest.mark.parametrize("name,nsample", [("verify_1seq", 8), ("verify_32seq", 256),
                                          ("share_64seq", 64)])
def test_full_size_workload_parity(name, nsample):
    """The whole 8- and 256-token batches against the oracle; at 512 tokens a
    64-token sample that holds tokens of every 64-pair chunk of the most
    loaded expert (the multi-chunk path).  Routing of every token is exact."""
    w = synth.workload(name)
    acts, wts = problems.problem(w)
    dev = problems.to_device(wts)
    got, _ = _run(w, acts, dev, out_dtype=0)            # bf16 output, as benchmarked
    _check_routing(w, acts, got)
    if nsample >= w.T:
        sample = np.arange(w.T)
    else:
        # 4 tokens from each chunk of the hottest expert's pairs (in sorted
        # order), the rest drawn at random
        ids = got["topk_ids"].reshape(w.T, w.k)
        hot = int(np.bincount(ids.ravel(), minlength=w.E).argmax())
        lo, hi = got["expert_offsets"][hot], got["expert_offsets"][hot + 1]
        hot_pairs = got["sorted_pairs"][lo:hi]
        picks = [hot_pairs[c:c + 64][:: max(1, len(hot_pairs[c:c + 64]) // 4)][:4] // w.k
                 for c in range(0, len(hot_pairs), 64)]
        sample = np.unique(np.concatenate(picks))
        assert len(picks) >= 2                      # the hot expert has several chunks
        rng = np.random.default_rng(7)
        rest = rng.permutation(np.setdiff1d(np.arange(w.T), sample))
        sample = np.sort(np.concatenate([sample, rest[:nsample - len(sample)]]))
    ref = oracle.moe_forward(acts["x_bf16"][sample], acts["logits"][sample], wts, w.k,
                             nthreads=problems.THREADS)["y"]
    err = problems.rel_max_err(got["y"][sample], ref)
    # where the error comes from: the same call with float32 output, and the
    # bf16 rounding of the reference alone (the output format's floor)
    got32, _ = _run(w, acts, dev, routing=False)
    err32 = problems.rel_max_err(got32["y"][sample], ref)
    floor = problems.rel_max_err(torch.from_numpy(ref).bfloat16().double().numpy(), ref)
    print(f"{name}: rel max err over {len(sample)} tokens: bf16 out {err:.3e}, float32 out {err32:.3e}; "
          f"bf16 rounding of the reference alone {floor:.3e}")
    assert err <= TOL and err32 <= TOL


@pytest.mark.parametrize("name", ["tiny", "verify_1seq", "verify_32seq"])
def test_gpu_quantiser_on_every_weight_of_the_workload(name):
    """The library's weight quantiser gives the oracle's bytes on every
    expert matrix of the workload."""
    from concurrent.futures import ThreadPoolExecutor
    moe = _moe()
    w = synth.workload(name)

    def host(e):
        mats = synth.expert_weights_f32(w, e)
        return e, mats, [oracle.quant_mxfp4(m) for m in mats]

    with ThreadPoolExecutor(problems.THREADS) as ex:
        for e, mats, ref in ex.map(host, range(w.E)):
            for m, (p_ref, s_ref) in zip(mats, ref):
                p, sc = moe.quantize_weights(torch.from_numpy(m).cuda())
                assert np.array_equal(p.cpu().numpy(), p_ref), e
                assert np.array_equal(sc.cpu().numpy(), s_ref), e


# -------------------------------------------------------------- edges ---

def _custom(T, d, f, E, k, seed, logits=None, scale=None):
    w = synth.Workload("edge", T, d, f, E, k, "bf16", "none", seed)
    acts = synth.make_activations(w)
    if logits is not None:
        acts["logits"] = np.ascontiguousarray(logits, np.float32)
    wts = problems.pack_experts(w)
    return w, acts, wts


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (13, 8, 2), (37, 4, 4), (5, 1, 1), (64, 16, 3),
                                   (1100, 64, 8)])         # 8800 pairs: the tiled sort, last tile partial
def test_edge_shapes(T, E, k):
    w, acts, wts = _custom(T, 256, 256, E, k, seed=50 + T)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)["y"]
    assert problems.rel_max_err(got["y"], ref) <= TOL


@pytest.mark.parametrize("T,E,k", [(64, 64, 1), (8, 64, 8), (1, 1, 1), (21, 3, 3), (32, 64, 2), (17, 50, 3),
                                   (16, 2, 2), (9, 7, 7)])
def test_single_wave_permutation_shapes(T, E, k):
    # at most 64 pairs over at most 64 experts: routing, then the permutation
    # by one wavefront (64 pairs exactly, 64 experts, k = 1, more tokens than
    # routing waves, skewed and tie-heavy logits)
    rng = np.random.default_rng(70 + T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if T % 2:
        lg = np.round(lg * 2) / 2                      # many exact ties
    lg[:, E // 2] += 3.0                                # one hot expert
    w, acts, wts = _custom(T, 256, 256, E, k, seed=90 + T, logits=lg)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)["y"]
    assert problems.rel_max_err(got["y"], ref) <= TOL


@pytest.mark.parametrize("d,f", [(8704, 512), (512, 8704), (256, 1024)])
def test_k_extents(d, f):
    # 68 K steps on either projection, and the 2-step (K = 256) pipeline
    w, acts, wts = _custom(24, d, f, 4, 2, seed=d + f)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    err = problems.rel_max_err(got["y"], ref)
    print(f"bf16 d={d} f={f}: f32-out rel max err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("T,E,k,coarse", [
    (20, 100, 6, False),      # E not a multiple of 64
    (24, 128, 8, True),       # many exact ties
    (33, 64, 8, True),        # routing launch + single-workgroup permutation
    (16, 64, 8, True),        # routing and permutation in one workgroup (one token per wave)
    (12, 20, 6, False),
    (17, 200, 8, False),      # wave-wide argmax rounds (E > 128)
    (9, 512, 32, True),       # largest E and k the library accepts
])
def test_routing_across_expert_counts(T, E, k, coarse):
    rng = np.random.default_rng(70 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if coarse:
        logits = np.round(logits * 2) / 2                     # values on a grid of 0.5
        logits[0, :] = 0.0                                     # a token with all logits tied
        logits[1, ::2] = -0.0                                  # signed zeros tie with +0
    w, acts, wts = _custom(T, 256, 256, E, k, seed=70 + E, logits=logits)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    if coarse:
        assert np.array_equal(got["topk_ids"].reshape(T, k)[0], np.arange(k))
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)["y"]
    assert problems.rel_max_err(got["y"], ref) <= TOL


def test_all_tokens_on_the_same_experts_multi_chunk():
    T, E, k = 150, 8, 2                                  # 150 pairs per expert: 3 chunks
    logits = np.zeros((T, E), np.float32)
    logits[:, 5] = 3.0
    logits[:, 2] = 2.0 + np.linspace(0, 0.5, T, dtype=np.float32)
    w, acts, wts = _custom(T, 256, 512, E, k, seed=60, logits=logits)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    assert got["expert_offsets"][E] == T * k
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)["y"]
    assert problems.rel_max_err(got["y"], ref) <= TOL


def test_exact_logit_ties_pick_lowest_experts():
    T, E, k = 16, 8, 3
    logits = np.zeros((T, E), np.float32)
    logits[::2, 7] = 1.0
    w, acts, wts = _custom(T, 256, 256, E, k, seed=61, logits=logits)
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    ids = got["topk_ids"].reshape(T, k)
    assert np.array_equal(ids[1], [0, 1, 2]) and np.array_equal(ids[0], [7, 0, 1])


def _edge_logits(T, E, seed):
    """Rows in turn: small integers (many exact ties), signed zeros with a
    few -1s (+0 and -0 compare equal, so the lower index wins), -inf but for
    three finite logits (fewer than k: the rest of the selection is -inf,
    lowest indices first, each with weight 0), and normal values."""
    rng = np.random.default_rng(seed)
    L = np.empty((T, E), np.float32)
    for t in range(T):
        kind = t % 4
        if kind == 0:
            L[t] = rng.integers(-2, 3, E)
        elif kind == 1:
            L[t] = np.where(rng.random(E) < 0.5, 0.0, -0.0)
            L[t, rng.choice(E, 3, replace=False)] = -1.0
        elif kind == 2:
            L[t] = -np.inf
            L[t, rng.choice(E, 3, replace=False)] = rng.standard_normal(3)
        else:
            L[t] = rng.standard_normal(E)
    assert np.signbit(L[1]).any() and (L[1] == 0).sum() > 3
    return L


@pytest.mark.parametrize("T,E,k", [(8, 64, 8), (8, 100, 8), (8, 128, 8),      # routed inside the expert launch
                                   (40, 64, 8), (40, 100, 6), (40, 200, 8), (24, 512, 8)])
def test_routing_edge_values_on_every_routing_path(T, E, k):
    """Exact ties, -0 against +0 and -inf logits, through the ranking (up to
    64 experts) and the argmax rounds (65-512), both in the routing launches
    and inside the expert launch of one verify block: the oracle's strict
    comparison (value descending, then the lower index) gives the ids, and
    a -inf slot weight 0."""
    w, acts, wts = _custom(T, 256, 256, E, k, seed=70 + E + T, logits=_edge_logits(T, E, 170 + E + T))
    got, _ = _run(w, acts, problems.to_device(wts))
    _check_routing(w, acts, got)
    ids = got["topk_ids"].reshape(T, k)
    assert np.array_equal(ids[2][3:], np.sort(ids[2][3:]))      # the -inf part: ascending indices
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, k)["y"]
    assert np.isfinite(got["y"]).all() and problems.rel_max_err(got["y"], ref) <= TOL


def test_zero_weights_give_zero_output():
    w, acts, wts = _custom(8, 256, 256, 4, 2, seed=62)
    for n in ("w_gate", "w_up", "w_down"):
        wts[n][:] = 0
    got, _ = _run(w, acts, problems.to_device(wts))
    assert np.all(got["y"] == 0.0)


def test_scaled_weights_exercise_far_scale_bytes():
    w, acts, wts = _custom(16, 256, 256, 4, 2, seed=63)
    for n, sh in (("w_gate_scale", 40), ("w_up_scale", -30), ("w_down_scale", 50)):
        wts[n] = (wts[n].astype(np.int32) + sh).astype(np.uint8)
    got, _ = _run(w, acts, problems.to_device(wts))
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, 2)["y"]
    assert np.isfinite(ref).all()
    assert problems.rel_max_err(got["y"], ref) <= TOL


def test_deterministic_and_workspace_reuse():
    moe = _moe()
    w, acts, wts = _custom(40, 256, 256, 8, 2, seed=64)
    dev = problems.to_device(wts)
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=40, out_dtype=moe.OUT_F32)
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    a = layer(x, lg).clone()
    b = layer(x, lg).clone()
    assert torch.equal(a, b)
    small = layer(x[:7], lg[:7]).clone()               # same workspace, fewer tokens
    big = layer(x, lg).clone()
    torch.cuda.synchronize()
    ref = oracle.moe_forward(acts["x_bf16"][:7], acts["logits"][:7], wts, w.k)["y"]
    assert problems.rel_max_err(small.cpu().numpy(), ref) <= TOL
    assert torch.equal(big, a)


def test_tile_weights_matches_header_formula():
    moe = _moe()
    rng = np.random.default_rng(70)
    for rows, K in ((32, 256), (48, 512), (16, 1536), (64, 2048)):
        p = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
        s = rng.integers(0, 255, (rows, K // 32), dtype=np.uint8)
        tp, ts = moe.tile_weights(torch.from_numpy(p).cuda(), torch.from_numpy(s).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(tp.cpu().numpy(), tiling.tile_packed(p)), (rows, K)
        assert np.array_equal(ts.cpu().numpy(), tiling.tile_scales(s)), (rows, K)
