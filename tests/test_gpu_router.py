"""GPU parity of the router projection and of the forward call that runs it.

Bounds: every product of two bf16 values is exact in float32, so a float32
sum of the d products, in any order and with up to 16 extra partial sums
added at the end, is within (d + 16) * u * sum_i |x_i w_i| of the exact
value (u = 2^-24); the oracle gives that exact value (in double) and the sum
of magnitudes.  The logits are checked against this worst-case bound.  It
is far from what rounding does in practice (errors of independent signs
add like a random walk), and would leave most tokens of a d = 4096 batch
too close to call, so routing uses the probabilistic bound of Higham and
Mary ("A New Approach to Probabilistic Rounding Error Analysis", SIAM J.
Sci. Comput. 2019): lambda * sqrt(n) * u * sum_i |x_i w_i| with lambda = 10,
which a sum of n terms exceeds with probability below 2 n exp(-lambda^2 / 2)
(about 1e-18 here).  Routing ids are compared exactly on tokens whose k + 1
largest exact logits are separated by more than twice that bound (both sides
then order them as the exact values do); on the other tokens the GPU's
choice is checked to be a valid top-k within the bound.  The layer output is
compared with the oracle on the unambiguous tokens, to max|y - y_ref| <=
2e-2 * RMS(y_ref).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import problems

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
U = 2.0 ** -24


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bound(d, absdot):
    return (d + 16) * U * absdot


def _bound_prob(d, absdot, lam=10.0):
    return lam * np.sqrt(d + 16) * U * absdot


def _unused_weights():
    # router_logits never reads the expert weights; the context only needs valid pointers
    t = torch.zeros(256, dtype=torch.uint8, device="cuda")
    return {n: t for n in ("w_gate", "w_gate_scale", "w_up", "w_up_scale", "w_down", "w_down_scale")}


@pytest.mark.parametrize("T,d,E", [
    (40, 512, 8), (1, 256, 1), (17, 1024, 100),   # 7 expert tiles, ragged token tile
    (300, 1536, 200),                              # 13 expert tiles, 19 token tiles
    (33, 4096, 64), (50, 512, 512),                # 32 expert tiles: two per wave
    (5, 8704, 16),                                 # 68 K steps of 128, two K splits
])
def test_router_logits_within_rounding_bound(T, d, E):
    moe = _moe()
    w = synth.Workload("router", T, d, 512, E, 1, "bf16", "none", 600 + E)
    acts = synth.make_activations(w)
    wr = synth.router_weights_bf16(w)
    layer = moe.MoeMxfp4(_unused_weights(), E, d, 512, 1, max_tokens=T)
    x = _dev_bf16(acts["x_bf16"])
    got = layer.router_logits(x, _dev_bf16(wr))
    again = layer.router_logits(x, _dev_bf16(wr))
    torch.cuda.synchronize()
    assert torch.equal(got, again)                  # deterministic
    ref, absdot = oracle.router_logits(acts["x_bf16"], wr)
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    bound = _bound(d, absdot)
    assert np.all(err <= bound), float((err / bound).max())
    print(f"router T={T} d={d} E={E}: max err / bound {float((err / bound).max()):.3e}")


@pytest.mark.parametrize("T,d,E,nsample", [
    (2000, 512, 250, None),                        # 64 x 64 tiles, ragged in tokens and experts
    (8192, 6144, 128, 48),                         # the 8192-token chunk's shape, sampled rows
])
def test_router_logits_large_batches(T, d, E, nsample):
    moe = _moe()
    w = synth.Workload("router", T, d, 512, E, 1, "bf16", "none", 650 + E)
    acts = synth.make_activations(w)
    wr = synth.router_weights_bf16(w)
    layer = moe.MoeMxfp4(_unused_weights(), E, d, 512, 1, max_tokens=T)
    got = layer.router_logits(_dev_bf16(acts["x_bf16"]), _dev_bf16(wr))
    torch.cuda.synchronize()
    rows = np.arange(T)
    if nsample is not None:
        rng = np.random.default_rng(3)
        rows = np.unique(np.concatenate([rng.choice(T, size=nsample, replace=False), [0, 63, 64, T - 1]]))
    ref, absdot = oracle.router_logits(acts["x_bf16"][rows], wr)
    err = np.abs(got.cpu().numpy()[rows].astype(np.float64) - ref)
    bound = _bound(d, absdot)
    assert np.all(err <= bound), float((err / bound).max())
    print(f"router T={T} d={d} E={E}: max err / bound {float((err / bound).max()):.3e} over {rows.size} rows")


def _check_routing(ids_gpu, w_gpu, exact, bound, k):
    """Exact on unambiguous tokens, valid top-k on the rest; returns the mask
    of unambiguous tokens."""
    T, E = exact.shape
    slack = 2.0 * (bound.max(axis=1) + U * np.abs(exact).max(axis=1))    # + float32 rounding of the logits
    order = np.lexsort((np.tile(np.arange(E), (T, 1)), -exact), axis=1)
    top = np.take_along_axis(exact, order, axis=1)[:, :min(k + 1, E)]
    gaps = -np.diff(top, axis=1)
    clear = np.all(gaps > slack[:, None], axis=1) if gaps.shape[1] else np.ones(T, bool)
    ids_ref, w_ref = oracle.route(exact.astype(np.float32), k)
    for t in range(T):
        if clear[t]:
            assert np.array_equal(ids_gpu[t], ids_ref[t]), t
            assert np.abs(w_gpu[t] - w_ref[t]).max() <= slack[t], t
        else:
            sel = ids_gpu[t]
            assert len(set(sel.tolist())) == k
            rest = np.setdiff1d(np.arange(E), sel)
            if rest.size:
                assert exact[t, sel].min() >= exact[t, rest].max() - slack[t], t
            assert np.all(np.diff(exact[t, sel]) <= slack[t]), t
    return clear


@pytest.mark.parametrize("T,d,f,E,k", [(40, 512, 512, 8, 2), (33, 1024, 256, 64, 8), (70, 512, 256, 128, 8),
                                       # one verify block, and one token: the expert launch routes the
                                       # projected logits itself
                                       (8, 512, 256, 64, 8), (1, 1024, 512, 16, 4)])
def test_forward_hidden_small(T, d, f, E, k):
    moe = _moe()
    w = synth.Workload("router", T, d, f, E, k, "bf16", "none", 700 + T)
    acts = synth.make_activations(w)
    wr = synth.router_weights_bf16(w)
    wts = problems.pack_experts(w)
    _run_and_check(moe, w, acts, wr, wts, problems.to_device(wts), sample=None)


def test_forward_hidden_verify_32seq_sampled():
    moe = _moe()
    w = synth.workload("verify_32seq")
    acts, wts = problems.problem(w)
    wr = synth.router_weights_bf16(w)
    _run_and_check(moe, w, acts, wr, wts, problems.to_device(wts), sample=12)


def _run_and_check(moe, w, acts, wr, wts, dev, sample):
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    x, wr_dev = _dev_bf16(acts["x_bf16"]), _dev_bf16(wr)
    P = w.T * w.k
    r = {"topk_ids": torch.empty(P, dtype=torch.int32, device="cuda"),
         "topk_w": torch.empty(P, dtype=torch.float32, device="cuda")}
    y = layer(x, None, w_router=wr_dev, routing=r)
    # the same call with the GPU's own logits passed in gives the same bits
    y2 = layer(x, layer.router_logits(x, wr_dev))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    exact, absdot = oracle.router_logits(acts["x_bf16"], wr)
    clear = _check_routing(r["topk_ids"].cpu().numpy().reshape(w.T, w.k),
                           r["topk_w"].cpu().numpy().reshape(w.T, w.k), exact, _bound_prob(w.d, absdot), w.k)
    assert clear.mean() >= 0.5, clear.mean()
    toks = np.nonzero(clear)[0]
    if sample is not None:
        rng = np.random.default_rng(9)
        toks = np.sort(rng.choice(toks, size=min(sample, toks.size), replace=False))
    ref = oracle.moe_forward(acts["x_bf16"][toks], exact[toks].astype(np.float32), wts, w.k,
                             nthreads=problems.THREADS)["y"]
    err = problems.rel_max_err(y.cpu().numpy()[toks], ref)
    print(f"forward_hidden {w.name} T={w.T}: {clear.mean():.0%} of tokens unambiguous, "
          f"f32-out rel max err {err:.3e} over {toks.size} of them")
    assert err <= TOL
