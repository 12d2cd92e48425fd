"""GPU behaviour of the C ABI beyond the numbers: streams, stage timing,
several contexts over one weight set, and workspaces sized for fewer tokens
than the context allows.  Results are compared bit for bit between runs (the
path is deterministic) and, once, against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import problems

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


@pytest.fixture(scope="module")
def small():
    w = synth.Workload("api", 40, 512, 1024, 8, 2, "bf16", "none", 404)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    return w, acts, wts, problems.to_device(wts)


def _inputs(acts, T):
    x = torch.from_numpy(acts["x_bf16"][:T].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"][:T]).cuda()
    return x, lg


def test_forward_on_a_side_stream_matches_the_default_stream(small):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    x, lg = _inputs(acts, w.T)
    y0 = layer(x, lg).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()                     # default priority
    with torch.cuda.stream(side):
        # queue unrelated work first so the call really runs behind it
        busy = torch.randn(2048, 2048, device="cuda")
        for _ in range(4):
            busy = busy @ busy.T * 1e-3
        y1 = layer(x, lg, stream=side)
    side.synchronize()
    assert torch.equal(y0, y1)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    assert problems.rel_max_err(y1.cpu().numpy(), ref) <= TOL


def test_two_contexts_over_one_weight_set(small):
    moe = _moe()
    w, acts, wts, dev = small
    a = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    b = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_BF16)
    x, lg = _inputs(acts, w.T)
    ya = a(x, lg)
    yb = b(x, lg)
    torch.cuda.synchronize()
    # the bf16 output is the float32 one rounded once
    assert torch.equal(yb, ya.bfloat16())
    a.close()
    yb2 = b(x, lg)                                  # b still works after a is destroyed
    torch.cuda.synchronize()
    assert torch.equal(yb, yb2)


def test_workspace_for_fewer_tokens_than_the_context_allows(small):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    for T in (1, 7, 17):
        ws = torch.empty(layer.workspace_bytes(T), dtype=torch.uint8, device="cuda")
        x, lg = _inputs(acts, T)
        y = layer(x, lg, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.moe_forward(acts["x_bf16"][:T], acts["logits"][:T], wts, w.k)["y"]
        assert problems.rel_max_err(y.cpu().numpy(), ref) <= TOL, T
        # the first T rows of a full-batch call are the same tokens
        yfull = layer(*_inputs(acts, w.T))
        torch.cuda.synchronize()
        assert torch.equal(y, yfull[:T])


def test_stage_timing_records_every_stage(small):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T)
    x, lg = _inputs(acts, w.T)
    y0 = layer(x, lg).clone()
    layer.stage_timing(4)
    for _ in range(3):
        y = layer(x, lg)
    torch.cuda.synchronize()
    times, n = layer.stage_times()
    assert n == 3
    assert set(times) == set(moe.STAGES)
    for name, ms in times.items():
        assert ms >= 0.0, name
        # no activation quantisation in bf16 mode; 40 tokens over 8 experts
        # route and permute in one launch, timed as the routing stage
        if name not in ("quant", "sort"):
            assert ms > 0.0, name
    assert torch.equal(y, y0)                       # timing does not change the result
    layer.stage_timing(0)                            # stop recording: nothing left to read
    y = layer(x, lg)
    torch.cuda.synchronize()
    with pytest.raises(moe.MoeError):
        layer.stage_times()
    assert torch.equal(y, y0)


def test_forward_replays_from_a_hip_graph(small):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    x, lg = _inputs(acts, w.T)
    ws = torch.empty(layer.workspace_bytes(w.T), dtype=torch.uint8, device="cuda")
    y_graph = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()                     # warm-up off the default stream, as capture expects
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x, lg, out=y_graph, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, lg, out=y_graph, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    for i in range(3):
        # new inputs in the captured buffers, a replay, then the eager call
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x.copy_(torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16))
        lg.copy_(torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32)).cuda())
        g.replay()
        torch.cuda.synchronize()
        y_eager = layer(x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), i


def test_empty_calls_are_no_ops(small):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    x, lg = _inputs(acts, w.T)
    y0 = layer(x, lg).clone()
    y = layer(x[:0], lg[:0])                        # no tokens: nothing launched, nothing written
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, w.d)
    n, tok = moe.dflash_accept(torch.zeros((0, 8), dtype=torch.int32, device="cuda"),
                               torch.zeros((0, 8, 16), device="cuda"), torch.zeros((0, 9, 16), device="cuda"),
                               torch.zeros((0, 8), device="cuda"), torch.zeros(0, device="cuda"))
    torch.cuda.synchronize()
    assert n.numel() == 0 and tok.numel() == 0
    assert torch.equal(layer(x, lg), y0)            # the context is unaffected


def test_probes_report_their_work_and_run():
    moe = _moe()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    assert moe.probe(moe.PROBE_STREAM, src=src, sink=sink) == float(1 << 20)
    # MFMA kinds: 2048 workgroups x 4 waves x 32 reps-rounds x 8 MFMAs
    per = {moe.PROBE_MFMA_BF16: 2 * 16 * 16 * 32, moe.PROBE_MFMA_FP8_FP4: 2 * 16 * 16 * 128,
           moe.PROBE_MFMA_FP4_FP4: 2 * 16 * 16 * 128, moe.PROBE_MFMA_BF16_RANDOM: 2 * 16 * 16 * 32,
           moe.PROBE_MFMA_FP8_FP4_RANDOM: 2 * 16 * 16 * 128, moe.PROBE_MFMA_FP4_FP4_RANDOM: 2 * 16 * 16 * 128}
    for kind, flops in per.items():
        assert moe.probe(kind, reps=1, sink=sink) == float(flops * 8 * 32 * 2048 * 4)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0                     # the sink is never written by real work


@pytest.mark.parametrize("site", ["route", "gateup", "down", "combine"])
def test_a_failed_launch_is_reported_and_leaves_the_context_usable(small, site, monkeypatch):
    # MOE_MXFP4_FAULT makes the call fail at one launch site as a failed
    # launch would; the error comes back as MOE_ERR_HIP and the next call,
    # with nothing failing, gives the same bits as before
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=moe.OUT_F32)
    x, lg = _inputs(acts, w.T)
    y0 = layer(x, lg).clone()
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_MXFP4_FAULT", site)
    with pytest.raises(moe.MoeError) as ei:
        layer(x, lg)
    assert ei.value.status == 6                       # MOE_ERR_HIP
    monkeypatch.delenv("MOE_MXFP4_FAULT")
    torch.cuda.synchronize()
    assert torch.equal(layer(x, lg), y0)


@pytest.mark.parametrize("site", ["gateup", "combine"])
def test_a_failed_call_is_not_counted_by_stage_timing(small, site, monkeypatch):
    # a call that fails part-way has recorded only some of its events: it
    # must not be summed, and the slot it used must be reusable
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T)
    x, lg = _inputs(acts, w.T)
    for cap, good_before, expect in ((4, 2, 2), (2, 2, 1)):
        layer.stage_timing(cap)
        for _ in range(good_before):
            layer(x, lg)
        monkeypatch.setenv("MOE_MXFP4_FAULT", site)
        with pytest.raises(moe.MoeError):
            layer(x, lg)
        monkeypatch.delenv("MOE_MXFP4_FAULT")
        torch.cuda.synchronize()
        # cap 4: slots 0, 1 hold good calls, the failed one is not counted;
        # cap 2: the failed call reused slot 0, so only slot 1 is whole
        times, n = layer.stage_times()
        assert n == expect, (cap, n)
        assert all(v >= 0.0 for v in times.values())
        assert times["gateup"] > 0.0 and times["combine"] > 0.0
        # after the failure the next good call records normally
        layer(x, lg)
        torch.cuda.synchronize()
        times, n = layer.stage_times()
        assert n == 1 and times["combine"] > 0.0
    layer.stage_timing(0)


def test_a_failed_acceptance_launch_is_reported(monkeypatch):
    moe = _moe()
    d = synth.dflash_batch(3, 4, 300, seed=12)
    args = [torch.from_numpy(d[k]).cuda() for k in ("draft", "p_draft", "p_target", "u", "r")]
    n0, t0 = [t.clone() for t in moe.dflash_accept(*args)]
    monkeypatch.setenv("MOE_MXFP4_FAULT", "dflash")
    with pytest.raises(moe.MoeError) as ei:
        moe.dflash_accept(*args)
    assert ei.value.status == 6
    monkeypatch.delenv("MOE_MXFP4_FAULT")
    n1, t1 = moe.dflash_accept(*args)
    torch.cuda.synchronize()
    assert torch.equal(n0, n1) and torch.equal(t0, t1)
