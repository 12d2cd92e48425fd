"""The expert launch that routes a verify block itself (routing, permutation,
gate/up and down in one persistent launch, then the combine) against the
paths that route in launches of their own, through the C ABI.

Every path runs the same routing code, the same unit pipeline and the same
combine, so the layer output and the routing outputs must agree bit for bit
with MOE_MXFP4_PATH=stream and =fused_launches; each case is also checked
against the oracle.  The kernel keeps its counters in a per-stream state
block that every call's combine launch must leave clear: repeated and
alternating calls on one stream, graph replays, calls on two streams at once,
more streams than blocks, and a call whose waits are forced to give up
(MOE_MXFP4_SPIN_LIMIT < 0) followed by exact calls again check that.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import problems

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
PATHS = ("stream", "fused_launches", "fused")


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


def _layers(monkeypatch, dev, w, out_dtype):
    moe = _moe()
    made = {}
    for path in PATHS:
        monkeypatch.setenv("MOE_MXFP4_PATH", path)
        made[path] = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=out_dtype)
    monkeypatch.delenv("MOE_MXFP4_PATH")
    return made


def _routing(T, k, E):
    P = T * k
    return {"topk_ids": torch.full((P,), -5, dtype=torch.int32, device="cuda"),
            "topk_w": torch.full((P,), -5.0, dtype=torch.float32, device="cuda"),
            "expert_offsets": torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"),
            "sorted_pairs": torch.full((P,), -5, dtype=torch.int32, device="cuda")}


def _inputs(acts):
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    return x, lg


def _eligible(w):
    return w.E <= 128 and w.T * w.k <= 64 and w.T * w.k <= w.E and w.T * w.E <= 1024


@pytest.mark.parametrize("T,E,k,d,f,out_dtype", [
    (8, 64, 8, 512, 1024, 1),     # one verify block at top-8 of 64
    (8, 64, 8, 512, 1024, 0),     # bf16 output
    (1, 8, 2, 512, 1024, 1),      # one token
    (3, 16, 4, 256, 512, 1),      # ragged block
    (1, 1, 1, 512, 256, 1),       # E = 1, K = 256 steps for down
    (16, 64, 4, 256, 512, 0),     # 16 tokens: 4 routed per wave, 1024 logits
    (5, 40, 8, 1024, 512, 1),     # E not a power of two
    (8, 128, 8, 512, 1024, 0),    # 128 experts: two logits per lane, argmax rounds, two experts per lane
    (4, 100, 6, 512, 512, 1),     # 65..128 experts, E not a power of two
    (1, 96, 8, 256, 512, 1),
])
def test_layer_equals_multi_launch_paths(monkeypatch, T, E, k, d, f, out_dtype):
    w = synth.Workload("ly", T, d, f, E, k, "bf16", "normal", 1200 + T + E + d)
    assert _eligible(w)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, out_dtype)
    x, lg = _inputs(acts)
    print(f"layer vs launches: T={T} E={E} k={k} d={d} f={f} out={out_dtype}", flush=True)
    ys, rs = {}, {}
    for p in PATHS:
        rs[p] = _routing(T, k, E)
        ys[p] = made[p](x, lg, routing=rs[p]).clone()
    torch.cuda.synchronize()
    assert made["fused"].device_status(T) == 0
    for p in ("stream", "fused_launches"):
        assert torch.equal(ys["fused"], ys[p]), p
        for n in rs[p]:
            assert torch.equal(rs["fused"][n], rs[p][n]), (p, n)
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    assert problems.rel_max_err(ys["fused"].float().cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("name,T", [("verify_1seq", None), ("share_64seq", 8)])
def test_layer_full_size_verify_block_equals_launches(monkeypatch, name, T):
    w = synth.workload(name)
    if T is not None:                                  # one verify block of that model
        w = synth.Workload(w.name, T, w.d, w.f, w.E, w.k, w.act, w.bias, w.seed)
    assert _eligible(w)
    acts, wts = problems.problem(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 0)
    x, lg = _inputs(acts)
    print(f"layer vs launches: {name} T={w.T}", flush=True)
    ys = {p: made[p](x, lg).clone() for p in PATHS}
    torch.cuda.synchronize()
    assert torch.equal(ys["fused"], ys["stream"])
    assert torch.equal(ys["fused"], ys["fused_launches"])


def test_layer_alternating_and_repeated_calls(monkeypatch):
    # consecutive calls with different inputs (and routing) on one stream:
    # a counter left behind by a call, or a stale h or o row, would show here
    w = synth.Workload("lya", 8, 512, 1024, 64, 8, "bf16", "normal", 1301)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 1)
    rng = np.random.default_rng(13)
    inputs = []
    for _ in range(3):
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x = torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16)
        lg = torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32) * 2).cuda()
        inputs.append((x, lg, made["stream"](x, lg).clone()))
    torch.cuda.synchronize()
    print("layer: 30 alternating calls", flush=True)
    for i in range(30):
        x, lg, y_ref = inputs[i % 3]
        y = made["fused"](x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), i
    assert made["fused"].device_status(w.T) == 0


def test_layer_forced_wait_timeout_raises_the_error_word_and_recovers(monkeypatch):
    w = synth.Workload("lyt", 8, 512, 1024, 64, 8, "bf16", "normal", 1302)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 1)
    x, lg = _inputs(acts)
    y_ref = made["stream"](x, lg).clone()
    layer = made["fused"]
    y = layer(x, lg)
    torch.cuda.synchronize()
    assert layer.device_status(w.T) == 0 and torch.equal(y, y_ref)
    monkeypatch.setenv("MOE_MXFP4_SPIN_LIMIT", "-1")
    print("layer: forced wait timeout", flush=True)
    layer(x, lg)                                       # every down unit gives up and its workgroup exits
    torch.cuda.synchronize()
    assert layer.device_status(w.T) == 1
    monkeypatch.delenv("MOE_MXFP4_SPIN_LIMIT")
    for i in range(3):
        y = layer(x, lg)
        torch.cuda.synchronize()
        assert layer.device_status(w.T) == 0, i
        assert torch.equal(y, y_ref), i


def test_layer_replays_from_a_hip_graph(monkeypatch):
    w = synth.Workload("lyg", 8, 512, 1024, 64, 8, "bf16", "normal", 1303)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 1)
    layer = made["fused"]
    x, lg = _inputs(acts)
    y_graph = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x, lg, out=y_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, lg, out=y_graph)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    for i in range(5):
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x.copy_(torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16))
        lg.copy_(torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32)).cuda())
        print(f"layer: graph replay {i}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        y_eager = made["stream"](x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), i
        # eager work on the current stream between replays
        y_cur = layer(x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y_cur, y_eager), i


def test_layer_on_more_streams_than_state_blocks(monkeypatch):
    # streams past the library's 16 blocks per GPU route in launches of
    # their own, with the same bits
    w = synth.Workload("lym", 8, 256, 512, 64, 8, "bf16", "normal", 1304)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 1)
    x, lg = _inputs(acts)
    y_ref = made["stream"](x, lg).clone()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(24)]
    outs = [torch.empty((w.T, w.d), dtype=torch.float32, device="cuda") for _ in streams]
    print("layer: 24 streams", flush=True)
    for _ in range(2):
        for st, out in zip(streams, outs):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                made["fused"](x, lg, out=out, stream=st)
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        for out in outs:
            assert torch.equal(out, y_ref)
    for st in streams:
        assert made["fused"].device_status(w.T, stream=st) == 0


def test_layer_capture_on_a_stream_then_eager_calls_on_it(monkeypatch):
    # calls captured on a stream and eager calls on the same stream share
    # that stream's state block: replays and eager calls alternate on it,
    # each exact
    w = synth.Workload("lyc", 8, 512, 1024, 64, 8, "bf16", "normal", 1305)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    made = _layers(monkeypatch, problems.to_device(wts), w, 1)
    layer = made["fused"]
    x, lg = _inputs(acts)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    y_graph = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(layer.workspace_bytes(w.T), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    print("layer: capture on a side stream", flush=True)
    with torch.cuda.graph(g, stream=st):
        layer(x, lg, out=y_graph, workspace=ws, stream=st)
    torch.cuda.synchronize()
    rng = np.random.default_rng(35)
    for i in range(4):
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x.copy_(torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16))
        lg.copy_(torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32)).cuda())
        torch.cuda.synchronize()
        y_ref = made["stream"](x, lg).clone()
        torch.cuda.synchronize()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            y_eager = layer(x, lg, stream=st)            # eager, on the capture stream, before the replay
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_eager, y_ref), i
        assert torch.equal(y_graph, y_ref), i
        assert layer.device_status(w.T, stream=st) == 0
