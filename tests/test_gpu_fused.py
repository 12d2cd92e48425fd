"""The persistent fused kernel (MOE_MXFP4_PATH=fused) against the per-phase
launches (MOE_MXFP4_PATH=stream), through the C ABI.

Both paths run the same unit pipeline with the same accumulation order, so
the layer output, the routing outputs and the permutation must agree bit for
bit; one case per workload is also checked against the oracle.  The fused
kernel's cross-workgroup waits are bounded: forcing every wait to give up
(MOE_MXFP4_SPIN_LIMIT < 0) must raise the device-side error word while every
workgroup exits normally, and the next call must be exact again.
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


def _layers(monkeypatch, dev, w, max_tokens, out_dtype):
    moe = _moe()
    made = {}
    for path in ("stream", "fused"):
        monkeypatch.setenv("MOE_MXFP4_PATH", path)
        made[path] = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=max_tokens, out_dtype=out_dtype)
    monkeypatch.delenv("MOE_MXFP4_PATH")
    return made["stream"], made["fused"]


def _routing(T, k, E):
    P = T * k
    return {"topk_ids": torch.full((P,), -5, dtype=torch.int32, device="cuda"),
            "topk_w": torch.full((P,), -5.0, dtype=torch.float32, device="cuda"),
            "expert_offsets": torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"),
            "sorted_pairs": torch.full((P,), -5, dtype=torch.int32, device="cuda")}


def _compare(monkeypatch, w, acts, wts_dev, T=None, out_dtype=1):
    T = w.T if T is None else T
    stream_l, fused_l = _layers(monkeypatch, wts_dev, w, T, out_dtype)
    x = torch.from_numpy(acts["x_bf16"][:T].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"][:T]).cuda()
    rs, rf = _routing(T, w.k, w.E), _routing(T, w.k, w.E)
    print(f"fused vs stream: {w.name} T={T} E={w.E} k={w.k} d={w.d} f={w.f}", flush=True)
    ys = stream_l(x, lg, routing=rs)
    yf = fused_l(x, lg, routing=rf)
    torch.cuda.synchronize()
    assert fused_l.device_status(T) == 0
    assert torch.equal(ys, yf)
    for n in rs:
        assert torch.equal(rs[n], rf[n]), n
    return yf


@pytest.mark.parametrize("T,E,k,d,f", [
    (8, 4, 2, 256, 512),          # the tiny workload's shape
    (1, 8, 2, 512, 1024),         # one token
    (13, 8, 2, 512, 1024),        # ragged
    (40, 8, 8, 512, 1024),        # k = E
    (37, 1, 1, 512, 256),         # E = 1, K = 256 steps for down
    (150, 2, 1, 256, 512),        # 75 pairs per expert on average: experts with 2 chunks
    (100, 128, 8, 512, 512),      # E > 64 (argmax routing)
    (64, 300, 4, 256, 512),       # E > 256: two experts per prefix thread
])
def test_fused_equals_stream_small(monkeypatch, T, E, k, d, f):
    w = synth.Workload("fz", T, d, f, E, k, "bf16", "normal", 700 + T + E)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    yf = _compare(monkeypatch, w, acts, problems.to_device(wts))
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    assert problems.rel_max_err(yf.cpu().numpy(), ref) <= TOL


def test_fused_all_pairs_on_one_expert(monkeypatch):
    # every token picks experts 0 and 1 first: 2 experts x 200 pairs = 4
    # chunks each, the rest untouched
    w = synth.Workload("fz1", 200, 256, 512, 16, 2, "bf16", "none", 77)
    acts = dict(synth.make_activations(w))
    lg = acts["logits"].copy()
    lg[:, 0] += 50.0
    lg[:, 1] += 40.0
    acts["logits"] = lg
    wts = problems.pack_experts(w)
    yf = _compare(monkeypatch, w, acts, problems.to_device(wts))
    ref = oracle.moe_forward(acts["x_bf16"], acts["logits"], wts, w.k)["y"]
    assert problems.rel_max_err(yf.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("name", ["verify_1seq", "verify_32seq", "share_64seq"])
def test_fused_equals_stream_full_size(monkeypatch, name):
    w = synth.workload(name)
    acts, wts = problems.problem(w)
    _compare(monkeypatch, w, acts, problems.to_device(wts), out_dtype=0)


def test_forced_wait_timeout_raises_the_error_word_and_recovers(monkeypatch):
    moe = _moe()
    w = synth.Workload("fzt", 40, 512, 1024, 8, 2, "bf16", "none", 909)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    dev = problems.to_device(wts)
    stream_l, fused_l = _layers(monkeypatch, dev, w, w.T, 1)
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    y_ref = stream_l(x, lg).clone()
    monkeypatch.setenv("MOE_MXFP4_SPIN_LIMIT", "-1")
    print("fused: forced wait timeout", flush=True)
    fused_l(x, lg)                                     # every workgroup gives up and exits
    torch.cuda.synchronize()
    assert fused_l.device_status(w.T) == 1
    monkeypatch.delenv("MOE_MXFP4_SPIN_LIMIT")
    y = fused_l(x, lg)
    torch.cuda.synchronize()
    assert fused_l.device_status(w.T) == 0
    assert torch.equal(y, y_ref)
    # paths without device-side waits always report 0
    assert stream_l.device_status(w.T) == 0


def test_fused_replays_from_a_hip_graph(monkeypatch):
    w = synth.Workload("fzg", 64, 512, 1024, 16, 4, "bf16", "normal", 910)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    dev = problems.to_device(wts)
    stream_l, fused_l = _layers(monkeypatch, dev, w, w.T, 1)
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    ws = torch.empty(fused_l.workspace_bytes(w.T), dtype=torch.uint8, device="cuda")
    y_graph = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fused_l(x, lg, out=y_graph, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fused_l(x, lg, out=y_graph, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    for i in range(4):
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x.copy_(torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16))
        lg.copy_(torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32)).cuda())
        print(f"fused: graph replay {i}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert fused_l.device_status(w.T, workspace=ws) == 0
        y_eager = stream_l(x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), i


def test_fused_alternating_inputs_on_one_workspace(monkeypatch):
    # consecutive calls with different inputs (and routing) on the same
    # workspace: every value a call reads must come from that call, so a
    # stale h row, list or count from the previous call would show here
    moe = _moe()
    w = synth.workload("verify_32seq")
    acts, wts = problems.problem(w)
    stream_l, fused_l = _layers(monkeypatch, problems.to_device(wts), w, w.T, 0)
    ws = torch.empty(fused_l.workspace_bytes(w.T), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(11)
    inputs = []
    for _ in range(3):
        xi = synth.bf16_bits_from_f32(rng.standard_normal((w.T, w.d)).astype(np.float32))
        x = torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16)
        lg = torch.from_numpy(rng.standard_normal((w.T, w.E)).astype(np.float32) * 2).cuda()
        inputs.append((x, lg, stream_l(x, lg).clone()))
    torch.cuda.synchronize()
    for i in range(9):
        x, lg, y_ref = inputs[i % 3]
        y = fused_l(x, lg, workspace=ws)
        torch.cuda.synchronize()
        assert fused_l.device_status(w.T, workspace=ws) == 0
        assert torch.equal(y, y_ref), i


def test_fused_repeated_calls_are_bit_identical(monkeypatch):
    w = synth.workload("verify_32seq")
    acts, wts = problems.problem(w)
    _, fused_l = _layers(monkeypatch, problems.to_device(wts), w, w.T, 0)
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    y0 = fused_l(x, lg).clone()
    for i in range(20):
        y = fused_l(x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), i
    assert fused_l.device_status(w.T) == 0


@pytest.mark.parametrize("T,E,k", [(8, 64, 8), (96, 16, 4)])     # persistent form (P <= E), ticketed form
def test_fused_calls_on_two_streams_at_once(monkeypatch, T, E, k):
    # two calls in flight together on distinct workspaces: each kernel's
    # units are handed out to running workgroups only, so neither waits on
    # work that the other's workgroups keep from starting
    w = synth.Workload("fzs", T, 512, 1024, E, k, "bf16", "normal", 915)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    stream_l, fused_l = _layers(monkeypatch, problems.to_device(wts), w, w.T, 1)
    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    y_ref = stream_l(x, lg).clone()
    nbytes = fused_l.workspace_bytes(w.T)
    ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty((w.T, w.d), dtype=torch.float32, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    print(f"fused: two streams, T={T} E={E} k={k}", flush=True)
    for _ in range(6):
        for st, wsp, out in zip(streams, ws, outs):
            with torch.cuda.stream(st):
                fused_l(x, lg, out=out, workspace=wsp)
    torch.cuda.synchronize()
    for st, wsp, out in zip(streams, ws, outs):
        assert fused_l.device_status(w.T, workspace=wsp, stream=st) == 0
        assert torch.equal(out, y_ref)
