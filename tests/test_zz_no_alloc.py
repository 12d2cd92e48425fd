"""moe_mxfp4_forward_noalloc, the forward variant for callers that cannot
allocate: its output and routing must equal moe_mxfp4_forward's bit for bit
(the same kernels run on the library's per-GPU scratch instead of a caller
workspace), on consecutive calls that reuse the scratch with different
sizes, and oversized calls must be refused before anything is queued."""
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
    w = synth.Workload("noalloc", 40, 512, 1024, 8, 2, "bf16", "none", 405)
    acts = synth.make_activations(w)
    wts = problems.pack_experts(w)
    return w, acts, wts, problems.to_device(wts)


def _inputs(acts, T):
    x = torch.from_numpy(acts["x_bf16"][:T].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"][:T]).cuda()
    return x, lg


def _routing(T, k, E):
    P = T * k
    return {"topk_ids": torch.full((P,), -7, dtype=torch.int32, device="cuda"),
            "topk_w": torch.full((P,), -7.0, dtype=torch.float32, device="cuda"),
            "expert_offsets": torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
            "sorted_pairs": torch.full((P,), -7, dtype=torch.int32, device="cuda")}


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_noalloc_equals_forward_on_two_calls_second_smaller(small, out_dtype):
    moe = _moe()
    w, acts, wts, dev = small
    layer = moe.MoeMxfp4(dev, w.E, w.d, w.f, w.k, max_tokens=w.T, out_dtype=out_dtype)
    odt = torch.bfloat16 if out_dtype == 0 else torch.float32
    for T in (w.T, 13):                              # the second call is smaller
        print(f"noalloc: T={T} out_dtype={out_dtype}", flush=True)
        x, lg = _inputs(acts, T)
        r_ref, r_na = _routing(T, w.k, w.E), _routing(T, w.k, w.E)
        y_ref = layer(x, lg, routing=r_ref)
        y_na = torch.full((T, w.d), 3.0, dtype=odt, device="cuda")
        layer.forward_noalloc(x, lg, y_na, routing=r_na)
        torch.cuda.synchronize()
        assert torch.equal(y_ref, y_na), T
        for n in r_ref:
            assert torch.equal(r_ref[n], r_na[n]), (T, n)
        ref = oracle.moe_forward(acts["x_bf16"][:T], acts["logits"][:T], wts, w.k)["y"]
        assert problems.rel_max_err(y_na.float().cpu().numpy(), ref) <= TOL


def test_noalloc_verify_batch_size_and_refusal():
    """The 256-token verify shape (d_model 4096, d_ff 1536, 64 experts,
    top-8) fits the scratch; a shape that does not is refused with
    MOE_ERR_WORKSPACE and leaves the output untouched."""
    moe = _moe()
    E, d, f, k = 64, 4096, 1536, 8
    rng = np.random.default_rng(9)
    wts = {"w_gate": rng.integers(0, 256, (E, f, d // 2), dtype=np.uint8),
           "w_gate_scale": rng.integers(118, 124, (E, f, d // 32), dtype=np.uint8),
           "w_up": rng.integers(0, 256, (E, f, d // 2), dtype=np.uint8),
           "w_up_scale": rng.integers(118, 124, (E, f, d // 32), dtype=np.uint8),
           "w_down": rng.integers(0, 256, (E, d, f // 2), dtype=np.uint8),
           "w_down_scale": rng.integers(118, 124, (E, d, f // 32), dtype=np.uint8)}
    dev = problems.to_device(wts)
    layer = moe.MoeMxfp4(dev, E, d, f, k, max_tokens=1024)
    assert layer.workspace_bytes(256) <= moe.NOALLOC_SCRATCH_BYTES < layer.workspace_bytes(1024)
    for T in (256, 8):
        print(f"noalloc: verify shape T={T}", flush=True)
        x = (torch.randn(T, d, device="cuda") * 1.0).to(torch.bfloat16)
        lg = torch.randn(T, E, device="cuda")
        y_ref = layer(x, lg)
        y_na = torch.empty_like(y_ref)
        layer.forward_noalloc(x, lg, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_ref, y_na), T
    x = torch.zeros(1024, d, dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(1024, E, device="cuda")
    y = torch.full((1024, d), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        layer.forward_noalloc(x, lg, y)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
