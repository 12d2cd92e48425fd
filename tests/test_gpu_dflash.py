"""GPU parity of the DFlash verify acceptance (moe_mxfp4_dflash_accept).

The result is integers: the accepted count decided by float32 comparisons
(both sides compute u * p_draft and compare in float32) and an index drawn
by exact integer sums, so it must equal the oracle's bit for bit on every
input, including those outside the method's domain (tokens outside the
vocabulary, NaN and negative entries, r outside [0, 1)).
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KEYS = ("draft", "p_draft", "p_target", "u", "r")


def _moe():
    import mxfp4_expert_ffn_amd as moe
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return moe


def _dev(inp):
    return [torch.from_numpy(np.ascontiguousarray(inp[k])).cuda() for k in KEYS]


def _check(moe, inp, workspace=None, label=""):
    n_gpu, tok_gpu = moe.dflash_accept(*_dev(inp), workspace=workspace)
    torch.cuda.synchronize()
    n_ref, tok_ref = oracle.dflash_accept(*[inp[k] for k in KEYS])
    n_gpu, tok_gpu = n_gpu.cpu().numpy(), tok_gpu.cpu().numpy()
    bad = np.nonzero((n_gpu != n_ref) | (tok_gpu != tok_ref))[0]
    assert bad.size == 0, (label, bad[:8], n_gpu[bad[:8]], n_ref[bad[:8]], tok_gpu[bad[:8]], tok_ref[bad[:8]])
    return n_ref, tok_ref


def test_dflash_verify_32seq_full_vocabulary():
    # 32 sequences x block 8 over the full vocabulary: the measured shape
    moe = _moe()
    B, G, V = 32, 8, synth.DFLASH_VOCAB
    inp = synth.dflash_batch(B, G, V, seed=2001)
    n, tok = _check(moe, inp, label="verify_32seq")
    assert 0 < (n == G).sum() < B                   # both the residual and the bonus draw occur
    print(f"dflash B={B} G={G} V={V}: mean accepted {n.mean():.2f}, whole block {np.mean(n == G):.0%}")


@pytest.mark.parametrize("B,G,V,eps", [
    (5, 8, 1001, 0.5),        # V % 4 != 0: scalar loads, ragged last block
    (7, 3, 4100, 0.8),        # float4 loads, last block partly past V
    (3, 1, 5, 1.0),           # a single partial block
    (16, 64, 2048, 0.05),     # the largest block (one lane per position)
    (4, 0, 300, 0.1),         # no drafted tokens: a plain draw from p_target
    (1, 8, 256, 0.3),         # exactly one block
    (9, 8, 70000, 0.3),       # many workgroups per row, ragged in blocks of 16
    (600, 2, 512, 2.0),       # many sequences, mostly rejected
])
def test_dflash_matches_oracle_on_ragged_shapes(B, G, V, eps):
    moe = _moe()
    inp = synth.dflash_batch(B, G, V, seed=2100 + V, eps=eps)
    _check(moe, inp, label=f"B={B} G={G} V={V}")


def test_dflash_edge_cases():
    moe = _moe()
    rng = np.random.default_rng(2200)
    B, G, V = 12, 8, 1024
    base = synth.dflash_batch(B, G, V, seed=2201, eps=0.4)

    # identical drafter and target: every token is accepted
    same = dict(base)
    same["p_draft"] = np.ascontiguousarray(base["p_target"][:, :G])
    n, _ = _check(moe, same, label="identical")
    assert np.all(n == G)

    # p_target = p_draft / 2 at the drafted positions and u = 0.75: rejected
    # at once with an all-zero residual, so the draw falls back to p_target
    half = dict(base)
    pt = base["p_target"].copy()
    pt[:, :G] = base["p_draft"] * np.float32(0.5)
    half["p_target"], half["u"] = pt, np.full((B, G), 0.75, np.float32)
    n, tok = _check(moe, half, label="zero residual")
    assert np.all(n == 0) and np.all(tok >= 0)

    # drafted tokens outside the vocabulary are rejected
    oob = dict(base)
    d = base["draft"].copy()
    d[np.arange(B), np.arange(B) % G] = np.array([-1, V, 2 ** 31 - 1, -2 ** 31] * 3, np.int32)
    oob["draft"] = d
    n, _ = _check(moe, oob, label="out of range")
    assert np.all(n <= np.arange(B) % G)

    # NaN, negative and zero entries in the rows drawn from
    junk = dict(base)
    pt = base["p_target"].copy()
    mask = rng.random(pt.shape) < 0.2
    pt[mask] = np.where(rng.random(pt.shape) < 0.5, np.float32(np.nan), np.float32(-0.5))[mask]
    junk["p_target"] = pt
    _check(moe, junk, label="junk entries")

    # r at and beyond the ends of [0, 1)
    ends = dict(base)
    ends["r"] = np.array([0.0, np.float32(1.0) - np.float32(2.0 ** -24), 1.0, 2.0, -1.0, np.nan,
                          np.inf, -np.inf, 2.0 ** -24, 0.5, 0.25, 0.999], np.float32)
    _check(moe, ends, label="r ends")

    # one-hot target rows, all-zero rows (no token: -1) and u = 0
    onehot = dict(base)
    pt = np.zeros_like(base["p_target"])
    hot = rng.integers(0, V, size=(B, G + 1))
    pt[np.arange(B)[:, None], np.arange(G + 1)[None, :], hot] = 1.0
    pt[0] = 0.0                                      # sequence 0: nothing to draw anywhere
    onehot["p_target"], onehot["u"] = pt, np.zeros((B, G), np.float32)
    n, tok = _check(moe, onehot, label="one-hot")
    assert tok[0] == -1


def test_dflash_workspace_holds_no_state_and_streams_work():
    moe = _moe()
    big = synth.dflash_batch(24, 8, 20000, seed=2301)
    small = synth.dflash_batch(5, 4, 3000, seed=2302)
    ws = torch.empty(moe.dflash_workspace_bytes(24, 20000), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)                                   # no initial contents are needed
    _check(moe, big, workspace=ws, label="big")
    _check(moe, small, workspace=ws, label="small after big")
    _check(moe, big, workspace=ws, label="big again")
    # on a side stream behind unrelated work, the same answer
    side = torch.cuda.Stream()
    ref = [t.cpu().numpy() for t in moe.dflash_accept(*_dev(big))]
    with torch.cuda.stream(side):
        a = torch.randn(2048, 2048, device="cuda")
        for _ in range(4):
            a = a @ a.T * 1e-3
        got = moe.dflash_accept(*_dev(big), stream=side)
    side.synchronize()
    assert np.array_equal(got[0].cpu().numpy(), ref[0]) and np.array_equal(got[1].cpu().numpy(), ref[1])


def test_dflash_replays_from_a_hip_graph():
    # the pass allocates nothing, copies nothing and does not synchronise, so
    # it can be captured; replays with new inputs match eager calls
    moe = _moe()
    B, G, V = 6, 8, 5000
    first = synth.dflash_batch(B, G, V, seed=2401)
    dev = _dev(first)
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.dflash_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.dflash_accept(*dev, n_accepted=n, next_token=tok, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.dflash_accept(*dev, n_accepted=n, next_token=tok, workspace=ws)
    torch.cuda.synchronize()
    for i in range(3):
        inp = synth.dflash_batch(B, G, V, seed=2410 + i)
        for t, k in zip(dev, KEYS):
            t.copy_(torch.from_numpy(np.ascontiguousarray(inp[k])).cuda())
        g.replay()
        torch.cuda.synchronize()
        n_ref, tok_ref = oracle.dflash_accept(*[inp[k] for k in KEYS])
        assert np.array_equal(n.cpu().numpy(), n_ref) and np.array_equal(tok.cpu().numpy(), tok_ref), i
