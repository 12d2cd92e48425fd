"""The C-ABI library: loads, exports what the header declares, and rejects
bad arguments on the host before queueing any device work (CPU only: no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import mxfp4_expert_ffn_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

FAKE = 1 << 20          # a 16-byte-aligned stand-in device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_mxfp4_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings_and_version():
    L = moe.lib()
    for s in range(8):
        assert moe.status_string(s).startswith(moe.STATUS_NAMES[s])
    assert "unknown" in moe.status_string(99)
    assert L.moe_mxfp4_abi_version() == 1


def _create(**kw):
    args = dict(num_experts=4, d_model=256, d_ff=512, top_k=2, max_tokens=8)
    args.update(kw)
    flags = args.pop("flags", 0)
    act = args.pop("act_mode", moe.ACT_BF16)
    out = args.pop("out_dtype", moe.OUT_BF16)
    cfg = moe.make_config(**args, act_mode=act, out_dtype=out, flags=flags)
    ptrs = kw.get("ptrs", [FAKE] * 6)
    w = moe.Weights(*ptrs)
    h = ctypes.c_void_p()
    st = moe.lib().moe_mxfp4_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(num_experts=0), 1), (dict(top_k=0), 1), (dict(max_tokens=0), 1),
    (dict(d_model=-256), 1), (dict(flags=1), 1), (dict(act_mode=7), 1), (dict(out_dtype=3), 1),
    (dict(top_k=5), 2), (dict(num_experts=513, top_k=2), 2), (dict(num_experts=64, top_k=33), 2),
    (dict(d_model=288), 2), (dict(d_ff=384), 2),
    (dict(act_mode=1), 0), (dict(act_mode=1, d_model=8704), 0), (dict(act_mode=1, d_model=8448), 2),
    # activation rows are addressed with 32-bit byte offsets: x (T x d) and
    # h (P x f) below 4 GiB -- 1 byte per element for MXFP8 codes, 2 for bf16
    (dict(act_mode=1, max_tokens=1 << 20, d_ff=2048), 2),
    (dict(act_mode=1, max_tokens=(1 << 20) - 1, d_ff=2048), 0),
    (dict(act_mode=1, max_tokens=1 << 20, top_k=1, d_model=4096, d_ff=256), 2),
    (dict(max_tokens=1 << 20, d_ff=2048), 2), (dict(max_tokens=1 << 19, d_ff=2048), 2),
    (dict(max_tokens=(1 << 19) - 1, d_ff=2048), 0),
    (dict(max_tokens=1 << 19, top_k=1, d_model=4096, d_ff=256), 2),
    (dict(max_tokens=(1 << 19) - 1, top_k=1, d_model=4096, d_ff=256), 0),
])
def test_create_validation(kw, status):
    ptrs = kw.pop("ptrs", None)
    st, h = _create(**kw) if ptrs is None else _create(ptrs=ptrs, **kw)
    assert st == status, moe.status_string(st)
    if st == 0:
        assert h.value and moe.lib().moe_mxfp4_destroy(h) == 0
    else:
        assert not h.value


def test_create_rejects_null_and_misaligned_weights():
    cfg = moe.make_config(4, 256, 512, 2, 8)
    L = moe.lib()
    h = ctypes.c_void_p()
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = None
        assert L.moe_mxfp4_create(ctypes.byref(cfg), ctypes.byref(moe.Weights(*ptrs)),
                                  ctypes.byref(h)) == 1
        ptrs[i] = FAKE + 8
        assert L.moe_mxfp4_create(ctypes.byref(cfg), ctypes.byref(moe.Weights(*ptrs)),
                                  ctypes.byref(h)) == 4
    assert L.moe_mxfp4_create(None, ctypes.byref(moe.Weights(*[FAKE] * 6)), ctypes.byref(h)) == 1
    bad = moe.make_config(4, 256, 512, 2, 8)
    bad.struct_size = 4
    assert L.moe_mxfp4_create(ctypes.byref(bad), ctypes.byref(moe.Weights(*[FAKE] * 6)),
                              ctypes.byref(h)) == 1
    assert L.moe_mxfp4_destroy(None) == 0


def test_workspace_bytes_grows_with_tokens():
    st, h = _create()
    L = moe.lib()
    try:
        assert L.moe_mxfp4_workspace_bytes(h, 0) == 0
        assert L.moe_mxfp4_workspace_bytes(None, 8) == 0
        a, b = L.moe_mxfp4_workspace_bytes(h, 1), L.moe_mxfp4_workspace_bytes(h, 8)
        assert 0 < a < b
        # holds the per-pair h (bf16, f wide) and weighted outputs (float, d wide)
        assert b >= 8 * 2 * (512 * 2 + 256 * 4)
    finally:
        L.moe_mxfp4_destroy(h)


def test_forward_validation_happens_before_any_launch():
    st, h = _create()
    L = moe.lib()
    need = L.moe_mxfp4_workspace_bytes(h, 8)
    fwd = L.moe_mxfp4_forward
    try:
        assert fwd(None, FAKE, FAKE, 1, FAKE, FAKE, need, None, None) == 1
        assert fwd(h, FAKE, FAKE, -1, FAKE, FAKE, need, None, None) == 1
        assert fwd(h, FAKE, FAKE, 9, FAKE, FAKE, 10**9, None, None) == 3       # > max_tokens
        assert fwd(h, None, None, 0, None, None, 0, None, None) == 0           # T = 0 no-op
        assert fwd(h, None, FAKE, 8, FAKE, FAKE, need, None, None) == 1
        assert fwd(h, FAKE, FAKE, 8, None, FAKE, need, None, None) == 1
        assert fwd(h, FAKE + 4, FAKE, 8, FAKE, FAKE, need, None, None) == 4
        assert fwd(h, FAKE, FAKE, 8, FAKE, FAKE, need - 1, None, None) == 5
        assert fwd(h, FAKE, FAKE, 8, FAKE, None, need, None, None) == 5
        assert fwd(h, FAKE, FAKE, 8, FAKE, FAKE + 8, need, None, None) == 4
        r = moe.Routing(FAKE + 2, None, None, None)
        assert fwd(h, FAKE, FAKE, 8, FAKE, FAKE, need, None, ctypes.byref(r)) == 4
    finally:
        L.moe_mxfp4_destroy(h)


def test_noalloc_forward_validates_before_touching_the_device():
    st, h = _create(max_tokens=1 << 16)
    L = moe.lib()
    na = L.moe_mxfp4_forward_noalloc
    try:
        assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20
        assert na(None, FAKE, FAKE, 1, FAKE, None, None) == 1
        assert na(h, FAKE, FAKE, -1, FAKE, None, None) == 1
        assert na(h, FAKE, FAKE, (1 << 16) + 1, FAKE, None, None) == 3     # > max_tokens
        assert na(h, None, None, 0, None, None, None) == 0                 # T = 0 no-op
        assert na(h, FAKE, None, 8, FAKE, None, None) == 1                 # no logits
        # a call whose workspace exceeds the scratch is refused (WORKSPACE)
        big = next(T for T in range(1024, 1 << 16, 1024)
                   if L.moe_mxfp4_workspace_bytes(h, T) > moe.NOALLOC_SCRATCH_BYTES)
        assert L.moe_mxfp4_workspace_bytes(h, big - 1024) <= moe.NOALLOC_SCRATCH_BYTES
        assert na(h, FAKE, FAKE, big, FAKE, None, None) == 5
        assert na(h, None, FAKE, 8, FAKE, None, None) == 1
        assert na(h, FAKE, FAKE, 8, None, None, None) == 1
    finally:
        L.moe_mxfp4_destroy(h)


def test_path_selection_and_device_status_validation(monkeypatch):
    L = moe.lib()
    for path, ok in (("stream", True), ("fused", True), ("fused_launches", True), ("", True), ("bogus", False)):
        monkeypatch.setenv("MOE_MXFP4_PATH", path)
        st, h = _create()
        assert (st == 0) == ok, (path, st)
        if st == 0:
            L.moe_mxfp4_destroy(h)
    monkeypatch.setenv("MOE_MXFP4_PATH", "stream")
    ds = L.moe_mxfp4_device_status
    st, h = _create()
    monkeypatch.delenv("MOE_MXFP4_PATH")
    out = ctypes.c_int32(7)
    try:
        assert ds(None, FAKE, 8, ctypes.byref(out), None) == 1
        assert ds(h, FAKE, 8, None, None) == 1
        assert ds(h, FAKE, -1, ctypes.byref(out), None) == 1
        assert ds(h, FAKE, 9, ctypes.byref(out), None) == 3
        # the per-phase path has no device-side waits: 0 without touching the device
        assert ds(h, FAKE, 8, ctypes.byref(out), None) == 0 and out.value == 0
    finally:
        L.moe_mxfp4_destroy(h)
    monkeypatch.setenv("MOE_MXFP4_PATH", "fused")
    st, h = _create()
    monkeypatch.delenv("MOE_MXFP4_PATH")
    try:
        out.value = 7
        assert ds(h, None, 0, ctypes.byref(out), None) == 0 and out.value == 0     # no tokens
        assert ds(h, None, 8, ctypes.byref(out), None) == 1                        # no workspace
    finally:
        L.moe_mxfp4_destroy(h)
    # a single verify block whose expert launch routes it itself keeps its
    # error word in the stream's state block: no workspace is read, and a
    # stream with no such call yet reports 0
    monkeypatch.setenv("MOE_MXFP4_PATH", "fused")
    st, h = _create(num_experts=16, max_tokens=8)
    monkeypatch.delenv("MOE_MXFP4_PATH")
    try:
        out.value = 7
        assert ds(h, None, 1, ctypes.byref(out), None) == 0 and out.value == 0
    finally:
        L.moe_mxfp4_destroy(h)


def test_router_entry_points_validate_before_any_launch():
    st, h = _create()
    L = moe.lib()
    need = L.moe_mxfp4_workspace_bytes(h, 8)
    rl, fh = L.moe_mxfp4_router_logits, L.moe_mxfp4_forward_hidden
    try:
        assert rl(None, FAKE, FAKE, 1, FAKE, None) == 1
        assert rl(h, FAKE, FAKE, -1, FAKE, None) == 1
        assert rl(h, FAKE, FAKE, 9, FAKE, None) == 3                # > max_tokens
        assert rl(h, None, None, 0, None, None) == 0                # T = 0 no-op
        assert rl(h, None, FAKE, 8, FAKE, None) == 1
        assert rl(h, FAKE, None, 8, FAKE, None) == 1
        assert rl(h, FAKE, FAKE, 8, None, None) == 1
        assert rl(h, FAKE + 2, FAKE, 8, FAKE, None) == 4
        assert rl(h, FAKE, FAKE + 8, 8, FAKE, None) == 4
        assert rl(h, FAKE, FAKE, 8, FAKE + 4, None) == 4
        assert fh(h, FAKE, None, 8, FAKE, FAKE, need, None, None) == 1     # no router weights
        assert fh(h, FAKE, FAKE, 9, FAKE, FAKE, 10**9, None, None) == 3
        assert fh(h, None, None, 0, None, None, 0, None, None) == 0
        assert fh(h, FAKE, FAKE + 4, 8, FAKE, FAKE, need, None, None) == 4
        assert fh(h, FAKE, FAKE, 8, FAKE, FAKE, need - 1, None, None) == 5
        # the forward path with logits still rejects missing logits
        assert L.moe_mxfp4_forward(h, FAKE, None, 8, FAKE, FAKE, need, None, None) == 1
    finally:
        L.moe_mxfp4_destroy(h)


def test_dflash_accept_validates_before_any_launch():
    L = moe.lib()
    wb, acc = L.moe_mxfp4_dflash_workspace_bytes, L.moe_mxfp4_dflash_accept
    B, G, V = 32, 8, 152064
    need = wb(B, V)
    # one int32 per sequence (rounded to 256 bytes) and one uint64 per 256 vocabulary entries
    assert need == 256 + B * ((V + 255) // 256) * 8
    assert wb(1, 1) == 256 + 8
    assert wb(0, 5) == 0
    assert wb(-1, 5) == 0 and wb(1, 0) == 0 and wb(1, (1 << 30) + 1) == 0 and wb(65536, 5) == 0
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None)
    assert acc(0, G, V, None, None, None, None, None, None, None, None, 0, None) == 0   # B = 0 no-op
    assert acc(-1, G, V, *ok) == 1
    assert acc(65536, G, V, *ok) == 1
    assert acc(B, -1, V, *ok) == 1
    assert acc(B, 65, V, *ok) == 1
    assert acc(B, G, 0, *ok) == 1
    assert acc(B, G, (1 << 30) + 1, *ok) == 1
    for i in range(7):                                  # each pointer argument missing in turn
        args = list(ok)
        args[i] = None
        assert acc(B, G, V, *args) == 1, i
    # G = 0: draft, p_draft and u are never read and may be NULL
    need0 = wb(B, V)
    st = acc(B, 0, V, None, None, FAKE, None, FAKE + 16, FAKE, FAKE, FAKE + 1, need0, None)
    assert st == 4                                      # reaches the checks after the NULL ones
    for i in range(7):                                  # each pointer misaligned in turn
        args = list(ok)
        args[i] = FAKE + 4
        assert acc(B, G, V, *args) == 4, i
    assert acc(B, G, V, *ok[:7], None, need, None) == 5
    assert acc(B, G, V, *ok[:8], need - 1, None) == 5
    assert acc(B, G, V, *ok[:7], FAKE + 8, need, None) == 4


def test_probe_validates_before_any_launch():
    L = moe.lib()
    pr = L.moe_mxfp4_probe
    w = ctypes.c_double()
    W = ctypes.byref(w)
    assert pr(-1, FAKE, 16, 1, FAKE, W, None) == 1
    assert pr(7, FAKE, 16, 1, FAKE, W, None) == 1
    assert pr(0, None, 16, 1, FAKE, W, None) == 1                  # stream needs a source
    assert pr(0, FAKE, 0, 1, FAKE, W, None) == 1
    assert pr(0, FAKE, 24, 1, FAKE, W, None) == 1                  # not a multiple of 16
    assert pr(0, FAKE + 8, 32, 1, FAKE, W, None) == 4
    assert pr(1, None, 0, 0, FAKE, W, None) == 1                   # reps out of range
    assert pr(2, None, 0, (1 << 20) + 1, FAKE, W, None) == 1
    assert pr(3, None, 0, 1, None, W, None) == 1                   # no sink
    assert pr(3, None, 0, 1, FAKE, None, None) == 1                # no work out-pointer
    assert pr(1, None, 0, 1, FAKE + 2, W, None) == 4


def test_debug_dequant_and_quantize_validation():
    st, h = _create()
    L = moe.lib()
    try:
        dq = L.moe_mxfp4_debug_dequant
        assert dq(h, 4, 0, 0, 1, FAKE, None) == 1          # expert out of range
        assert dq(h, 0, 3, 0, 1, FAKE, None) == 1          # matrix out of range
        assert dq(h, 0, 0, 510, 4, FAKE, None) == 1        # rows past d_ff
        assert dq(h, 0, 2, 0, 257, FAKE, None) == 1        # rows past d_model
        assert dq(h, 0, 0, 0, 1, None, None) == 1
        assert dq(h, 0, 0, 0, 1, FAKE + 4, None) == 4
        assert dq(h, 0, 0, 0, 0, FAKE, None) == 0          # nothing to do
        q = L.moe_mxfp4_quantize_weights
        assert q(FAKE, 4, 48, FAKE, FAKE, None) == 1        # K not a multiple of 32
        assert q(None, 4, 64, FAKE, FAKE, None) == 1
        assert q(FAKE, -1, 64, FAKE, FAKE, None) == 1
        assert q(FAKE + 4, 4, 64, FAKE, FAKE, None) == 4
        assert q(FAKE, 0, 64, FAKE, FAKE, None) == 0
    finally:
        L.moe_mxfp4_destroy(h)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        moe.lib()


def test_tiled_scale_bytes_and_tile_validation():
    L = moe.lib()
    assert L.moe_mxfp4_tiled_scale_bytes(32, 256) == 2 * 1 * 256
    assert L.moe_mxfp4_tiled_scale_bytes(16, 4096) == 1 * 8 * 256
    assert L.moe_mxfp4_tiled_scale_bytes(1536, 1536) == 96 * 3 * 256
    assert L.moe_mxfp4_tiled_scale_bytes(8, 256) == 0 and L.moe_mxfp4_tiled_scale_bytes(16, 96) == 0
    t = L.moe_mxfp4_tile_weights
    assert t(FAKE, FAKE, 8, 256, FAKE, FAKE, None) == 1        # rows % 16
    assert t(FAKE, FAKE, 16, 96, FAKE, FAKE, None) == 1        # K % 128
    assert t(None, FAKE, 16, 256, FAKE, FAKE, None) == 1
    assert t(FAKE, FAKE, 16, 256, FAKE + 4, FAKE, None) == 4
    assert t(FAKE, FAKE, 0, 256, FAKE, FAKE, None) == 0


def test_create_rejects_k_without_a_pipeline():
    st, _ = _create(d_model=768)           # 6 steps: neither 2 nor a multiple of 4
    assert st == 2
    st, _ = _create(d_ff=768)
    assert st == 2
    st, h = _create(d_model=1024, d_ff=256)
    assert st == 0 and moe.lib().moe_mxfp4_destroy(h) == 0


def test_quantize_act_validation():
    q = moe.lib().moe_mxfp4_quantize_act_mxfp8
    assert q(FAKE, 4, 48, FAKE, FAKE, None) == 1
    assert q(None, 4, 64, FAKE, FAKE, None) == 1
    assert q(FAKE, -1, 64, FAKE, FAKE, None) == 1
    assert q(FAKE + 2, 4, 64, FAKE, FAKE, None) == 4
    assert q(FAKE, 0, 64, FAKE, FAKE, None) == 0


def test_dflash_binding_rejects_wrong_dtypes_before_the_library():
    torch = pytest.importorskip("torch")
    B, G, V = 2, 3, 8
    args = [torch.zeros((B, G), dtype=torch.int32), torch.zeros((B, G, V)), torch.zeros((B, G + 1, V)),
            torch.zeros((B, G)), torch.zeros(B)]
    with pytest.raises(ValueError):                  # CPU tensors
        moe.dflash_accept(*args)
    bad = list(args)
    bad[2] = torch.zeros((B, G + 2, V))
    with pytest.raises(ValueError):                  # inconsistent shapes
        moe.dflash_accept(*bad)
