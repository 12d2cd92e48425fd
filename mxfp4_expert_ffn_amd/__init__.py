"""Python binding of libmoe_mxfp4 (the MXFP4 MoE expert FFN on MI355X).

Argument marshalling only: every step of the forward path runs in the HIP
kernels behind the C ABI in ``include/moe_mxfp4.h``.  PyTorch supplies device
memory and the current stream; nothing here computes any part of the method,
and there is no CPU fallback -- if the library is missing, loading fails.

Names follow the C ABI: ``MoeMxfp4`` wraps ``moe_mxfp4_create / _forward /
_destroy / _workspace_bytes / _debug_dequant``; ``quantize_weights`` wraps
``moe_mxfp4_quantize_weights``; ``dflash_accept`` wraps
``moe_mxfp4_dflash_accept`` (the rejection-sampling pass of a verify step).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SHAPE",
                3: "MOE_ERR_CAPACITY", 4: "MOE_ERR_ALIGNMENT", 5: "MOE_ERR_WORKSPACE",
                6: "MOE_ERR_HIP", 7: "MOE_ERR_INTERNAL"}
ACT_BF16, ACT_MXFP8_E4M3 = 0, 1
OUT_BF16, OUT_F32 = 0, 1

# Every symbol include/moe_mxfp4.h declares.
EXPORTS = ("moe_mxfp4_status_string", "moe_mxfp4_abi_version", "moe_mxfp4_create",
           "moe_mxfp4_destroy", "moe_mxfp4_workspace_bytes", "moe_mxfp4_forward",
           "moe_mxfp4_debug_dequant", "moe_mxfp4_quantize_weights", "moe_mxfp4_stage_timing",
           "moe_mxfp4_stage_times", "moe_mxfp4_tiled_scale_bytes", "moe_mxfp4_tile_weights",
           "moe_mxfp4_quantize_act_mxfp8", "moe_mxfp4_router_logits", "moe_mxfp4_forward_hidden",
           "moe_mxfp4_dflash_workspace_bytes", "moe_mxfp4_dflash_accept", "moe_mxfp4_probe",
           "moe_mxfp4_forward_noalloc", "moe_mxfp4_device_status", "moe_mxfp4_debug_hidden")
# Scratch bytes moe_mxfp4_forward_noalloc holds per GPU (MOE_MXFP4_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20
# Largest batch (tokens x top_k) the fused path runs (MOE_MXFP4_FUSED_MAX_PAIRS);
# larger ones take the per-phase launches.
FUSED_MAX_PAIRS = 8192
NUM_STAGES = 6
STAGES = ("route", "sort", "quant", "gateup", "down", "combine")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("num_experts", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("act_mode", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_gate_scale", "w_up", "w_up_scale",
                                               "w_down", "w_down_scale")]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_ids", "topk_w", "expert_offsets",
                                               "sorted_pairs")]


_lib = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -m mxfp4_expert_ffn_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_mxfp4_status_string.argtypes = [ctypes.c_int]
        L.moe_mxfp4_status_string.restype = ctypes.c_char_p
        L.moe_mxfp4_abi_version.argtypes = []
        L.moe_mxfp4_abi_version.restype = i32
        L.moe_mxfp4_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                                       ctypes.POINTER(P)]
        L.moe_mxfp4_create.restype = ctypes.c_int
        L.moe_mxfp4_destroy.argtypes = [P]
        L.moe_mxfp4_destroy.restype = ctypes.c_int
        L.moe_mxfp4_workspace_bytes.argtypes = [P, i32]
        L.moe_mxfp4_workspace_bytes.restype = sz
        L.moe_mxfp4_forward.argtypes = [P, P, P, i32, P, P, sz, P, ctypes.POINTER(Routing)]
        L.moe_mxfp4_forward.restype = ctypes.c_int
        L.moe_mxfp4_forward_noalloc.argtypes = [P, P, P, i32, P, P, ctypes.POINTER(Routing)]
        L.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
        L.moe_mxfp4_debug_hidden.argtypes = [P, P, i32, P, P, P]
        L.moe_mxfp4_debug_hidden.restype = ctypes.c_int
        L.moe_mxfp4_device_status.argtypes = [P, P, i32, ctypes.POINTER(i32), P]
        L.moe_mxfp4_device_status.restype = ctypes.c_int
        L.moe_mxfp4_forward_hidden.argtypes = [P, P, P, i32, P, P, sz, P, ctypes.POINTER(Routing)]
        L.moe_mxfp4_forward_hidden.restype = ctypes.c_int
        L.moe_mxfp4_router_logits.argtypes = [P, P, P, i32, P, P]
        L.moe_mxfp4_router_logits.restype = ctypes.c_int
        L.moe_mxfp4_debug_dequant.argtypes = [P, i32, i32, i32, i32, P, P]
        L.moe_mxfp4_debug_dequant.restype = ctypes.c_int
        L.moe_mxfp4_quantize_weights.argtypes = [P, i64, i64, P, P, P]
        L.moe_mxfp4_quantize_weights.restype = ctypes.c_int
        L.moe_mxfp4_quantize_act_mxfp8.argtypes = [P, i64, i64, P, P, P]
        L.moe_mxfp4_quantize_act_mxfp8.restype = ctypes.c_int
        L.moe_mxfp4_tiled_scale_bytes.argtypes = [i64, i64]
        L.moe_mxfp4_tiled_scale_bytes.restype = sz
        L.moe_mxfp4_tile_weights.argtypes = [P, P, i64, i64, P, P, P]
        L.moe_mxfp4_tile_weights.restype = ctypes.c_int
        L.moe_mxfp4_dflash_workspace_bytes.argtypes = [i32, i32]
        L.moe_mxfp4_dflash_workspace_bytes.restype = sz
        L.moe_mxfp4_dflash_accept.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
        L.moe_mxfp4_dflash_accept.restype = ctypes.c_int
        L.moe_mxfp4_probe.argtypes = [i32, P, sz, i32, P, ctypes.POINTER(ctypes.c_double), P]
        L.moe_mxfp4_probe.restype = ctypes.c_int
        L.moe_mxfp4_stage_timing.argtypes = [P, i32]
        L.moe_mxfp4_stage_timing.restype = ctypes.c_int
        L.moe_mxfp4_stage_times.argtypes = [P, ctypes.POINTER(ctypes.c_float),
                                            ctypes.POINTER(i32)]
        L.moe_mxfp4_stage_times.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_mxfp4_status_string(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, dtype, shape, name):
    """Argument check of the binding: a contiguous CUDA tensor of this dtype and shape."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous CUDA {dtype} tensor of shape {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _torch_stream(stream=None):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


ROUTING_FIELDS = ("topk_ids", "topk_w", "expert_offsets", "sorted_pairs")


def _routing_struct(routing, T, k, E):
    """Routing outputs (dict of optional CUDA tensors) -> the C struct, after
    checking each tensor's dtype, size and contiguity."""
    import torch
    if routing is None:
        return None
    unknown = set(routing) - set(ROUTING_FIELDS)
    if unknown:
        raise ValueError(f"routing: unknown outputs {sorted(unknown)}")
    want = {"topk_ids": (torch.int32, T * k), "topk_w": (torch.float32, T * k),
            "expert_offsets": (torch.int32, E + 1), "sorted_pairs": (torch.int32, T * k)}
    for n, t in routing.items():
        if t is None:
            continue
        dt, numel = want[n]
        if t.dtype != dt or t.numel() < numel or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"routing[{n!r}]: expected a contiguous CUDA {dt} tensor of at least {numel} "
                             f"elements, got {t.dtype} {tuple(t.shape)} on {t.device}")
    return Routing(*[_ptr(routing.get(n)) for n in ROUTING_FIELDS])


def make_config(num_experts, d_model, d_ff, top_k, max_tokens, act_mode=ACT_BF16,
                out_dtype=OUT_BF16, flags=0) -> Config:
    return Config(ctypes.sizeof(Config), num_experts, d_model, d_ff, top_k, max_tokens,
                  act_mode, out_dtype, flags)


class MoeMxfp4:
    """One expert layer: borrowed packed weights + configuration.

    ``weights``: dict of uint8 CUDA tensors in the TILED layout of the C
    header (``tile_expert_weights`` converts the row-major form): ``w_gate``,
    ``w_gate_scale``, ``w_up``, ``w_up_scale``, ``w_down``, ``w_down_scale``.
    References are kept for the life of this object.
    """

    def __init__(self, weights: dict, num_experts: int, d_model: int, d_ff: int, top_k: int,
                 max_tokens: int, act_mode: int = ACT_BF16, out_dtype: int = OUT_BF16):
        self.cfg = make_config(num_experts, d_model, d_ff, top_k, max_tokens, act_mode, out_dtype)
        self.weights = dict(weights)
        self.out_dtype = out_dtype
        w = Weights(*[_ptr(self.weights[n]) for n in ("w_gate", "w_gate_scale", "w_up",
                                                      "w_up_scale", "w_down", "w_down_scale")])
        h = ctypes.c_void_p()
        _check(lib().moe_mxfp4_create(ctypes.byref(self.cfg), ctypes.byref(w), ctypes.byref(h)),
               "moe_mxfp4_create")
        self._ctx = h
        self._ws = {}            # cached workspace per stream handle

    def close(self):
        if getattr(self, "_ctx", None) is not None and self._ctx.value:
            lib().moe_mxfp4_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, num_tokens: int) -> int:
        return lib().moe_mxfp4_workspace_bytes(self._ctx, num_tokens)

    def workspace(self, num_tokens: int, stream=None):
        """A cached uint8 workspace large enough for ``num_tokens``, one per
        stream (calls that may run at the same time need distinct
        workspaces).  It is allocated on that stream, so the caching
        allocator reuses its memory only after the stream's queued work."""
        import torch
        s = _torch_stream(stream)
        need = self.workspace_bytes(num_tokens)
        ws = self._ws.get(s.cuda_stream)
        if ws is None or ws.numel() < need:
            with torch.cuda.stream(s):
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
            self._ws[s.cuda_stream] = ws
        return ws

    def _out(self, out, T, device, stream):
        import torch
        dt = torch.bfloat16 if self.out_dtype == OUT_BF16 else torch.float32
        if out is None:
            with torch.cuda.stream(_torch_stream(stream)):
                return torch.empty((T, self.cfg.d_model), dtype=dt, device=device)
        _require(out, dt, (T, self.cfg.d_model), "out")
        return out

    def forward(self, hidden, logits, out=None, workspace=None, routing: dict | None = None,
                stream=None, w_router=None):
        """hidden: bf16 [T, d] CUDA; logits: float32 [T, E] CUDA -> out [T, d].

        With ``w_router`` (bf16 [E, d] CUDA) and ``logits=None`` the logits are
        projected from ``hidden`` inside the call (moe_mxfp4_forward_hidden).
        """
        import torch
        if (logits is None) == (w_router is None):
            raise ValueError("pass exactly one of logits and w_router")
        T = hidden.shape[0]
        E, d = self.cfg.num_experts, self.cfg.d_model
        _require(hidden, torch.bfloat16, (T, d), "hidden")
        if logits is not None:
            _require(logits, torch.float32, (T, E), "logits")
        else:
            _require(w_router, torch.bfloat16, (E, d), "w_router")
        out = self._out(out, T, hidden.device, stream)
        ws = self.workspace(T, stream) if workspace is None else workspace
        r = _routing_struct(routing, T, self.cfg.top_k, E)
        fn, name = ((lib().moe_mxfp4_forward, "moe_mxfp4_forward") if w_router is None else
                    (lib().moe_mxfp4_forward_hidden, "moe_mxfp4_forward_hidden"))
        st = fn(self._ctx, _ptr(hidden), _ptr(logits if w_router is None else w_router), T, _ptr(out),
                _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream),
                ctypes.byref(r) if r is not None else None)
        _check(st, name)
        return out

    __call__ = forward

    def forward_noalloc(self, hidden, logits, out, routing: dict | None = None, stream=None):
        """moe_mxfp4_forward_noalloc: as ``forward`` with the logits given,
        but on the library's own per-GPU scratch (no workspace, nothing
        allocated); ``out`` must be given.  Calls on one GPU share the
        scratch, so they must not overlap in time."""
        import torch
        T = hidden.shape[0]
        _require(hidden, torch.bfloat16, (T, self.cfg.d_model), "hidden")
        _require(logits, torch.float32, (T, self.cfg.num_experts), "logits")
        out = self._out(out, T, hidden.device, stream)
        r = _routing_struct(routing, T, self.cfg.top_k, self.cfg.num_experts)
        _check(lib().moe_mxfp4_forward_noalloc(self._ctx, _ptr(hidden), _ptr(logits), T, _ptr(out), _stream(stream),
                                               ctypes.byref(r) if r is not None else None),
               "moe_mxfp4_forward_noalloc")
        return out

    def device_status(self, num_tokens: int, workspace=None, stream=None) -> int:
        """The fused kernels' error word of the last call with ``num_tokens``
        tokens: on ``stream`` where the expert launch routes a verify block itself,
        else on ``workspace`` (default: this object's cached workspace for
        ``stream``); waits for the stream.  0 = no device-side wait gave up."""
        ws = self.workspace(num_tokens, stream) if workspace is None else workspace
        st = ctypes.c_int32()
        _check(lib().moe_mxfp4_device_status(self._ctx, _ptr(ws), num_tokens, ctypes.byref(st), _stream(stream)),
               "moe_mxfp4_device_status")
        return st.value

    def debug_hidden(self, num_tokens: int, workspace=None, stream=None):
        """h of the last call with ``num_tokens`` tokens on ``workspace``
        (default: the cached one), rows in expert-sorted order: MXFP8 mode
        (uint8 codes [P, d_ff], uint8 E8M0 scales [P, d_ff/32]); bf16 mode
        (bf16 [P, d_ff], None)."""
        import torch
        ws = self.workspace(num_tokens, stream) if workspace is None else workspace
        P, f = num_tokens * self.cfg.top_k, self.cfg.d_ff
        if self.cfg.act_mode == ACT_MXFP8_E4M3:
            h = torch.empty((P, f), dtype=torch.uint8, device="cuda")
            sc = torch.empty((P, f // 32), dtype=torch.uint8, device="cuda")
        else:
            h, sc = torch.empty((P, f), dtype=torch.bfloat16, device="cuda"), None
        _check(lib().moe_mxfp4_debug_hidden(self._ctx, _ptr(ws), num_tokens, _ptr(h), _ptr(sc), _stream(stream)),
               "moe_mxfp4_debug_hidden")
        return h, sc

    def router_logits(self, hidden, w_router, out=None, stream=None):
        """hidden: bf16 [T, d]; w_router: bf16 [E, d] -> float32 logits [T, E]."""
        import torch
        T = hidden.shape[0]
        _require(hidden, torch.bfloat16, (T, self.cfg.d_model), "hidden")
        _require(w_router, torch.bfloat16, (self.cfg.num_experts, self.cfg.d_model), "w_router")
        if out is None:
            out = torch.empty((T, self.cfg.num_experts), dtype=torch.float32, device=hidden.device)
        _check(lib().moe_mxfp4_router_logits(self._ctx, _ptr(hidden), _ptr(w_router), T, _ptr(out),
                                             _stream(stream)), "moe_mxfp4_router_logits")
        return out

    def stage_timing(self, capacity: int):
        """Record HIP events around each stage of the next forward calls."""
        _check(lib().moe_mxfp4_stage_timing(self._ctx, capacity), "moe_mxfp4_stage_timing")

    def stage_times(self):
        """(per-stage summed ms as a dict, number of calls) since the last read."""
        ms = (ctypes.c_float * NUM_STAGES)()
        n = ctypes.c_int32()
        _check(lib().moe_mxfp4_stage_times(self._ctx, ms, ctypes.byref(n)), "moe_mxfp4_stage_times")
        return dict(zip(STAGES, list(ms))), n.value

    def debug_dequant(self, expert: int, matrix: int, row0: int, nrows: int, out=None, stream=None):
        import torch
        K = self.cfg.d_ff if matrix == 2 else self.cfg.d_model
        if out is None:
            out = torch.empty((nrows, K), dtype=torch.float32, device="cuda")
        _check(lib().moe_mxfp4_debug_dequant(self._ctx, expert, matrix, row0, nrows, _ptr(out),
                                             _stream(stream)), "moe_mxfp4_debug_dequant")
        return out


def quantize_weights(w, packed=None, scales=None, stream=None):
    """float32 CUDA [rows, K] -> (packed uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    import torch
    rows, K = w.shape
    if packed is None:
        packed = torch.empty((rows, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=w.device)
    _check(lib().moe_mxfp4_quantize_weights(_ptr(w), rows, K, _ptr(packed), _ptr(scales),
                                            _stream(stream)), "moe_mxfp4_quantize_weights")
    return packed, scales


def tiled_scale_bytes(rows: int, K: int) -> int:
    return lib().moe_mxfp4_tiled_scale_bytes(rows, K)


def tile_weights(packed, scales, stream=None):
    """Row-major packed [rows, K/2] + scales [rows, K/32] (uint8 CUDA) -> tiled
    (packed uint8 [rows*K/2], scales uint8 [tiled_scale_bytes(rows, K)])."""
    import torch
    rows, K = packed.shape[0], packed.shape[1] * 2
    tp = torch.empty(rows * K // 2, dtype=torch.uint8, device=packed.device)
    ts = torch.empty(tiled_scale_bytes(rows, K), dtype=torch.uint8, device=packed.device)
    _check(lib().moe_mxfp4_tile_weights(_ptr(packed), _ptr(scales), rows, K, _ptr(tp), _ptr(ts),
                                        _stream(stream)), "moe_mxfp4_tile_weights")
    return tp, ts


def tile_expert_weights(rowmajor: dict, stream=None) -> dict:
    """Row-major expert weights (uint8 CUDA tensors shaped [E, N, K/2] and
    [E, N, K/32]) -> the tiled dict the forward path takes."""
    out = {}
    for name in ("w_gate", "w_up", "w_down"):
        p, sc = rowmajor[name], rowmajor[name + "_scale"]
        E, N, half = p.shape
        tp, ts = tile_weights(p.reshape(E * N, half), sc.reshape(E * N, sc.shape[2]), stream)
        out[name], out[name + "_scale"] = tp, ts
    return out


def quantize_act_mxfp8(x, codes=None, scales=None, stream=None):
    """bf16 CUDA [rows, K] -> (E4M3 codes uint8 [rows, K], E8M0 scales uint8 [rows, K/32])."""
    import torch
    rows, K = x.shape
    if codes is None:
        codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_mxfp4_quantize_act_mxfp8(_ptr(x), rows, K, _ptr(codes), _ptr(scales),
                                              _stream(stream)), "moe_mxfp4_quantize_act_mxfp8")
    return codes, scales


def dflash_workspace_bytes(batch: int, vocab: int) -> int:
    return lib().moe_mxfp4_dflash_workspace_bytes(batch, vocab)


def dflash_accept(draft, p_draft, p_target, u, r, n_accepted=None, next_token=None, workspace=None,
                  stream=None):
    """Rejection-sampling acceptance of drafted blocks (moe_mxfp4_dflash_accept).

    draft int32 [B, G], p_draft float32 [B, G, V], p_target float32 [B, G+1, V],
    u float32 [B, G], r float32 [B], all contiguous CUDA tensors ->
    (n_accepted int32 [B], next_token int32 [B]).
    """
    import torch
    B, G = draft.shape
    V = p_target.shape[2]
    if p_target.shape != (B, G + 1, V) or p_draft.shape != (B, G, V) or u.shape != (B, G) or r.shape != (B,):
        raise ValueError("dflash_accept: inconsistent shapes")
    want = ((draft, torch.int32), (p_draft, torch.float32), (p_target, torch.float32), (u, torch.float32),
            (r, torch.float32))
    for t, dt in want:
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("dflash_accept: draft must be int32 and the rest float32, all contiguous CUDA tensors")
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=p_target.device)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=p_target.device)
    if workspace is None:
        workspace = torch.empty(max(dflash_workspace_bytes(B, V), 256), dtype=torch.uint8,
                                device=p_target.device)
    _check(lib().moe_mxfp4_dflash_accept(B, G, V, _ptr(draft), _ptr(p_draft), _ptr(p_target), _ptr(u),
                                         _ptr(r), _ptr(n_accepted), _ptr(next_token), _ptr(workspace),
                                         workspace.numel(), _stream(stream)), "moe_mxfp4_dflash_accept")
    return n_accepted, next_token


PROBE_STREAM, PROBE_MFMA_BF16, PROBE_MFMA_FP8_FP4, PROBE_MFMA_FP4_FP4 = 0, 1, 2, 3
# the same instructions on random operands that change every MFMA
PROBE_MFMA_BF16_RANDOM, PROBE_MFMA_FP8_FP4_RANDOM, PROBE_MFMA_FP4_FP4_RANDOM = 4, 5, 6


def probe(kind: int, src=None, reps: int = 0, sink=None, stream=None) -> float:
    """Launch one measurement probe (moe_mxfp4_probe); returns the bytes or
    flops it does.  ``src``: a CUDA tensor to read (kind 0)."""
    import torch
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    work = ctypes.c_double()
    nbytes = 0 if src is None else src.numel() * src.element_size()
    _check(lib().moe_mxfp4_probe(kind, _ptr(src), nbytes, reps, _ptr(sink), ctypes.byref(work), _stream(stream)),
           "moe_mxfp4_probe")
    return work.value
