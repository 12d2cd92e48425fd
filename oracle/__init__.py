"""CPU oracle of the MXFP4 MoE expert FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them.

This is a thin ctypes wrapper over ``moe_oracle.c`` (plain C, double
precision), which carries the definitions and their citations.  Parity status
of every function is listed in ``PINS`` below; each is checked by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py`` against something other
than the oracle itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Function -> what pins it (none is "parity unpinned").
PINS = {
    "orc_e2m1_value": "bit-field closed form over all 16 codes",
    "orc_e8m0_value": "torch float8_e8m0fnu decode over all 256 bytes",
    "orc_e4m3_value": "torch float8_e4m3fn decode over all 256 codes",
    "orc_e2m1_round": "independent threshold-table rounding; tie points and neighbours",
    "orc_e4m3_round": "torch float8_e4m3fn round-to-nearest-even below saturation",
    "orc_quant_mxfp4": "exact round trip of codebook x 2^e blocks; second quantiser",
    "orc_quant_mxfp8": "torch E4M3 rounding with the OCP scale rule; round trips",
    "orc_router_logits": "pure-Python brute force on small shapes; one-hot rows pick "
                         "weight entries; sign flip; split-support additivity",
    "orc_dflash_accept": "losslessness: Monte Carlo distribution of the first emitted token "
                         "against p_target (chi-square) and acceptance rate against "
                         "sum min(p_draft, p_target); identical distributions accept all; "
                         "one-hot targets; draws against an independent searchsorted",
    "orc_route": "brute-force sort on (-logit, index); forced ties; 1-ulp gaps",
    "orc_permute": "stable sort of pair ids by expert; invariants",
    "orc_moe_forward": "dense numpy evaluation over all experts; E=1 matmul "
                       "reduction; one-hot closed form; zero weights; equal logits",
}


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def bind(L):
    """Declare the C signatures on a loaded copy of the oracle library."""
    P = ctypes.c_void_p
    i32, i64, dbl, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_uint32
    L.orc_e2m1_value.argtypes = [u32]; L.orc_e2m1_value.restype = dbl
    L.orc_e8m0_value.argtypes = [u32]; L.orc_e8m0_value.restype = dbl
    L.orc_e4m3_value.argtypes = [u32]; L.orc_e4m3_value.restype = dbl
    L.orc_e2m1_round.argtypes = [dbl]; L.orc_e2m1_round.restype = u32
    L.orc_e4m3_round.argtypes = [dbl]; L.orc_e4m3_round.restype = u32
    for name in ("orc_dequant_mxfp4", "orc_dequant_mxfp8"):
        getattr(L, name).argtypes = [P, P, i64, i64, P]
        getattr(L, name).restype = None
    for name in ("orc_quant_mxfp4", "orc_quant_mxfp8"):
        getattr(L, name).argtypes = [P, i64, i64, P, P]
        getattr(L, name).restype = None
    L.orc_router_logits.argtypes = [P, P, i32, i32, i32, P, P]; L.orc_router_logits.restype = None
    L.orc_dflash_accept.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
    L.orc_dflash_accept.restype = None
    L.orc_route.argtypes = [P, i32, i32, i32, P, P]; L.orc_route.restype = None
    L.orc_permute.argtypes = [P, i32, i32, i32, P, P, P, P]; L.orc_permute.restype = None
    L.orc_moe_forward.argtypes = [i32] * 6 + [P] * 8 + [P, P, P, P, i32]
    L.orc_moe_forward.restype = i32
    return L


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


ACT_BF16, ACT_MXFP8 = 0, 1


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e8m0_value(byte: int) -> float:
    return lib().orc_e8m0_value(byte)


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(byte)


def e2m1_round(q: float) -> int:
    return lib().orc_e2m1_round(q)


def e4m3_round(q: float) -> int:
    return lib().orc_e4m3_round(q)


def quant_mxfp4(w: np.ndarray):
    """float32 [rows, K] -> (packed uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    w = _c(w, np.float32)
    rows, K = w.shape
    packed = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    lib().orc_quant_mxfp4(_p(w), rows, K, _p(packed), _p(scales))
    return packed, scales


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed, scales = _c(packed, np.uint8), _c(scales, np.uint8)
    rows, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    lib().orc_dequant_mxfp4(_p(packed), _p(scales), rows, K, _p(out))
    return out


def quant_mxfp8(v: np.ndarray):
    """float64 [rows, K] -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    v = _c(v, np.float64)
    rows, K = v.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    lib().orc_quant_mxfp8(_p(v), rows, K, _p(codes), _p(scales))
    return codes, scales


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, K = codes.shape
    out = np.empty((rows, K), np.float64)
    lib().orc_dequant_mxfp8(_p(codes), _p(scales), rows, K, _p(out))
    return out


def router_logits(x_bf16: np.ndarray, w_bf16: np.ndarray):
    """bf16 bits x [T, d], W [E, d] -> (logits float64 [T, E], absdot float64 [T, E])."""
    x_bf16, w_bf16 = _c(x_bf16, np.uint16), _c(w_bf16, np.uint16)
    T, d = x_bf16.shape
    E = w_bf16.shape[0]
    assert w_bf16.shape == (E, d)
    logits = np.empty((T, E), np.float64)
    absdot = np.empty((T, E), np.float64)
    lib().orc_router_logits(_p(x_bf16), _p(w_bf16), T, d, E, _p(logits), _p(absdot))
    return logits, absdot


def dflash_accept(draft, p_draft, p_target, u, r):
    """draft int32 [B, G], p_draft float32 [B, G, V], p_target float32 [B, G+1, V],
    u float32 [B, G], r float32 [B] -> (n_accepted int32 [B], next_token int32 [B])."""
    draft, u, r = _c(draft, np.int32), _c(u, np.float32), _c(r, np.float32)
    p_draft, p_target = _c(p_draft, np.float32), _c(p_target, np.float32)
    B, G = draft.shape
    V = p_draft.shape[2]
    assert p_draft.shape == (B, G, V) and p_target.shape == (B, G + 1, V)
    assert u.shape == (B, G) and r.shape == (B,)
    n_acc = np.empty(B, np.int32)
    tok = np.empty(B, np.int32)
    lib().orc_dflash_accept(B, G, V, _p(draft), _p(p_draft), _p(p_target), _p(u), _p(r), _p(n_acc), _p(tok))
    return n_acc, tok


def route(logits: np.ndarray, k: int):
    """float32 [T, E] -> (ids int32 [T, k], weights float64 [T, k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_route(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids: np.ndarray, E: int):
    """int32 [T, k] -> dict(counts [E], offsets [E+1], sorted_pairs [P], inverse [P])."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    P = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(P, np.int32)
    inv = np.empty(P, np.int32)
    lib().orc_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sp), _p(inv))
    return {"counts": counts, "offsets": offsets, "sorted_pairs": sp, "inverse": inv}


def moe_forward(x_bf16: np.ndarray, logits: np.ndarray, weights: dict, k: int,
                act_mode: int = ACT_BF16, want_h: bool = False, nthreads: int = 0):
    """Whole expert layer in double precision.

    ``weights`` holds uint8 arrays ``w_gate, w_gate_scale, w_up, w_up_scale,
    w_down, w_down_scale`` shaped [E, f, d/2], [E, f, d/32], ..., [E, d, f/2],
    [E, d, f/32].  Returns dict(y [T, d] float64, ids, w, h (optional), threads).
    """
    x_bf16 = _c(x_bf16, np.uint16)
    logits = _c(logits, np.float32)
    T, d = x_bf16.shape
    E = logits.shape[1]
    f = weights["w_gate"].shape[1]
    ws = [_c(weights[n], np.uint8) for n in
          ("w_gate", "w_gate_scale", "w_up", "w_up_scale", "w_down", "w_down_scale")]
    assert ws[0].shape == (E, f, d // 2) and ws[1].shape == (E, f, d // 32)
    assert ws[4].shape == (E, d, f // 2) and ws[5].shape == (E, d, f // 32)
    y = np.empty((T, d), np.float64)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    h = np.empty((T, k, f), np.float64) if want_h else None
    used = lib().orc_moe_forward(T, d, f, E, k, act_mode, _p(x_bf16), _p(logits),
                                 *[_p(a) for a in ws], _p(y), _p(ids), _p(w),
                                 _p(h) if h is not None else None, nthreads)
    if used < 0:
        raise ValueError("orc_moe_forward rejected its arguments")
    out = {"y": y, "ids": ids, "w": w, "threads": used}
    if want_h:
        out["h"] = h
    return out


def quantize_experts(gates, ups, downs):
    """Stack per-expert float32 matrices into the packed MXFP4 weight dict."""
    out = {n: [] for n in ("w_gate", "w_gate_scale", "w_up", "w_up_scale",
                           "w_down", "w_down_scale")}
    for g, u, dn in zip(gates, ups, downs):
        for name, m in (("w_gate", g), ("w_up", u), ("w_down", dn)):
            p, s = quant_mxfp4(m)
            out[name].append(p)
            out[name + "_scale"].append(s)
    return {n: np.stack(v) for n, v in out.items()}
