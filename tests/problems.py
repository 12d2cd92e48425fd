"""Seeded problems for the parity tests: inputs from ``synth``, MXFP4 weights
packed by the CPU oracle's quantiser (so no oracle input ever comes from the
HIP path), cached per workload for the life of the test process."""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

THREADS = min(16, os.cpu_count() or 1)
WNAMES = ("w_gate", "w_gate_scale", "w_up", "w_up_scale", "w_down", "w_down_scale")


def pack_experts(w: synth.Workload, seed=None) -> dict:
    """All experts of ``w`` quantised by the oracle, stacked [E, ...]."""
    out = {
        "w_gate": np.empty((w.E, w.f, w.d // 2), np.uint8),
        "w_gate_scale": np.empty((w.E, w.f, w.d // 32), np.uint8),
        "w_up": np.empty((w.E, w.f, w.d // 2), np.uint8),
        "w_up_scale": np.empty((w.E, w.f, w.d // 32), np.uint8),
        "w_down": np.empty((w.E, w.d, w.f // 2), np.uint8),
        "w_down_scale": np.empty((w.E, w.d, w.f // 32), np.uint8),
    }

    def job(e):
        g, u, dn = synth.expert_weights_f32(w, e, seed)
        for name, m in (("w_gate", g), ("w_up", u), ("w_down", dn)):
            p, s = oracle.quant_mxfp4(m)
            out[name][e] = p
            out[name + "_scale"][e] = s

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(job, range(w.E)))
    return out


@functools.lru_cache(maxsize=2)
def problem(w: synth.Workload):
    """(activations dict, packed weights dict) for a workload, cached."""
    return synth.make_activations(w), pack_experts(w)


def to_device(weights: dict):
    """Row-major oracle-packed weights -> the library's tiled layout on the GPU
    (the conversion is the library's own moe_mxfp4_tile_weights)."""
    import torch
    import mxfp4_expert_ffn_amd as moe
    rm = {n: torch.from_numpy(np.ascontiguousarray(weights[n])).cuda() for n in WNAMES}
    tiled = moe.tile_expert_weights(rm)
    torch.cuda.synchronize()
    return tiled


def rel_max_err(y, ref) -> float:
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref))) / rms
