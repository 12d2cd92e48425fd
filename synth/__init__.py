"""Seeded synthetic inputs for the MXFP4 MoE expert FFN.

This module only draws random numbers: it holds none of the method's
arithmetic (no quantisation, routing, decode or FFN).  Both the CPU oracle
and the HIP path take their inputs from here, so it imports neither.

Recipe (one workload = one ``Workload`` below):

* x: T x d, N(0, 1) drawn in float32, then rounded to bfloat16 (round to
  nearest even on the float32 bits).  Returned as uint16 bf16 bit patterns.
* logits: T x E, N(0, 1) float32, plus a per-expert bias added in float32:
  "none" (0), "normal" (N(0, 0.5) per expert) or "zipf" (a log-Zipf tilt,
  ``-s * alpha * ln(rank)`` with s = 1.1, alpha = 0.34 and a random rank
  permutation, which gives the hottest expert about ten times the pairs of
  the median one at top-8 of 128).
* expert weights: for expert e, W_gate (f x d), W_up (f x d), W_down (d x f),
  N(0, 0.02) float32, drawn from a stream of their own per expert so that any
  subset of experts can be regenerated alone and in parallel.

* DFlash verify batches (``dflash_batch``): per sequence and position,
  target logits N(0, sigma^2) over the vocabulary (sigma = 4: about 4.8
  nats of entropy) and drafter logits = target logits + N(0, eps^2) (eps =
  0.15), each turned into a distribution by a float64 softmax rounded to
  float32; draft tokens are drawn from the drafter distributions, u and r
  are uniform float32 in [0, 1).  With these values the drafter's tokens
  are accepted about 95% of the time, 6.4 of a block of 8 on average -- the
  acceptance length the pages report for coding (6.30).

Streams: ``numpy.random.default_rng([seed, 0])`` for x then logits then bias;
``numpy.random.default_rng([seed, 1, e])`` for expert e's three matrices in
the order gate, up, down.  The default seed of a named workload is
1000 + its index.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_activations",
           "expert_weights_f32", "all_expert_weights_f32", "bf16_bits_from_f32",
           "bf16_bits_to_f32", "router_weights_bf16", "dflash_batch", "DFLASH_VOCAB"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (sequences x draft block of 8)
    d: int            # d_model
    f: int            # d_ff
    E: int            # experts
    k: int            # top-k
    act: str = "bf16"     # "bf16" or "mxfp8" (activations micro-scaled to E4M3)
    bias: str = "none"    # "none" | "normal" | "zipf"
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny case, one verify step (1 sequence x block 8),
# a batched verify step (32 sequences x 8), one GPU's expert share under a
# skewed load (64 sequences x 8) and a dense 8192-token chunk.
WORKLOADS = (
    Workload("tiny",            8,  256,  512,   4, 2, "bf16",  "none",   1000),
    Workload("verify_1seq",     8, 4096, 1536,  64, 8, "bf16",  "none",   1001),
    Workload("verify_32seq",  256, 4096, 1536,  64, 8, "bf16",  "normal", 1002),
    Workload("share_64seq",   512, 6144, 2048, 128, 8, "bf16",  "zipf",   1003),
    Workload("chunk_8192",   8192, 6144, 2048, 128, 8, "mxfp8", "none",   1004),
)


def workload(key) -> Workload:
    """Look a workload up by index or name."""
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _bias(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.bias == "none":
        return np.zeros(w.E, np.float32)
    if w.bias == "normal":
        return rng.normal(0.0, 0.5, size=w.E).astype(np.float32)
    if w.bias == "zipf":
        rank = rng.permutation(w.E).astype(np.float64) + 1.0
        return (-1.1 * 0.34 * np.log(rank)).astype(np.float32)
    raise ValueError(f"unknown bias kind {w.bias!r}")


def make_activations(w: Workload, seed: int | None = None) -> dict:
    """Hidden states and router logits of one verify batch.

    Returns ``{"x_bf16": uint16 [T, d], "x": float32 [T, d] (the same values),
    "logits": float32 [T, E], "bias": float32 [E]}``.
    """
    rng = np.random.default_rng([w.seed if seed is None else seed, 0])
    x32 = rng.standard_normal((w.T, w.d), dtype=np.float32)
    logits = rng.standard_normal((w.T, w.E), dtype=np.float32)
    bias = _bias(w, rng)
    logits = (logits + bias[None, :]).astype(np.float32)
    xb = bf16_bits_from_f32(x32)
    return {"x_bf16": xb, "x": bf16_bits_to_f32(xb), "logits": logits, "bias": bias}


def router_weights_bf16(w: Workload, seed: int | None = None) -> np.ndarray:
    """Router projection weights, bf16 bit patterns [E, d]: N(0, 0.02) rounded
    to bf16, so x W^T of the N(0, 1) hidden states has standard deviation
    0.02 * sqrt(d) (1.28 at d = 4096), the scale of the synthetic logits."""
    rng = np.random.default_rng([w.seed if seed is None else seed, 2])
    wr = rng.standard_normal((w.E, w.d), dtype=np.float32) * np.float32(0.02)
    return bf16_bits_from_f32(wr)


def expert_weights_f32(w: Workload, e: int, seed: int | None = None):
    """(W_gate [f, d], W_up [f, d], W_down [d, f]) of expert e, float32 N(0, 0.02)."""
    rng = np.random.default_rng([w.seed if seed is None else seed, 1, e])
    gate = rng.standard_normal((w.f, w.d), dtype=np.float32)
    up = rng.standard_normal((w.f, w.d), dtype=np.float32)
    down = rng.standard_normal((w.d, w.f), dtype=np.float32)
    for m in (gate, up, down):
        m *= np.float32(0.02)
    return gate, up, down


def all_expert_weights_f32(w: Workload, experts=None, seed: int | None = None,
                           threads: int | None = None):
    """Yield ``(e, gate, up, down)`` for the given experts (default: all), in order.

    Generation runs on a thread pool (numpy releases the GIL while filling),
    a few experts ahead of the consumer so that memory stays bounded.
    """
    experts = list(range(w.E)) if experts is None else list(experts)
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        pending = []
        it = iter(experts)
        for e in it:
            pending.append((e, ex.submit(expert_weights_f32, w, e, seed)))
            if len(pending) >= threads:
                break
        while pending:
            e, fut = pending.pop(0)
            nxt = next(it, None)
            if nxt is not None:
                pending.append((nxt, ex.submit(expert_weights_f32, w, nxt, seed)))
            yield (e, *fut.result())


# The pages give no vocabulary size; 152064 entries is the size class of
# current open LLM tokenisers (a multiple of 256).
DFLASH_VOCAB = 152064


def _softmax_f32(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=-1, keepdims=True)
    return z.astype(np.float32)


def dflash_batch(B: int, G: int, V: int, seed: int, sigma: float = 4.0, eps: float = 0.15) -> dict:
    """One verify step's inputs for the acceptance pass: ``draft`` int32 [B, G],
    ``p_draft`` float32 [B, G, V], ``p_target`` float32 [B, G+1, V], ``u``
    float32 [B, G], ``r`` float32 [B].  Stream ``default_rng([seed, 3])``."""
    rng = np.random.default_rng([seed, 3])
    zt = rng.standard_normal((B, G + 1, V)) * sigma
    zd = zt[:, :G] + rng.standard_normal((B, G, V)) * eps
    p_target = _softmax_f32(zt)
    del zt
    p_draft = _softmax_f32(zd)
    del zd
    # draft tokens: inverse CDF of the drafter distribution (float64 cumulative sums)
    c = np.cumsum(p_draft, axis=-1, dtype=np.float64)
    v = rng.random((B, G)) * c[..., -1]
    draft = np.empty((B, G), np.int32)
    for b in range(B):
        for j in range(G):
            draft[b, j] = min(int(np.searchsorted(c[b, j], v[b, j], side="right")), V - 1)
    del c
    u = rng.random((B, G), dtype=np.float32)
    r = rng.random(B, dtype=np.float32)
    return {"draft": draft, "p_draft": p_draft, "p_target": p_target, "u": u, "r": r}
