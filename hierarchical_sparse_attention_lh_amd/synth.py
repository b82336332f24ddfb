"""Seeded synthetic inputs for the Lighthouse layer (shared by the tests, the oracle side and
the benchmark).  It holds no arithmetic of the method itself: only the workload table and
the random draws.

Recipe (the pages name no value distribution; this is the stand-in for the per-token norm
spread that a norm scorer feeds on):
  * one scale per token, s = exp(0.5 * z) with z ~ N(0, 1) drawn in float64 (lognormal(0, 0.5)),
    shared by that token's Q, K and V rows across all heads;
  * Q, K, V = standard normal float32 [B, N, H, D] times s (a float32 product);
  * the upstream gradient dY = standard normal float32, unscaled;
  * bf16 workloads round every value float32 -> bf16 to nearest even.
Every draw comes from numpy's PCG64, one child stream per (tensor, batch, slab of 2048 tokens)
keyed as SeedSequence(entropy=seed, spawn_key=(tensor, batch, slab)); slabs are filled in
parallel threads, so the values do not depend on the thread count.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

SLAB = 2048
_T_SCALE, _T_Q, _T_K, _T_V, _T_DY = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """One layer workload: shapes, dtype, pyramid parameters and seed."""

    name: str
    batch: int
    n_tokens: int
    heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16" for Q, K, V, Y, dY, dQ, dK, dV
    levels: int
    pool: int
    k: int
    chunk: int
    seed: int
    backward: bool
    mode: str = "refine"  # selection reading: "refine" (the contract) or "direct"
    scorer: str = "k"  # score of a pooled entry: "k", "qk" or "qkv"


WORKLOADS = {
    "tiny-4k": Workload("tiny-4k", 1, 4096, 2, 64, "f32", 3, 4, 128, 64, 0, False),
    "medium-32k": Workload("medium-32k", 1, 32768, 8, 64, "bf16", 3, 4, 1024, 256, 1, True),
    "layer-98k": Workload("layer-98k", 1, 98304, 16, 64, "bf16", 4, 4, 2048, 512, 2, True),
    "lh-512k": Workload("lh-512k", 1, 524288, 16, 64, "bf16", 4, 4, 4096, 1024, 3, True),
    "stress-1m": Workload("stress-1m", 1, 1048576, 8, 128, "bf16", 4, 4, 4096, 1024, 4, True),
}


def _gen(seed: int, tensor: int, b: int, slab: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=(tensor, b, slab))))


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16 values (as uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def token_scales(seed: int, batch: int, n_tokens: int) -> np.ndarray:
    """The per-token lognormal(0, 0.5) scales [B, N] as float32."""
    out = np.empty((batch, n_tokens), np.float32)
    for b in range(batch):
        for s0 in range(0, n_tokens, SLAB):
            s1 = min(n_tokens, s0 + SLAB)
            z = _gen(seed, _T_SCALE, b, s0 // SLAB).standard_normal(s1 - s0)
            out[b, s0:s1] = np.exp(0.5 * z).astype(np.float32)
    return out


def _fill(out: np.ndarray, seed: int, tensor: int, scales, bf16: bool):
    batch, n_tokens, heads, dim = out.shape
    jobs = [(b, s0) for b in range(batch) for s0 in range(0, n_tokens, SLAB)]

    def work(job):
        b, s0 = job
        s1 = min(n_tokens, s0 + SLAB)
        x = _gen(seed, tensor, b, s0 // SLAB).standard_normal((s1 - s0, heads, dim), np.float32)
        if scales is not None:
            x *= scales[b, s0:s1, None, None]
        out[b, s0:s1] = bf16_round_f32(x) if bf16 else x

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, jobs))


def make_tensor(shape, seed: int, which: str, dtype: str) -> np.ndarray:
    """One input tensor ("q", "k", "v" or "dy") of shape [B, N, H, D] as float32 values."""
    tensor = {"q": _T_Q, "k": _T_K, "v": _T_V, "dy": _T_DY}[which]
    out = np.empty(shape, np.float32)
    scales = None if which == "dy" else token_scales(seed, shape[0], shape[1])
    _fill(out, seed, tensor, scales, dtype == "bf16")
    return out


def make_inputs(batch, n_tokens, heads, head_dim, seed, dtype="bf16", with_grad=True):
    """Q, K, V (and dY) as float32 arrays [B, N, H, D]; bf16-representable when dtype=bf16."""
    shape = (batch, n_tokens, heads, head_dim)
    out = {w: make_tensor(shape, seed, w, dtype) for w in ("q", "k", "v")}
    if with_grad:
        out["dy"] = make_tensor(shape, seed, "dy", dtype)
    return out


def workload_inputs(w: Workload, with_grad=None):
    """Inputs of a named workload."""
    g = w.backward if with_grad is None else with_grad
    return make_inputs(w.batch, w.n_tokens, w.heads, w.head_dim, w.seed, w.dtype, g)
