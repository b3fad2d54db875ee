"""Seeded synthetic inputs for the MoE layer forward.

This module is shared by the oracle, the tests and the benchmark.  It holds
no arithmetic of the MoE method itself: it only draws random tensors, rounds
them once to the storage precision (bf16 round-to-nearest-even, or plain
fp32), and hands back NumPy arrays.  bf16 tensors are returned as their raw
``uint16`` bit patterns so that every consumer decodes the very same bits.

Recipe (every draw is reproducible from ``seed`` alone):

* every tensor chunk owns a child stream ``PCG64(SeedSequence([seed, tensor_id,
  chunk]))`` so chunks can be drawn on several threads without changing a bit;
* ``x`` ~ N(0, 1) in chunks of 256 rows, router weight, expert weights,
  shared-expert weights and the shared gate vector ~ N(0, 0.02) (standard
  deviation 0.02), ``w13``/``w2`` one chunk per expert;
* values are drawn as float32 standard normals times sigma, then rounded to the
  storage dtype;
* the skewed-routing workload adds a per-expert router bias: 16 experts
  (chosen without replacement) get -1e4 so that they never enter the top-k,
  the other experts get ``-1.2 * ln(r)`` for a random rank ``r`` in 1..E-16,
  i.e. Zipf(s=1.2) popularity at softmax temperature 1.

Shapes follow the Qwen-MoE models the pages name (Qwen1.5-MoE-A2.7B, Qwen3-30B-A3B)
and the explicit layer of the DWDP README ("How To Use": hidden 4096, 64 experts,
top-2); no checkpoint is read.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "MoeConfig",
    "CONFIGS",
    "config",
    "generate",
    "round_to_bf16_bits",
]

# Tensor ids of the child streams.  Changing them changes every input.
_TID_X = 1
_TID_ROUTER = 2
_TID_W13 = 3
_TID_W2 = 4
_TID_SHARED_W13 = 5
_TID_SHARED_W2 = 6
_TID_SHARED_GATE = 7
_TID_BIAS = 8

_X_ROWS_PER_CHUNK = 256


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    """One synthetic MoE layer workload."""

    name: str
    num_tokens: int
    hidden_size: int
    num_experts: int
    top_k: int
    intermediate_size: int
    dtype: str = "bf16"               # "bf16" or "f32": x and every weight
    shared_intermediate_size: int = 0  # 0: no shared expert
    renormalize: bool = True
    zipf_bias: bool = False            # skewed routing through a router bias
    zipf_s: float = 1.2
    zero_experts: int = 0              # experts forced to receive no token
    x_sigma: float = 1.0
    w_sigma: float = 0.02

    @property
    def num_assignments(self) -> int:
        return self.num_tokens * self.top_k

    def scaled(self, **kw) -> "MoeConfig":
        """Same workload recipe with some sizes replaced (for small test cases)."""
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoeConfig] = {
    c.name: c
    for c in [
        # tiny fp32 layer: 64 tokens, H=128, 8 experts, top-2, I=256
        MoeConfig("tiny_fp32", 64, 128, 8, 2, 256, dtype="f32"),
        # the explicit layer of the DWDP README: H=4096, 64 experts, top-2, I=2048
        MoeConfig("dwdp_h4096_e64", 4096, 4096, 64, 2, 2048),
        # Qwen1.5-MoE-A2.7B-shaped decode step with a sigmoid-gated shared expert
        MoeConfig("qwen15_moe_decode", 16, 2048, 60, 4, 1408,
                  shared_intermediate_size=5632),
        # Qwen3-30B-A3B-shaped prefill
        MoeConfig("qwen3_30b_a3b_prefill", 8192, 2048, 128, 8, 768),
        # the same shape with Zipf(1.2) expert popularity and 16 empty experts
        MoeConfig("qwen3_30b_a3b_prefill_zipf", 8192, 2048, 128, 8, 768,
                  zipf_bias=True, zero_experts=16),
    ]
}

# Order in which the workloads are usually listed.
CONFIG_ORDER = list(CONFIGS)


def config(name: str) -> MoeConfig:
    return CONFIGS[name]


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs are finite (normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _stream(seed: int, tid: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def _threads() -> int:
    n = os.environ.get("MOE_GEN_THREADS")
    if n:
        return max(1, int(n))
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _normal_tensor(seed: int, tid: int, shape, sigma: float, chunk_axis0: int,
                   dtype: str, pool: Optional[ThreadPoolExecutor]) -> np.ndarray:
    """Draw ``shape`` in chunks of ``chunk_axis0`` leading rows, one stream per chunk."""
    shape = tuple(int(s) for s in shape)
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty(shape, dtype=out_dtype)
    n0 = shape[0]
    chunks = [(c, lo, min(lo + chunk_axis0, n0)) for c, lo in enumerate(range(0, n0, chunk_axis0))]

    def work(item):
        c, lo, hi = item
        vals = _stream(seed, tid, c).standard_normal((hi - lo,) + shape[1:], dtype=np.float32)
        vals *= np.float32(sigma)
        if dtype == "bf16":
            out[lo:hi] = round_to_bf16_bits(vals)
        else:
            out[lo:hi] = vals

    if pool is None or len(chunks) == 1:
        for it in chunks:
            work(it)
    else:
        list(pool.map(work, chunks))
    return out


def zipf_bias(cfg: MoeConfig, seed: int) -> np.ndarray:
    """Per-expert router bias (float32) giving Zipf(s) popularity, with
    ``cfg.zero_experts`` experts pushed out of every top-k."""
    E = cfg.num_experts
    g = _stream(seed, _TID_BIAS, 0)
    zero = g.choice(E, size=cfg.zero_experts, replace=False)
    rest = np.setdiff1d(np.arange(E), zero)
    ranks = g.permutation(len(rest)) + 1
    bias = np.empty(E, dtype=np.float64)
    bias[zero] = -1.0e4
    bias[rest] = -cfg.zipf_s * np.log(ranks.astype(np.float64))
    return bias.astype(np.float32)


def generate(cfg: MoeConfig, seed: int = 0, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of one MoE layer forward.

    Returns a dict with ``x [T,H]``, ``router_weight [E,H]``, ``w13 [E,2I,H]``
    (gate rows then up rows), ``w2 [E,H,I]``, optional ``router_bias [E]`` (float32),
    and for a shared expert ``shared_w13 [2Is,H]``, ``shared_w2 [H,Is]``,
    ``shared_gate [H]``.  bf16 tensors are uint16 bit patterns; f32 tensors are float32.
    """
    T, H, E, I = cfg.num_tokens, cfg.hidden_size, cfg.num_experts, cfg.intermediate_size
    dt = cfg.dtype
    n = _threads() if threads is None else threads
    pool = ThreadPoolExecutor(n) if n > 1 else None
    try:
        out = {
            "x": _normal_tensor(seed, _TID_X, (T, H), cfg.x_sigma, _X_ROWS_PER_CHUNK, dt, pool),
            "router_weight": _normal_tensor(seed, _TID_ROUTER, (E, H), cfg.w_sigma, E, dt, pool),
            "w13": _normal_tensor(seed, _TID_W13, (E, 2 * I, H), cfg.w_sigma, 1, dt, pool),
            "w2": _normal_tensor(seed, _TID_W2, (E, H, I), cfg.w_sigma, 1, dt, pool),
        }
        Is = cfg.shared_intermediate_size
        if Is:
            out["shared_w13"] = _normal_tensor(seed, _TID_SHARED_W13, (2 * Is, H), cfg.w_sigma, 2 * Is, dt, pool)
            out["shared_w2"] = _normal_tensor(seed, _TID_SHARED_W2, (H, Is), cfg.w_sigma, H, dt, pool)
            out["shared_gate"] = _normal_tensor(seed, _TID_SHARED_GATE, (H,), cfg.w_sigma, H, dt, pool)
        if cfg.zipf_bias:
            out["router_bias"] = zipf_bias(cfg, seed)
    finally:
        if pool is not None:
            pool.shutdown()
    return out
