"""Helpers shared by the GPU parity tests (not a test module)."""
import functools
import sys

import numpy as np
import torch

import workloads


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray) -> torch.Tensor:
    """Copy a generator array to the GPU: uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def device_inputs(inp):
    return {k: to_device(v) for k, v in inp.items()}


@functools.lru_cache(maxsize=4)
def full_inputs(name: str, seed: int = 0):
    """Full-size inputs of a named workload (cached for the session)."""
    cfg = workloads.config(name)
    return cfg, workloads.generate(cfg, seed=seed)


def gpu_forward(cfg, dev, renormalize=None, out_dtype=torch.float32):
    import route_dispatch_grouped_amd as rdg
    return rdg.moe_forward(dev["x"], dev["router_weight"], dev["w13"], dev["w2"], cfg.top_k,
                           router_bias=dev.get("router_bias"), shared_w13=dev.get("shared_w13"),
                           shared_w2=dev.get("shared_w2"), shared_gate=dev.get("shared_gate"),
                           renormalize=cfg.renormalize if renormalize is None else renormalize,
                           out_dtype=out_dtype, return_routing=True)


def logit_error_bound(inp, tokens=None):
    """Rigorous bound of an fp32 dot product of H terms, per (token, expert):
    |err| <= H * 2^-24 * sum_h |x_h w_h| (+ the bias rounding)."""
    import oracle
    x = oracle.widen(inp["x"] if tokens is None else inp["x"][tokens])
    w = oracle.widen(inp["router_weight"])
    H = x.shape[1]
    mag = np.abs(x) @ np.abs(w).T
    bound = (H + 2) * 2.0 ** -24 * mag
    if "router_bias" in inp:
        bound = bound + 2.0 ** -24 * np.abs(oracle.widen(inp["router_bias"]))[None, :]
    return bound + 1e-30


def near_tie_tokens(L_oracle, eps, k):
    """Tokens whose oracle top-(k+1) sorted logits have an adjacent gap <= 2*eps:
    there either selection is a correct result."""
    s = -np.sort(-L_oracle, axis=1)[:, :k + 1]
    gaps = s[:, :-1] - s[:, 1:]
    return np.nonzero((gaps <= 2 * eps).any(axis=1))[0]


def rel_max_err(got, ref):
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err, rms


def tol_for(cfg):
    return 1e-4 if cfg.dtype == "f32" else 2e-2
