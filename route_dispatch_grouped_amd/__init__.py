"""MI355X-native single-GPU MoE layer forward: Python binding of the C ABI.

This module only marshals arguments: it checks tensor devices, dtypes, shapes
and contiguity, allocates outputs and workspaces with torch, and calls the
entry points of ``lib/libmoe_mi355x.so`` (declared in ``include/moe.h``) on
torch's current HIP stream.  Every step of the layer runs in the library's
HIP kernels; there is no Python or CPU fallback.  Importing works without a
GPU; the first call raises if the library is missing.

Entry points (same names as the C ABI):
  moe_router_topk, moe_router_topk_grouped, moe_dispatch_plan,
  moe_ep_routing_table, moe_ep_rank_counts, moe_grouped_ffn, moe_combine,
  moe_forward, moe_tp_load_expert
plus ``moe_tp_slice_experts`` (one tensor-parallel rank's fused weights,
loaded expert by expert through moe_tp_load_expert) and ``MoeLayer``, a bound layer with a reusable workspace (the "explicit
layer" of the DWDP README's ``build_reference``).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Dict, Optional

import torch

from .build import LIB_PATH

__all__ = [
    "LIB_PATH",
    "MOE_OK",
    "MOE_DTYPE_F32",
    "MOE_DTYPE_BF16",
    "MOE_DTYPE_BF16_KB32",
    "MoeError",
    "PackedWeights",
    "pack_weights",
    "load_library",
    "library_loaded",
    "moe_router_topk",
    "moe_router_topk_grouped",
    "moe_dispatch_plan",
    "moe_dispatch_plan_noalloc",
    "moe_ep_routing_table",
    "moe_ep_rank_counts",
    "moe_grouped_ffn",
    "moe_combine",
    "moe_forward",
    "moe_forward_workspace_size",
    "moe_tp_load_expert",
    "moe_tp_slice_experts",
    "MOE_PROJ_GATE",
    "MOE_PROJ_UP",
    "MOE_PROJ_DOWN",
    "MoeLayer",
    "profile_enable",
    "profile_collect",
]

MOE_OK = 0
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DTYPE_BF16_KB32 = 2
MOE_PROJ_GATE = 0
MOE_PROJ_UP = 1
MOE_PROJ_DOWN = 2

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t

_SIGNATURES = {
    "moe_abi_version": (_int, []),
    "moe_status_string": (ctypes.c_char_p, [_int]),
    "moe_last_error_message": (ctypes.c_char_p, []),
    "moe_router_topk": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _int, _int,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "moe_router_topk_grouped": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                                       _int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "moe_dispatch_workspace_size": (_size, [_i64, _i64, _i64]),
    "moe_dispatch_plan": (_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "moe_dispatch_noalloc_max_workspace": (_size, []),
    "moe_dispatch_plan_noalloc": (_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "moe_ep_routing_table_workspace_size": (_size, [_i64, _i64]),
    "moe_ep_routing_table": (_int, [_c_void_p, _i64, _c_void_p, _i64, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size,
                                    _c_void_p]),
    "moe_grouped_ffn_workspace_size": (_size, [_i64, _i64, _i64, _i64, _i64, _int]),
    "moe_grouped_ffn": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64,
                               _i64, _int, _int, _c_void_p, _c_void_p, _size, _c_void_p]),
    "moe_combine": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _int, _int,
                           _c_void_p, _c_void_p]),
    "moe_forward_workspace_size": (_size, [_i64, _i64, _i64, _i64, _i64, _i64, _int]),
    "moe_forward": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "moe_ep_rank_counts": (_int, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "moe_tp_load_expert": (_int, [_c_void_p, _int, _i64, _i64, _int, _int, _i64, _i64, _int, _c_void_p,
                                  _c_void_p]),
    "moe_packed_weights_size": (_size, [_i64, _i64, _i64]),
    "moe_pack_weights": (_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p]),
    "moe_profile_enable": (None, [_int]),
    "moe_profile_collect": (_int, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(_i64), _int]),
}

EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class MoeError(RuntimeError):
    """A library call returned a status other than MOE_OK."""

    def __init__(self, fn: str, status: int, text: str, message: str):
        super().__init__(f"{fn}: {text}: {message}")
        self.status = status
        self.text = text
        self.message = message


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the built HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is missing: build it with route_dispatch_grouped_amd.build.build()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def library_loaded() -> bool:
    return _lib is not None


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        lib = load_library()
        raise MoeError(fn, status, lib.moe_status_string(status).decode(), lib.moe_last_error_message().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t == torch.float32:
        return MOE_DTYPE_F32
    raise TypeError(f"unsupported dtype {t}; use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream=None):
    """Context in which outputs and workspaces are allocated: torch's current
    stream switched to ``stream``, the stream the library's kernels run on.
    torch's caching allocator hands a freed block only to later allocations on
    the stream it was allocated on, which run after those kernels; a block
    allocated on another stream could be reused while they still read or write
    it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _need(t: torch.Tensor, name: str, shape, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} length mismatch: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def moe_router_topk(hidden_states: torch.Tensor, router_weight: torch.Tensor, top_k: int,
                    router_bias: Optional[torch.Tensor] = None, shared_gate: Optional[torch.Tensor] = None,
                    renormalize: bool = True, return_probs: bool = False, stream=None) -> Dict[str, torch.Tensor]:
    """Router logits -> softmax -> top-k -> routing weights (include/moe.h: moe_router_topk).

    Returns ``logits [T,E] f32``, ``topk_ids [T,k] int32``, ``topk_weights [T,k] f32`` and
    optionally ``probs [T,E]`` and ``shared_gate_logit [T]``.
    """
    lib = load_library()
    T, H = hidden_states.shape
    E = router_weight.shape[0]
    dt = hidden_states.dtype
    _need(hidden_states, "hidden_states", (T, H), dt)
    _need(router_weight, "router_weight", (E, H), dt)
    if router_bias is not None:
        _need(router_bias, "router_bias", (E,), torch.float32)
    if shared_gate is not None:
        _need(shared_gate, "shared_gate", (H,), dt)
    dev = hidden_states.device
    with _on(stream):
        out = {
            "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
            "topk_ids": torch.empty((T, top_k), dtype=torch.int32, device=dev),
            "topk_weights": torch.empty((T, top_k), dtype=torch.float32, device=dev),
        }
        if return_probs:
            out["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
        if shared_gate is not None:
            out["shared_gate_logit"] = torch.empty((T,), dtype=torch.float32, device=dev)
    st = lib.moe_router_topk(_ptr(hidden_states), _ptr(router_weight), _ptr(router_bias), _ptr(shared_gate),
                             T, H, E, int(top_k), int(bool(renormalize)), _dtype_code(dt),
                             _ptr(out["logits"]), _ptr(out.get("probs")), _ptr(out["topk_ids"]),
                             _ptr(out["topk_weights"]), _ptr(out.get("shared_gate_logit")), _stream(stream))
    _check("moe_router_topk", st)
    return out


def moe_router_topk_grouped(hidden_states: torch.Tensor, router_weight: torch.Tensor, top_k: int, n_group: int,
                            topk_group: int, router_bias: Optional[torch.Tensor] = None, renormalize: bool = True,
                            return_probs: bool = False, stream=None) -> Dict[str, torch.Tensor]:
    """Router with group-limited expert selection (include/moe.h: moe_router_topk_grouped).

    Returns ``logits [T,E] f32``, ``topk_ids [T,k] int32``, ``topk_weights [T,k] f32`` and
    optionally ``probs [T,E]``.
    """
    lib = load_library()
    T, H = hidden_states.shape
    E = router_weight.shape[0]
    dt = hidden_states.dtype
    _need(hidden_states, "hidden_states", (T, H), dt)
    _need(router_weight, "router_weight", (E, H), dt)
    if router_bias is not None:
        _need(router_bias, "router_bias", (E,), torch.float32)
    dev = hidden_states.device
    with _on(stream):
        out = {
            "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
            "topk_ids": torch.empty((T, top_k), dtype=torch.int32, device=dev),
            "topk_weights": torch.empty((T, top_k), dtype=torch.float32, device=dev),
        }
        if return_probs:
            out["probs"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    st = lib.moe_router_topk_grouped(_ptr(hidden_states), _ptr(router_weight), _ptr(router_bias), T, H, E,
                                     int(top_k), int(n_group), int(topk_group), int(bool(renormalize)),
                                     _dtype_code(dt), _ptr(out["logits"]), _ptr(out.get("probs")),
                                     _ptr(out["topk_ids"]), _ptr(out["topk_weights"]), _stream(stream))
    _check("moe_router_topk_grouped", st)
    return out


def moe_dispatch_plan(topk_ids: torch.Tensor, topk_weights: Optional[torch.Tensor], num_experts: int,
                      stream=None) -> Dict[str, torch.Tensor]:
    """Token-major assignments -> expert-major plan (include/moe.h: moe_dispatch_plan).

    Returns int32 ``counts [E]``, ``offsets [E+1]``, ``perm [P]``, ``inv [P]``,
    ``packed_ids [P]`` and f32 ``packed_w [P]`` (when weights are given).
    """
    lib = load_library()
    T, k = topk_ids.shape
    _need(topk_ids, "topk_ids", (T, k), torch.int32)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", (T, k), torch.float32)
    with _on(stream):
        out = _plan_outputs(T * k, num_experts, topk_ids.device, topk_weights is not None)
        ws_bytes = lib.moe_dispatch_workspace_size(T, k, num_experts)
        ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=topk_ids.device)
    st = lib.moe_dispatch_plan(_ptr(topk_ids), _ptr(topk_weights), T, k, int(num_experts), _ptr(out["counts"]),
                               _ptr(out["offsets"]), _ptr(out["perm"]), _ptr(out["inv"]), _ptr(out["packed_ids"]),
                               _ptr(out.get("packed_w")), _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_dispatch_plan", st)
    return out


def _plan_outputs(P: int, num_experts: int, dev, with_weights: bool) -> Dict[str, torch.Tensor]:
    out = {
        "counts": torch.empty((num_experts,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((num_experts + 1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((P,), dtype=torch.int32, device=dev),
        "inv": torch.empty((P,), dtype=torch.int32, device=dev),
        "packed_ids": torch.empty((P,), dtype=torch.int32, device=dev),
    }
    if with_weights:
        out["packed_w"] = torch.empty((P,), dtype=torch.float32, device=dev)
    return out


def moe_dispatch_plan_noalloc(topk_ids: torch.Tensor, topk_weights: Optional[torch.Tensor], num_experts: int,
                              out: Dict[str, torch.Tensor], stream=None) -> Dict[str, torch.Tensor]:
    """The dispatch plan into caller-provided outputs, with the library's fixed
    scratch instead of a workspace (include/moe.h: moe_dispatch_plan_noalloc).

    ``out`` holds int32 ``counts [E]``, ``offsets [E+1]``, ``perm``, ``inv``,
    ``packed_ids`` ``[P]`` and, with weights, f32 ``packed_w [P]``; nothing is
    allocated here or in the library.  Calls that overlap in time on one GPU
    race on the shared scratch.
    """
    lib = load_library()
    T, k = topk_ids.shape
    P = T * k
    _need(topk_ids, "topk_ids", (T, k), torch.int32)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", (T, k), torch.float32)
        _need(out["packed_w"], "packed_w", (P,), torch.float32)
    _need(out["counts"], "counts", (num_experts,), torch.int32)
    _need(out["offsets"], "offsets", (num_experts + 1,), torch.int32)
    for name in ("perm", "inv", "packed_ids"):
        _need(out[name], name, (P,), torch.int32)
    st = lib.moe_dispatch_plan_noalloc(_ptr(topk_ids), _ptr(topk_weights), T, k, int(num_experts),
                                       _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["perm"]),
                                       _ptr(out["inv"]), _ptr(out["packed_ids"]),
                                       _ptr(out.get("packed_w") if topk_weights is not None else None),
                                       _stream(stream))
    _check("moe_dispatch_plan_noalloc", st)
    return out


def moe_ep_routing_table(gate_indices: torch.Tensor, gate_weights: torch.Tensor, num_tokens: int, top_k: int,
                         local_expert_start: int, local_expert_end: int, trim: bool = True, stream=None):
    """Local/remote split of the assignments (include/moe.h: moe_ep_routing_table).

    ``gate_indices`` int32 and ``gate_weights`` f32 device tensors are read as
    flat arrays; their lengths are passed through, so a length other than
    ``num_tokens * top_k`` raises ``MoeError`` with the page's message.  Returns
    a dict of the six buckets and ``counts [2]``; with ``trim`` the buckets are
    cut to their counts (this reads the counts back to the host).
    """
    lib = load_library()
    gi = gate_indices.reshape(-1)
    gw = gate_weights.reshape(-1)
    if gi.dtype != torch.int32 or gw.dtype != torch.float32 or not gi.is_cuda or not gw.is_cuda:
        raise TypeError("gate_indices must be an int32 and gate_weights a float32 device tensor")
    dev = gi.device
    P = max(int(num_tokens) * int(top_k), 0)
    with _on(stream):
        out = {name: torch.empty((P,), dtype=torch.float32 if name.endswith("weights") else torch.int32, device=dev)
               for name in ("local_token_indices", "local_expert_ids", "local_weights", "remote_token_indices",
                            "remote_expert_ids", "remote_weights")}
        out["counts"] = torch.empty((2,), dtype=torch.int32, device=dev)
        ws_bytes = lib.moe_ep_routing_table_workspace_size(int(num_tokens), int(top_k))
        ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=dev)
    st = lib.moe_ep_routing_table(_ptr(gi), gi.numel(), _ptr(gw), gw.numel(), int(num_tokens), int(top_k),
                                  int(local_expert_start), int(local_expert_end), _ptr(out["local_token_indices"]),
                                  _ptr(out["local_expert_ids"]), _ptr(out["local_weights"]),
                                  _ptr(out["remote_token_indices"]), _ptr(out["remote_expert_ids"]),
                                  _ptr(out["remote_weights"]), _ptr(out["counts"]), _ptr(ws), ws.numel(),
                                  _stream(stream))
    _check("moe_ep_routing_table", st)
    if trim:
        if stream is not None:
            stream.synchronize()
        nl, nr = (int(v) for v in out["counts"].cpu().tolist())
        for name in list(out):
            if name.startswith("local_"):
                out[name] = out[name][:nl]
            elif name.startswith("remote_"):
                out[name] = out[name][:nr]
    return out


def moe_ep_rank_counts(expert_offsets: torch.Tensor, num_ranks: int, stream=None) -> Dict[str, torch.Tensor]:
    """Rows of the expert-major packed order per expert-parallel rank with
    contiguous expert ranges (include/moe.h: moe_ep_rank_counts): send_counts
    [G] and send_offsets [G+1], int32 on the GPU."""
    _need(expert_offsets, "expert_offsets", None, torch.int32)
    if expert_offsets.dim() != 1 or expert_offsets.numel() < 2:
        raise ValueError("expert_offsets must be [E+1]")
    E = expert_offsets.numel() - 1
    with _on(stream):
        counts = torch.empty((max(int(num_ranks), 0),), dtype=torch.int32, device=expert_offsets.device)
        starts = torch.empty((max(int(num_ranks), 0) + 1,), dtype=torch.int32, device=expert_offsets.device)
    lib = load_library()
    _check("moe_ep_rank_counts", lib.moe_ep_rank_counts(_ptr(expert_offsets), E, int(num_ranks), _ptr(counts),
                                                        _ptr(starts), _stream(stream)))
    return {"send_counts": counts, "send_offsets": starts}


class PackedWeights:
    """Expert weights in the K-blocked layout of ``moe_pack_weights``: ``data``,
    a flat bf16 device tensor, and ``shape``, the (groups, rows, k) shape of the
    row-major weights it was packed from (``(rows, k)`` for the shared
    expert's)."""

    def __init__(self, data: torch.Tensor, shape):
        self.data = data
        self.shape = tuple(int(v) for v in shape)
        self.dtype = torch.bfloat16
        self.device = data.device


def pack_weights(w: torch.Tensor, stream=None) -> PackedWeights:
    """K-blocked copy of bf16 expert weights ``[groups, rows, k]`` or ``[rows, k]``
    (include/moe.h: moe_pack_weights), for layers called with packed weights."""
    lib = load_library()
    if w.dtype != torch.bfloat16:
        raise TypeError("only bf16 weights are packed")
    shape = tuple(w.shape)
    G, R, K = (1,) + shape if w.dim() == 2 else shape
    _need(w, "weights", shape, torch.bfloat16)
    with _on(stream):
        n = int(lib.moe_packed_weights_size(G, R, K))
        data = torch.empty((n // 2,), dtype=torch.bfloat16, device=w.device)
    _check("moe_pack_weights", lib.moe_pack_weights(_ptr(w), _ptr(data), G, R, K, _stream(stream)))
    return PackedWeights(data, shape)


def _weights(ws, names, shapes, dt):
    """Checks expert weights given all row-major (tensors of `shapes`) or all
    packed (PackedWeights of those shapes); returns (pointers, packed)."""
    given = [w for w in ws if w is not None]
    packed = [isinstance(w, PackedWeights) for w in given]
    if any(packed) and not all(packed):
        raise ValueError("expert weights must be all packed or all row-major")
    ptrs = []
    for w, name, shape in zip(ws, names, shapes):
        if w is None:
            ptrs.append(None)
        elif isinstance(w, PackedWeights):
            if w.shape != tuple(shape) or dt != torch.bfloat16:
                raise ValueError(f"{name}: packed weights of shape {w.shape}, expected {tuple(shape)} (bf16 layers)")
            ptrs.append(_ptr(w.data))
        else:
            _need(w, name, shape, dt)
            ptrs.append(_ptr(w))
    return ptrs, bool(given) and all(packed)


def moe_grouped_ffn(hidden_states: torch.Tensor, packed_token_indices: Optional[torch.Tensor],
                    expert_offsets: Optional[torch.Tensor], w13: torch.Tensor, w2: torch.Tensor, top_k: int,
                    out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """Grouped SwiGLU experts over the expert-major layout (include/moe.h: moe_grouped_ffn).

    Returns the packed expert outputs ``[T*top_k, H]`` in ``out_dtype`` (float32,
    or bfloat16 for a bf16 layer; routing weights not applied).
    """
    lib = load_library()
    T, H = hidden_states.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    dt = hidden_states.dtype
    P = T * top_k
    _need(hidden_states, "hidden_states", (T, H), dt)
    (p13, p2), packed = _weights([w13, w2], ["w13", "w2"], [(E, 2 * I, H), (E, H, I)], dt)
    code = MOE_DTYPE_BF16_KB32 if packed else _dtype_code(dt)
    if packed_token_indices is not None:
        _need(packed_token_indices, "packed_token_indices", (P,), torch.int32)
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", (E + 1,), torch.int32)
    dev = hidden_states.device
    with _on(stream):
        y = torch.empty((P, H), dtype=out_dtype, device=dev)
        ws_bytes = lib.moe_grouped_ffn_workspace_size(T, H, top_k, E, I, _dtype_code(dt))
        ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=dev)
    st = lib.moe_grouped_ffn(_ptr(hidden_states), _ptr(packed_token_indices), _ptr(expert_offsets), p13, p2,
                             T, H, E, int(top_k), I, code, _dtype_code(out_dtype), _ptr(y), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check("moe_grouped_ffn", st)
    return y


def moe_combine(packed_expert_outputs: torch.Tensor, inverse_permutation: torch.Tensor, topk_weights: torch.Tensor,
                shared_output: Optional[torch.Tensor] = None, shared_gate_logit: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """Weighted combine to token order (include/moe.h: moe_combine).

    ``packed_expert_outputs`` (and ``shared_output``) are float32 or bfloat16.
    """
    lib = load_library()
    T, k = topk_weights.shape
    H = packed_expert_outputs.shape[1]
    ydt = packed_expert_outputs.dtype
    _need(packed_expert_outputs, "packed_expert_outputs", (T * k, H), ydt)
    _need(inverse_permutation, "inverse_permutation", (T * k,), torch.int32)
    _need(topk_weights, "topk_weights", (T, k), torch.float32)
    if shared_output is not None:
        _need(shared_output, "shared_output", (T, H), ydt)
    if shared_gate_logit is not None:
        _need(shared_gate_logit, "shared_gate_logit", (T,), torch.float32)
    with _on(stream):
        out = torch.empty((T, H), dtype=out_dtype, device=packed_expert_outputs.device)
    st = lib.moe_combine(_ptr(packed_expert_outputs), _ptr(inverse_permutation), _ptr(topk_weights),
                         _ptr(shared_output), _ptr(shared_gate_logit), T, H, k, _dtype_code(ydt),
                         _dtype_code(out_dtype), _ptr(out), _stream(stream))
    _check("moe_combine", st)
    return out


def moe_tp_load_expert(src: torch.Tensor, proj: int, dst: torch.Tensor, tp_size: int, tp_rank: int, expert: int,
                       stream=None) -> None:
    """Copy rank ``tp_rank``'s slice of one expert projection into the rank's
    fused buffer (include/moe.h: moe_tp_load_expert).

    ``src``: the full per-expert matrix, ``[I, H]`` for MOE_PROJ_GATE /
    MOE_PROJ_UP, ``[H, I]`` for MOE_PROJ_DOWN; a GPU or CPU tensor.  ``dst``:
    ``w13 [E, 2*Ip, H]`` (gate/up) or ``w2 [E, H, Ip]`` (down) on the GPU,
    ``Ip = I / tp_size``.  A CPU source is waited for before returning, so the
    caller may free it at once.
    """
    if not isinstance(src, torch.Tensor) or not src.is_contiguous() or src.dim() != 2:
        raise ValueError("src must be a contiguous 2-D tensor")
    if src.device.type not in ("cuda", "cpu"):
        raise ValueError("src must be a GPU or CPU tensor")
    _need(dst, "dst", None, src.dtype)
    if dst.dim() != 3:
        raise ValueError("dst must be [E, 2*Ip, H] or [E, H, Ip]")
    if proj == MOE_PROJ_DOWN:
        H, I = src.shape
    else:
        I, H = src.shape
    if tp_size >= 1 and I % tp_size == 0:
        Ip = I // tp_size
        want = (dst.shape[0], H, Ip) if proj == MOE_PROJ_DOWN else (dst.shape[0], 2 * Ip, H)
        _need(dst, "dst", want, src.dtype)
    lib = load_library()
    _check("moe_tp_load_expert",
           lib.moe_tp_load_expert(_ptr(src), int(proj), H, I, int(tp_size), int(tp_rank), int(expert),
                                  dst.shape[0], _dtype_code(src.dtype), _ptr(dst), _stream(stream)))
    if src.device.type == "cpu":
        (stream if stream is not None else torch.cuda.current_stream()).synchronize()


def moe_tp_slice_experts(w13: torch.Tensor, w2: torch.Tensor, tp_size: int, tp_rank: int, stream=None):
    """One tensor-parallel rank's ``(w13 [E, 2*Ip, H], w2 [E, H, Ip])`` from the
    unsliced fused ``w13 [E, 2I, H]`` and ``w2 [E, H, I]`` (GPU or CPU): the
    gate rows, up rows and down columns of every expert are loaded by
    ``moe_tp_load_expert``.  A 2-D ``[2I, H]`` / ``[H, I]`` pair (a shared
    expert) gives a 2-D pair."""
    flat = w13.dim() == 2
    if flat:
        w13, w2 = w13.unsqueeze(0), w2.unsqueeze(0)
    if w13.dim() != 3 or w2.dim() != 3 or w13.shape[0] != w2.shape[0] or w13.shape[1] % 2:
        raise ValueError("w13 must be [E, 2I, H] and w2 [E, H, I]")
    E, twoI, H = w13.shape
    I = twoI // 2
    if tuple(w2.shape) != (E, H, I):
        raise ValueError(f"w2 length mismatch: expected shape {(E, H, I)}, got {tuple(w2.shape)}")
    if tp_size < 1 or I % tp_size:
        raise ValueError("tp_size must divide the intermediate size")
    Ip = I // tp_size
    d13 = torch.empty((E, 2 * Ip, H), dtype=w13.dtype, device="cuda")
    d2 = torch.empty((E, H, Ip), dtype=w2.dtype, device="cuda")
    for e in range(E):
        moe_tp_load_expert(w13[e, :I], MOE_PROJ_GATE, d13, tp_size, tp_rank, e, stream)
        moe_tp_load_expert(w13[e, I:], MOE_PROJ_UP, d13, tp_size, tp_rank, e, stream)
        moe_tp_load_expert(w2[e], MOE_PROJ_DOWN, d2, tp_size, tp_rank, e, stream)
    return (d13[0], d2[0]) if flat else (d13, d2)


def moe_forward_workspace_size(T: int, H: int, E: int, k: int, I: int, Is: int, dtype: torch.dtype) -> int:
    return int(load_library().moe_forward_workspace_size(T, H, E, k, I, Is, _dtype_code(dtype)))


def moe_forward(hidden_states: torch.Tensor, router_weight: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                top_k: int, router_bias: Optional[torch.Tensor] = None, shared_w13: Optional[torch.Tensor] = None,
                shared_w2: Optional[torch.Tensor] = None, shared_gate: Optional[torch.Tensor] = None,
                renormalize: bool = True, out_dtype: torch.dtype = torch.float32, return_routing: bool = False,
                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None):
    """Whole layer forward (include/moe.h: moe_forward).

    Returns ``out [T,H]``; with ``return_routing`` a dict with ``out``,
    ``topk_ids``, ``topk_weights`` and ``logits``.
    """
    lib = load_library()
    T, H = hidden_states.shape
    E = router_weight.shape[0]
    I = w13.shape[1] // 2
    dt = hidden_states.dtype
    _need(hidden_states, "hidden_states", (T, H), dt)
    _need(router_weight, "router_weight", (E, H), dt)
    if router_bias is not None:
        _need(router_bias, "router_bias", (E,), torch.float32)
    Is = 0
    if shared_w13 is not None:
        Is = shared_w13.shape[0] // 2
        _need(shared_gate, "shared_gate", (H,), dt)
    (p13, p2, ps13, ps2), packed = _weights(
        [w13, w2, shared_w13, shared_w2], ["w13", "w2", "shared_w13", "shared_w2"],
        [(E, 2 * I, H), (E, H, I), (2 * Is, H), (H, Is)], dt)
    code = MOE_DTYPE_BF16_KB32 if packed else _dtype_code(dt)
    dev = hidden_states.device
    with _on(stream):
        if out is None:
            out = torch.empty((T, H), dtype=out_dtype, device=dev)
        else:
            _need(out, "out", (T, H), out_dtype)
        ws_bytes = lib.moe_forward_workspace_size(T, H, E, top_k, I, Is, _dtype_code(dt))
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=dev)
        ids = wts = logits = None
        if return_routing:
            ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
            wts = torch.empty((T, top_k), dtype=torch.float32, device=dev)
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    st = lib.moe_forward(_ptr(hidden_states), _ptr(router_weight), _ptr(router_bias), p13, p2,
                         ps13, ps2, _ptr(shared_gate), T, H, E, int(top_k), I, Is,
                         int(bool(renormalize)), code, _dtype_code(out_dtype), _ptr(out), _ptr(ids),
                         _ptr(wts), _ptr(logits), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("moe_forward", st)
    if return_routing:
        return {"out": out, "topk_ids": ids, "topk_weights": wts, "logits": logits}
    return out


class MoeLayer:
    """One bound MoE layer with a reusable workspace and output buffer.

    Mirrors the explicit-layer binding of the DWDP README ("How To Use",
    ``build_reference(hidden_size, num_experts, top_k, experts)``): the expert
    weights are given as the fused ``w13 [E, 2I, H]`` and ``w2 [E, H, I]``.
    A bf16 layer keeps K-blocked copies of its expert weights
    (``pack_weights``, made here once; ``pack=False`` keeps the tensors as
    given).  ``forward`` allocates nothing once the layer has seen the largest
    token count it will be called with.
    """

    def __init__(self, router_weight, w13, w2, top_k, router_bias=None, shared_w13=None, shared_w2=None,
                 shared_gate=None, renormalize=True, out_dtype=torch.float32, pack=None):
        if pack is None:
            pack = isinstance(w13, torch.Tensor) and w13.dtype == torch.bfloat16
        if pack:
            w13, w2 = pack_weights(w13), pack_weights(w2)
            if shared_w13 is not None:
                shared_w13, shared_w2 = pack_weights(shared_w13), pack_weights(shared_w2)
        self.router_weight, self.w13, self.w2 = router_weight, w13, w2
        self.router_bias = router_bias
        self.shared_w13, self.shared_w2, self.shared_gate = shared_w13, shared_w2, shared_gate
        self.top_k = int(top_k)
        self.renormalize = renormalize
        self.out_dtype = out_dtype
        self.hidden_size = w13.shape[2]
        self.num_experts = w13.shape[0]
        self.intermediate_size = w13.shape[1] // 2
        self.shared_intermediate_size = 0 if shared_w13 is None else shared_w13.shape[0] // 2
        self._ws = None
        self._out = None
        self._last_stream = None

    def workspace_bytes(self, num_tokens: int) -> int:
        return moe_forward_workspace_size(num_tokens, self.hidden_size, self.num_experts, self.top_k,
                                          self.intermediate_size, self.shared_intermediate_size, self.w13.dtype)

    def reserve(self, num_tokens: int, device, stream=None) -> None:
        """Grow the workspace and output buffer to ``num_tokens`` tokens.  New
        buffers are allocated on ``stream``; a replaced buffer is released only
        after the work already enqueued on the stream of the layer's last
        forward (which may still use it)."""
        need = max(self.workspace_bytes(num_tokens), 256)
        grow_ws = self._ws is None or self._ws.numel() < need
        grow_out = self._out is None or self._out.shape[0] < num_tokens
        if not (grow_ws or grow_out):
            return
        for old, grow in ((self._ws, grow_ws), (self._out, grow_out)):
            if grow and old is not None and self._last_stream is not None:
                old.record_stream(self._last_stream)
        with _on(stream):
            if grow_ws:
                self._ws = torch.empty((need,), dtype=torch.uint8, device=device)
            if grow_out:
                self._out = torch.empty((num_tokens, self.hidden_size), dtype=self.out_dtype, device=device)

    def forward(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        """The layer's output ``[T, H]`` for ``x [T, H]``, enqueued on ``stream``
        (torch's current stream by default).  The result is a view of the
        layer's own output buffer, which the next call overwrites (clone it to
        keep it); the workspace is the layer's too, so calls of one layer that
        may overlap in time must be on one stream."""
        T = x.shape[0]
        self.reserve(T, x.device, stream)
        self._last_stream = stream if stream is not None else torch.cuda.current_stream()
        out = self._out[:T]
        return moe_forward(x, self.router_weight, self.w13, self.w2, self.top_k, self.router_bias, self.shared_w13,
                           self.shared_w2, self.shared_gate, self.renormalize, self.out_dtype,
                           workspace=self._ws, out=out, stream=stream)

    __call__ = forward


def profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (see moe_profile_enable)."""
    load_library().moe_profile_enable(1 if on else 0)


def profile_collect() -> Dict[str, tuple]:
    """Wait for recorded events; return {kernel name: (total ms, launches)} and clear."""
    lib = load_library()
    cap = 64
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (_i64 * cap)()
    n = lib.moe_profile_collect(names, ms, cnt, cap)
    return {names[i].decode(): (ms[i], int(cnt[i])) for i in range(min(n, cap))}
