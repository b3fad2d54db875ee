"""Staged float64 NumPy oracle of the MoE layer forward (test infrastructure only).

Pages cited (by title and section):

* [DWDP] README of "DWDP-Triton-MoE-Inference-Engine": sections "How To Use",
  "Router Module", "Dispatcher Module", "Scheduler Module", "Executor Module",
  "Merger Module", "Runtime Integration Layer", "Hugging Face Adapter Layer".
* [diffulex] API reference "diffulex.moe": sections "diffulex.moe.topk",
  "diffulex.moe.layer".
* [refit] modelexpress test "test_reshard_refit_moe_experts.py": the module
  docstring and class ``FusedMoEModel`` (fused ``w13`` = gate rows then up rows;
  its expert loader takes the tensor-parallel rank's rows of each source).
* [ep_dispatch] metrale "ep_dispatch.rs": ``EpRoutingTable``,
  ``build_ep_routing_table`` and its tests.

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):

* the router weight is ``[E, H]`` (a linear layer), logits = x . Wr^T (+ bias);
* top-k is taken on the logits (softmax is monotone), ties go to the lower
  expert id, -0.0 equals +0.0, and slots are ordered by descending logit;
* renormalised weights are p[id_j] / sum_j p[id_j] with p = softmax(logits);
* the token permutation is a gather map ``perm[p] = a`` over the token-major
  flat assignment index ``a = t*k + j``, sorted stably by (expert, a), and
  ``inv[a] = p``; offsets have E+1 entries;
* an expert computes ``h = silu(gate) * up`` with ``silu(z) = z / (1 + e^-z)``,
  then ``y = W2 h``; routing weights are applied in the combine;
* the shared expert output is scaled by sigmoid(x . g) for a gate vector g [H];
* group-limited selection (diffulex "diffulex.moe.topk" names a router with
  group-limited expert selection and nothing more): the experts form n_group
  contiguous groups of E / n_group; a group's score is its largest logit; the
  topk_group best groups are kept (equal scores: the lower group), and the
  top-k is taken among their experts by the plain rule.  Weights follow the
  plain router's rule (softmax over all experts, renormalised over the k).
* tensor parallelism ([refit] slices only the gate/up sources): the down
  projection ``[H, I]`` is split along the same intermediate index, i.e. its
  columns, so that the ranks' layer outputs add up to the unsliced layer's;
  a shared expert is split the same way, router and gate are replicated.

Everything is float64; bf16 inputs are widened exactly and nothing is rounded
on the way.  This module imports NumPy only.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

__all__ = [
    "widen",
    "router_logits",
    "shared_gate_logit",
    "select_topk",
    "select_topk_grouped",
    "routing_probs",
    "routing_weights",
    "dispatch_plan",
    "w13_gate",
    "w13_up",
    "silu",
    "swiglu_expert",
    "expert_ffn",
    "combine",
    "shared_expert",
    "forward",
    "token_outputs",
    "ep_routing_table",
    "ep_rank_ranges",
    "ep_rank_counts",
    "tp_load_expert",
    "tp_slice",
]


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    """Decode a stored tensor to float64 exactly.

    ``uint16`` arrays are bf16 bit patterns: the 16 bits are the upper half of
    an IEEE binary32, so shifting them up by 16 gives the exact value.
    ``float32``/``float64`` arrays are converted (exactly).
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


# --------------------------------------------------------------------------
# router  ([DWDP] "Router Module"; [diffulex] "diffulex.moe.topk")
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, router_weight: np.ndarray,
                  router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits ``L[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e])`` in float64.

    [DWDP] "Router Module" lists router logits as the first router output.  The
    weight layout [E, H] (a linear layer from H to E) is the reading taken.  The
    optional bias is the per-expert bias of the skewed-routing workload; it is
    added before softmax, so it moves both the selection and the weights.
    """
    L = widen(x) @ widen(router_weight).T
    if router_bias is not None:
        L = L + widen(router_bias)[None, :]
    return L


def shared_gate_logit(x: np.ndarray, shared_gate: np.ndarray) -> np.ndarray:
    """Scalar gate logit of the shared expert, ``x[t] . g``  ([diffulex]
    "diffulex.moe.layer" names a shared expert MLP; the sigmoid gate on it is
    the Qwen1.5-MoE form the [DWDP] "Hugging Face Adapter Layer" targets)."""
    return widen(x) @ widen(shared_gate)


def select_topk(logits: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k expert ids per token, ``[T, k]`` int32.

    [DWDP] "Router Module" (top-k expert indices).  The k largest logits are
    chosen; slots are in descending logit order, equal values go to the lower
    expert id (a stable sort of the negated logits keeps index order among
    equal keys, and -0.0 compares equal to +0.0).
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k out of range")
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :top_k].astype(np.int32)


def select_topk_grouped(logits: np.ndarray, top_k: int, n_group: int, topk_group: int) -> np.ndarray:
    """Group-limited top-k expert ids per token, ``[T, k]`` int32.

    [diffulex] "diffulex.moe.topk" (a router with group-limited expert
    selection; the steps are the reading stated in the module docstring):
    group g holds experts [g*E/n_group, (g+1)*E/n_group); its score is the
    largest logit it holds; the topk_group highest-scoring groups are kept,
    equal scores going to the lower group; then the plain selection of
    ``select_topk`` runs over the kept groups' experts only.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if n_group < 1 or E % n_group != 0:
        raise ValueError("n_group must divide the number of experts")
    gs = E // n_group
    if not (1 <= topk_group <= n_group):
        raise ValueError("topk_group out of range")
    if not (1 <= top_k <= topk_group * gs):
        raise ValueError("top_k exceeds the experts of the kept groups")
    score = L.reshape(T, n_group, gs).max(axis=2)
    kept = np.argsort(-score, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, kept, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), L, -np.inf)
    order = np.argsort(-masked, axis=1, kind="stable")
    return order[:, :top_k].astype(np.int32)


def routing_probs(logits: np.ndarray) -> np.ndarray:
    """Softmax over all experts per token, float64 ([DWDP] "Router Module":
    routing probabilities)."""
    L = np.asarray(logits, dtype=np.float64)
    m = L.max(axis=1, keepdims=True)
    e = np.exp(L - m)
    return e / e.sum(axis=1, keepdims=True)


def routing_weights(logits: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Routing weights of the selected experts, ``[T, k]`` float64.

    [DWDP] "Router Module" (normalized routing weights): the softmax
    probabilities of the chosen experts, divided by their sum when
    ``renormalize`` is set, so that each token's weights sum to one.
    """
    p = routing_probs(logits)
    sel = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


# --------------------------------------------------------------------------
# dispatch plan  ([DWDP] "Dispatcher Module"; [ep_dispatch] flat index order)
# --------------------------------------------------------------------------
def dispatch_plan(ids: np.ndarray, weights: np.ndarray, num_experts: int) -> Dict[str, np.ndarray]:
    """Token-major assignments -> expert-major layout.

    [DWDP] "Dispatcher Module" names the outputs: expert-major grouping,
    per-expert counts, expert offsets, token permutation, inverse permutation,
    packed token indices and packed routing weights.  The assignments are read
    row-major from ``[T, k]`` (flat index ``a = t*k + j``, as
    ``build_ep_routing_table`` in [ep_dispatch] does), and kept in the order
    given within each expert (a stable sort by expert id).

    Returns int32 ``counts [E]``, ``offsets [E+1]`` (exclusive scan,
    ``offsets[E] = T*k``), ``perm [P]`` (``perm[p] = a``), ``inv [P]``
    (``inv[a] = p``), ``packed_ids [P]`` (``a // k``) and float64
    ``packed_w [P]``.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    P = flat.size
    perm = np.argsort(flat, kind="stable")
    inv = np.empty(P, dtype=np.int64)
    inv[perm] = np.arange(P)
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    packed_ids = perm // k
    packed_w = np.asarray(weights, dtype=np.float64).reshape(-1)[perm]
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "perm": perm.astype(np.int32),
        "inv": inv.astype(np.int32),
        "packed_ids": packed_ids.astype(np.int32),
        "packed_w": packed_w,
    }


# --------------------------------------------------------------------------
# experts  ([DWDP] "Executor Module"; [refit] FusedMoEModel w13 layout)
# --------------------------------------------------------------------------
def w13_gate(w13: np.ndarray, e: int) -> np.ndarray:
    """Gate (w1) rows of expert ``e`` in a fused ``w13 [E, 2I, H]`` buffer: the
    low half of the expert's slot ([refit] FusedMoEModel: member 0 is w1)."""
    I = w13.shape[1] // 2
    return w13[e, 0:I, :]


def w13_up(w13: np.ndarray, e: int) -> np.ndarray:
    """Up (w3) rows of expert ``e``: the high half of the slot ([refit]
    FusedMoEModel: member 1 is w3, placed after INTER_PER_TP gate rows)."""
    I = w13.shape[1] // 2
    return w13[e, I:2 * I, :]


def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z * sigmoid(z) = z / (1 + exp(-z))`` (standard SwiGLU
    activation; the pages name SwiGLU experts but print no formula).  For
    z below about -709, exp(-z) overflows to inf and the quotient is the
    exact limit 0; the overflow is expected, not reported."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU MLP on rows ``X [M, H]``: ``W_down (silu(W_gate x) * (W_up x))``.

    ``w_gate``/``w_up`` are ``[I, H]``, ``w_down`` is ``[H, I]``; all float64.
    """
    g = X @ w_gate.T
    u = X @ w_up.T
    return (silu(g) * u) @ w_down.T


def expert_ffn(x: np.ndarray, packed_ids: np.ndarray, offsets: np.ndarray,
               w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Grouped expert FFN over the expert-major layout, ``y [P, H]`` float64.

    [DWDP] "Executor Module": gather the token rows of each expert range, run
    the expert MLP, write packed expert outputs.  Expert ``e`` owns rows
    ``offsets[e]:offsets[e+1]`` of the packed layout; row ``p`` reads token
    ``packed_ids[p]``.  Routing weights are not applied here (see ``combine``).
    """
    X = widen(x)
    W13 = widen(w13)
    W2 = widen(w2)
    E = W13.shape[0]
    P = int(offsets[E])
    y = np.zeros((P, X.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue  # empty expert: its weights are never read
        rows = X[np.asarray(packed_ids[lo:hi], dtype=np.int64)]
        y[lo:hi] = swiglu_expert(rows, w13_gate(W13, e), w13_up(W13, e), W2[e])
    return y


def combine(y: np.ndarray, inv: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """Weighted combine back to token order, ``out [T, H]`` float64.

    [DWDP] "Merger Module": restore token-major assignment order, accumulate the
    top-k expert outputs, apply the routing weights.
    ``out[t] = sum_j w[t, j] * y[inv[t*k + j]]``, summed in ascending j.
    """
    w = np.asarray(weights, dtype=np.float64)
    T, k = w.shape
    rows = np.asarray(inv, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[rows[:, j]]
    return out


def shared_expert(x: np.ndarray, shared_w13: np.ndarray, shared_w2: np.ndarray,
                  gate_logit: np.ndarray) -> np.ndarray:
    """Shared expert term ``sigmoid(x.g) * SwiGLU_s(x)``, ``[T, H]`` float64.

    [diffulex] "diffulex.moe.layer" (SharedExpertMLP) with the Qwen1.5-MoE
    sigmoid gate; ``shared_w13 [2Is, H]`` is gate rows then up rows like an
    expert slot, ``shared_w2 [H, Is]``.
    """
    X = widen(x)
    W13 = widen(shared_w13)
    Is = W13.shape[0] // 2
    s = swiglu_expert(X, W13[:Is], W13[Is:], widen(shared_w2))
    sig = 1.0 / (1.0 + np.exp(-np.asarray(gate_logit, dtype=np.float64)))
    return sig[:, None] * s


# --------------------------------------------------------------------------
# the whole layer  ([DWDP] "Runtime Integration Layer": Router -> Dispatcher ->
# Scheduler -> Executor -> Merger; the comms planner has no single-GPU role)
# --------------------------------------------------------------------------
def forward(inputs: Dict[str, np.ndarray], top_k: int, renormalize: bool = True,
            ids: Optional[np.ndarray] = None, weights: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Full staged forward.  ``inputs`` holds the arrays of ``workloads.generate``.

    When ``ids``/``weights`` are given they replace the oracle's own routing, so
    that the expert and combine stages can be checked on a GPU routing result.
    """
    x = inputs["x"]
    E = inputs["router_weight"].shape[0]
    L = router_logits(x, inputs["router_weight"], inputs.get("router_bias"))
    if ids is None:
        ids = select_topk(L, top_k)
    if weights is None:
        weights = routing_weights(L, ids, renormalize)
    plan = dispatch_plan(ids, weights, E)
    y = expert_ffn(x, plan["packed_ids"], plan["offsets"], inputs["w13"], inputs["w2"])
    out = combine(y, plan["inv"], weights)
    res = {"logits": L, "ids": np.asarray(ids, dtype=np.int32), "weights": np.asarray(weights, dtype=np.float64),
           "y": y, "out": out, **plan}
    if "shared_w13" in inputs:
        gl = shared_gate_logit(x, inputs["shared_gate"])
        s = shared_expert(x, inputs["shared_w13"], inputs["shared_w2"], gl)
        res["shared_gate_logit"] = gl
        res["shared"] = s
        res["out"] = out + s
    return res


def token_outputs(inputs: Dict[str, np.ndarray], tokens: np.ndarray, ids: np.ndarray,
                  weights: np.ndarray) -> np.ndarray:
    """Layer output for a sample of tokens, float64.

    Uses the dispatch-free form ``out[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t])``
    (plus the gated shared expert), which needs only the chosen experts'
    weights, so it runs at full workload sizes.  ``ids``/``weights`` are the
    full ``[T, k]`` routing (for instance a GPU result); only the sampled rows
    are read.  Each touched expert is decoded once for all sampled tokens
    routed to it (a token picks an expert at most once).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    X = widen(inputs["x"][tokens])
    sel = np.asarray(ids)[tokens].astype(np.int64)
    wsel = np.asarray(weights, dtype=np.float64)[tokens]
    out = np.zeros_like(X)
    for e in np.unique(sel):
        rows, slots = np.nonzero(sel == e)
        W13e = widen(inputs["w13"][e])
        I = W13e.shape[0] // 2
        y = swiglu_expert(X[rows], W13e[:I], W13e[I:], widen(inputs["w2"][e]))
        out[rows] += wsel[rows, slots][:, None] * y
    if "shared_w13" in inputs:
        gl = shared_gate_logit(inputs["x"][tokens], inputs["shared_gate"])
        out += shared_expert(inputs["x"][tokens], inputs["shared_w13"], inputs["shared_w2"], gl)
    return out


# --------------------------------------------------------------------------
# expert-parallel local/remote split  ([ep_dispatch] build_ep_routing_table)
# --------------------------------------------------------------------------
def ep_routing_table(gate_indices, gate_weights, num_tokens: int, top_k: int,
                     local_expert_start: int, local_expert_end: int) -> Dict[str, np.ndarray]:
    """Split row-major ``[num_tokens, top_k]`` assignments into the experts of
    one rank (``start <= id < end``) and the rest, each bucket in assignment
    order, as ``build_ep_routing_table`` in [ep_dispatch] specifies.

    Raises ``ValueError`` with "gate_indices length mismatch" /
    "gate_weights length mismatch" when a length differs from
    ``num_tokens * top_k`` (the Rust function panics with those texts).
    """
    gi = np.asarray(gate_indices).reshape(-1)
    gw = np.asarray(gate_weights).reshape(-1)
    total = num_tokens * top_k
    if gi.size != total:
        raise ValueError("gate_indices length mismatch")
    if gw.size != total:
        raise ValueError("gate_weights length mismatch")
    a = np.arange(total)
    local = (gi >= local_expert_start) & (gi < local_expert_end)
    tok = a // max(top_k, 1)
    return {
        "local_token_indices": tok[local].astype(np.uint32),
        "local_expert_ids": gi[local].astype(np.uint32),
        "local_weights": gw[local].astype(np.float32),
        "remote_token_indices": tok[~local].astype(np.uint32),
        "remote_expert_ids": gi[~local].astype(np.uint32),
        "remote_weights": gw[~local].astype(np.float32),
    }



def ep_rank_ranges(num_experts: int, num_ranks: int):
    """Contiguous expert ranges of ``num_ranks`` expert-parallel ranks:
    rank r owns ``[floor(r*E/G), floor((r+1)*E/G))`` (reading: the pages give
    one rank's ``local_expert_start``/``local_expert_end`` [ep_dispatch] and
    no rule for choosing them; this split is contiguous, covers every expert
    once and differs by at most one expert between ranks)."""
    return [((r * num_experts) // num_ranks, ((r + 1) * num_experts) // num_ranks) for r in range(num_ranks)]


def ep_rank_counts(ids: np.ndarray, num_experts: int, num_ranks: int) -> Dict[str, np.ndarray]:
    """Per-rank send counts of the expert-major packed order: how many
    assignments go to each rank's experts (``ep_rank_ranges``), and where each
    rank's segment starts in the packed order (exclusive scan, G+1 entries).
    Counted directly from the assignments, one range at a time, as the local
    bucket of ``ep_routing_table`` with that rank's range would count them."""
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    counts = np.array([int(((ids >= lo) & (ids < hi)).sum()) for lo, hi in ep_rank_ranges(num_experts, num_ranks)],
                      dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return {"send_counts": counts.astype(np.int32), "send_offsets": offsets.astype(np.int32)}

# --------------------------------------------------------------------------
# tensor-parallel expert slices  ([refit] module docstring and
# FusedMoEModel._expert_loader)
# --------------------------------------------------------------------------
def tp_load_expert(w13: np.ndarray, w2: np.ndarray, expert: int, gate: np.ndarray, up: np.ndarray,
                   down: np.ndarray, tp_size: int, tp_rank: int) -> None:
    """Write rank ``tp_rank``'s slice of one expert into per-rank fused buffers.

    Sources are the expert's full per-expert matrices: ``gate``/``up``
    ``[I, H]`` (HF ``gate_proj``/``up_proj``) and ``down`` ``[H, I]``
    (``down_proj``).  With ``Ip = I / tp_size`` the rank owns intermediate
    indices ``tp_rank*Ip .. tp_rank*Ip + Ip - 1``.  [refit] ``_expert_loader``:
    the rank's rows of the source go to member half ``member*Ip`` of the
    destination slot, member 0 for gate (w1) and 1 for up (w3), so
    ``w13 [E, 2*Ip, H]``.  ``w2 [E, H, Ip]`` receives the same indices as
    columns of ``down`` (reading: the pages print no down-projection loader).
    Plain copies of stored values, any stored dtype.  Raises ``ValueError``
    when ``I`` is not a multiple of ``tp_size`` or a shape disagrees.
    """
    I, H = gate.shape
    if tp_size < 1 or not 0 <= tp_rank < tp_size or I % tp_size:
        raise ValueError("tp_size must divide the intermediate size and 0 <= tp_rank < tp_size")
    Ip = I // tp_size
    if up.shape != (I, H) or down.shape != (H, I) or w13.shape[1:] != (2 * Ip, H) or w2.shape[1:] != (H, Ip):
        raise ValueError("shape mismatch")
    rows = slice(tp_rank * Ip, tp_rank * Ip + Ip)
    for member, src in ((0, gate), (1, up)):
        w13[expert, member * Ip:member * Ip + Ip, :] = src[rows, :]
    w2[expert, :, :] = down[:, rows]


def tp_slice(inputs: Dict[str, np.ndarray], tp_size: int, tp_rank: int) -> Dict[str, np.ndarray]:
    """The layer inputs one tensor-parallel rank holds: every routed expert
    (and the shared expert, as one more slot) loaded by ``tp_load_expert``
    from its per-expert sources; tokens, router, bias and shared gate are
    replicated.  Summing ``forward(tp_slice(inputs, G, r))["out"]`` over
    ``r < G`` gives ``forward(inputs)["out"]`` up to rounding, since the
    expert MLP is a sum over intermediate indices and everything after it is
    linear."""
    res = dict(inputs)
    pairs = [("w13", "w2")]
    if "shared_w13" in inputs:
        pairs.append(("shared_w13", "shared_w2"))
    for k13, k2 in pairs:
        full13, full2 = inputs[k13], inputs[k2]
        stacked = full13.ndim == 2  # the shared expert: one slot, no expert axis
        f13 = full13[None] if stacked else full13
        f2 = full2[None] if stacked else full2
        E, twoI, H = f13.shape
        I = twoI // 2
        if I % tp_size:
            raise ValueError("tp_size must divide the intermediate size")
        Ip = I // tp_size
        d13 = np.zeros((E, 2 * Ip, H), dtype=f13.dtype)
        d2 = np.zeros((E, H, Ip), dtype=f2.dtype)
        for e in range(E):
            tp_load_expert(d13, d2, e, w13_gate(f13, e), w13_up(f13, e), f2[e], tp_size, tp_rank)
        res[k13] = d13[0] if stacked else d13
        res[k2] = d2[0] if stacked else d2
    return res
