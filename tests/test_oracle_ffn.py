"""Pins of the oracle's expert FFN, combine, shared expert and whole forward.

Pinned against: the fused w13 byte offset of the modelexpress refit test, a
library SwiGLU MLP (torch CPU ops in float64), a dense routing-mask identity
that needs no dispatch plan, a scalar pure-Python loop, and special cases
(identical experts, zero down projection, zero gate, k=1 permutation, shared
expert with a zero gate vector).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(seed=0, **kw):
    base = dict(num_tokens=9, hidden_size=12, num_experts=5, top_k=2, intermediate_size=6)
    base.update(kw)
    cfg = workloads.config("tiny_fp32").scaled(**base)
    return cfg, workloads.generate(cfg, seed=seed)


def test_w13_layout_byte_offset():
    g = json.load(open(os.path.join(GOLDEN, "w13_layout.json")))
    H, I, E = g["hidden"], g["inter_per_tp"], g["local_experts"]
    w13 = np.zeros((E, 2 * I, H), dtype=np.float32)
    up = oracle.w13_up(w13, g["expert"])
    gate = oracle.w13_gate(w13, g["expert"])
    base = w13.__array_interface__["data"][0]
    assert up.__array_interface__["data"][0] - base == g["expected_byte_offset"]
    assert gate.__array_interface__["data"][0] - base == g["expected_byte_offset"] - I * H * g["elsize"]
    assert up.shape == (I, H) and gate.shape == (I, H)


def test_silu_against_library():
    z = np.linspace(-30, 30, 1001)
    ref = F.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(oracle.silu(z), ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_single_expert_is_textbook_swiglu():
    """E=1, k=1: the layer is a dense SwiGLU MLP (torch F.linear / F.silu, float64)."""
    cfg, inp = tiny(num_experts=1, top_k=1, num_tokens=7, hidden_size=10, intermediate_size=4, seed=5)
    res = oracle.forward(inp, cfg.top_k)
    w13 = torch.from_numpy(inp["w13"].astype(np.float64))[0]
    w2 = torch.from_numpy(inp["w2"].astype(np.float64))[0]
    x = torch.from_numpy(inp["x"].astype(np.float64))
    I = cfg.intermediate_size
    ref = F.linear(F.silu(F.linear(x, w13[:I])) * F.linear(x, w13[I:]), w2)
    assert np.allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-15)
    assert (res["weights"] == 1.0).all()


def _dense_reference(inp, ids, w):
    """out = sum_e G[:, e] * FFN_e(x), G[t, e] = w[t, j] if ids[t, j] == e.  No plan."""
    x = inp["x"].astype(np.float64)
    E = inp["w13"].shape[0]
    I = inp["w13"].shape[1] // 2
    T = x.shape[0]
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            G[t, ids[t, j]] += w[t, j]
    out = np.zeros_like(x)
    for e in range(E):
        W = inp["w13"][e].astype(np.float64)
        g = x @ W[:I].T
        u = x @ W[I:].T
        ffn = ((g / (1 + np.exp(-g))) * u) @ inp["w2"][e].astype(np.float64).T
        out += G[:, e:e + 1] * ffn
    return out


@pytest.mark.parametrize("seed", range(4))
def test_forward_matches_dense_mask_identity(seed):
    cfg, inp = tiny(seed=seed, num_tokens=16, num_experts=6, top_k=3)
    res = oracle.forward(inp, cfg.top_k)
    assert np.allclose(res["out"], _dense_reference(inp, res["ids"], res["weights"]), rtol=1e-12, atol=1e-14)


def test_scatter_form_equals_gather_form():
    cfg, inp = tiny(seed=1)
    res = oracle.forward(inp, cfg.top_k)
    out = np.zeros_like(res["out"])
    for p in range(len(res["perm"])):
        out[res["packed_ids"][p]] += res["packed_w"][p] * res["y"][p]
    assert np.allclose(out, res["out"], rtol=1e-13, atol=1e-15)


def test_token_outputs_matches_staged():
    cfg, inp = tiny(seed=2, num_tokens=11)
    res = oracle.forward(inp, cfg.top_k)
    toks = np.array([0, 3, 10])
    sample = oracle.token_outputs(inp, toks, res["ids"], res["weights"])
    assert np.allclose(sample, res["out"][toks], rtol=1e-13, atol=1e-15)


def test_identical_experts_give_plain_ffn():
    cfg, inp = tiny(seed=3)
    inp["w13"][:] = inp["w13"][0:1]
    inp["w2"][:] = inp["w2"][0:1]
    res = oracle.forward(inp, cfg.top_k)
    x = inp["x"].astype(np.float64)
    I = cfg.intermediate_size
    W = inp["w13"][0].astype(np.float64)
    ffn = oracle.silu(x @ W[:I].T) * (x @ W[I:].T) @ inp["w2"][0].astype(np.float64).T
    assert np.allclose(res["out"], ffn, rtol=1e-12, atol=1e-15)


def test_zero_down_projection_and_zero_gate():
    cfg, inp = tiny(seed=4)
    a = dict(inp)
    a["w2"] = np.zeros_like(inp["w2"])
    assert (oracle.forward(a, cfg.top_k)["out"] == 0).all()
    b = dict(inp)
    w13 = inp["w13"].copy()
    w13[:, :cfg.intermediate_size] = 0  # gate rows: silu(0) = 0
    b["w13"] = w13
    assert (oracle.forward(b, cfg.top_k)["out"] == 0).all()
    c = dict(inp)
    w13 = inp["w13"].copy()
    w13[:, cfg.intermediate_size:] = 0  # up rows
    c["w13"] = w13
    assert (oracle.forward(c, cfg.top_k)["out"] == 0).all()


def test_top1_unit_weight_combine_is_a_permutation():
    rng = np.random.default_rng(0)
    T, E, H = 13, 4, 6
    ids = rng.integers(0, E, size=(T, 1))
    plan = oracle.dispatch_plan(ids, np.ones((T, 1)), E)
    y = rng.standard_normal((T, H))
    out = oracle.combine(y, plan["inv"], np.ones((T, 1)))
    assert (out == y[plan["inv"]]).all()
    assert (out[plan["packed_ids"]] == y).all()


def test_scalar_loop_reference():
    """Pure-Python triple loop over a tiny layer, independent of NumPy matmul."""
    cfg, inp = tiny(seed=6, num_tokens=4, hidden_size=3, num_experts=3, top_k=2, intermediate_size=2)
    res = oracle.forward(inp, cfg.top_k)
    x, W13, W2 = inp["x"], inp["w13"], inp["w2"]
    H, I = 3, 2
    for t in range(4):
        for c in range(H):
            total = 0.0
            for j in range(2):
                e = int(res["ids"][t, j])
                acc = 0.0
                for i in range(I):
                    g = sum(float(x[t, h]) * float(W13[e, i, h]) for h in range(H))
                    u = sum(float(x[t, h]) * float(W13[e, I + i, h]) for h in range(H))
                    acc += float(W2[e, c, i]) * (g / (1.0 + math.exp(-g))) * u
                total += float(res["weights"][t, j]) * acc
            assert res["out"][t, c] == pytest.approx(total, rel=1e-10, abs=1e-14)


def test_shared_expert_special_cases():
    cfg = workloads.config("qwen15_moe_decode").scaled(num_tokens=5, hidden_size=16, num_experts=6,
                                                        top_k=2, intermediate_size=8, shared_intermediate_size=12)
    inp = workloads.generate(cfg, seed=1)
    # zero gate vector -> sigmoid(0) = 0.5 exactly; routed path off (w2 = 0)
    a = dict(inp)
    a["shared_gate"] = np.zeros_like(inp["shared_gate"])
    a["w2"] = np.zeros_like(inp["w2"])
    res = oracle.forward(a, cfg.top_k)
    x = oracle.widen(inp["x"])
    W = oracle.widen(inp["shared_w13"])
    Is = cfg.shared_intermediate_size
    s = oracle.silu(x @ W[:Is].T) * (x @ W[Is:].T) @ oracle.widen(inp["shared_w2"]).T
    assert np.allclose(res["out"], 0.5 * s, rtol=1e-12, atol=1e-15)
    # full: out = routed + sigmoid(x.g) * shared
    res = oracle.forward(inp, cfg.top_k)
    gl = x @ oracle.widen(inp["shared_gate"])
    routed = _dense_reference({k: oracle.widen(v) if v.dtype == np.uint16 else v for k, v in inp.items()},
                              res["ids"], res["weights"])
    ref = routed + (1 / (1 + np.exp(-gl)))[:, None] * s
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-14)
    sample = oracle.token_outputs(inp, np.array([1, 4]), res["ids"], res["weights"])
    assert np.allclose(sample, res["out"][[1, 4]], rtol=1e-12, atol=1e-14)


def test_shared_gate_sign_and_dot_product():
    """The shared expert's gate is sigmoid(+x.g): with x.g far above zero the
    term is the whole shared expert (out = routed + s), far below zero it
    vanishes (out = routed).  Two tokens are +v and -v and g = 8 sign(v), so
    x.g = +-8 sum|v| (about +-100): sigmoid(-x.g), a dropped gate, or a dot
    product with another row fails one of the two.  The gate logits equal the
    closed form 8 sum|v| exactly and torch's fp64 product on every token; the
    gate factor on every token equals torch.sigmoid of them."""
    cfg = workloads.config("qwen15_moe_decode").scaled(num_tokens=6, hidden_size=16, num_experts=6,
                                                        top_k=2, intermediate_size=8, shared_intermediate_size=12)
    inp = dict(workloads.generate(cfg, seed=3))
    v = oracle.widen(inp["x"][0])
    x = inp["x"].copy()
    x[1] = x[0] ^ np.uint16(0x8000)  # -v, exactly (bf16 sign bit)
    inp["x"] = x
    inp["shared_gate"] = workloads.round_to_bf16_bits((8.0 * np.sign(v)).astype(np.float32))
    res = oracle.forward(inp, cfg.top_k)
    X = oracle.widen(x)
    W = oracle.widen(inp["shared_w13"])
    Is = cfg.shared_intermediate_size
    s = (oracle.silu(X @ W[:Is].T) * (X @ W[Is:].T)) @ oracle.widen(inp["shared_w2"]).T
    routed = _dense_reference({k: oracle.widen(a) if a.dtype == np.uint16 else a for k, a in inp.items()},
                              res["ids"], res["weights"])
    gl = res["shared_gate_logit"]
    assert gl[0] == 8.0 * np.sum(np.abs(v)) and gl[1] == -gl[0] and gl[0] > 60.0
    assert np.allclose(res["out"][0], routed[0] + s[0], rtol=1e-12, atol=1e-14)
    assert np.allclose(res["out"][1], routed[1], rtol=1e-12, atol=1e-14)
    assert not np.allclose(res["out"][1], routed[1] + s[1], rtol=1e-6, atol=1e-9)
    # every token: the logit is torch's fp64 product, the factor torch.sigmoid
    Xt = torch.from_numpy(X)
    gt = torch.from_numpy(oracle.widen(inp["shared_gate"]))
    assert np.allclose(gl, (Xt @ gt).numpy(), rtol=1e-14, atol=1e-14)
    sig = torch.sigmoid(torch.from_numpy(gl)).numpy()
    assert np.allclose(res["out"] - routed, sig[:, None] * s, rtol=1e-10, atol=1e-14)
    assert np.allclose(res["shared"], sig[:, None] * s, rtol=1e-12, atol=1e-15)


def test_empty_experts_are_skipped():
    cfg, inp = tiny(seed=8, num_tokens=6, num_experts=8, top_k=1)
    ids = np.zeros((6, 1), np.int32)  # every token to expert 0
    w = np.ones((6, 1))
    plan = oracle.dispatch_plan(ids, w, 8)
    y = oracle.expert_ffn(inp["x"], plan["packed_ids"], plan["offsets"], inp["w13"], inp["w2"])
    x = inp["x"].astype(np.float64)
    ref = oracle.swiglu_expert(x, oracle.w13_gate(inp["w13"].astype(np.float64), 0),
                               oracle.w13_up(inp["w13"].astype(np.float64), 0), inp["w2"][0].astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-13)


# --------------------------------------------------------------------------
# tensor-parallel slices of the expert weights
# --------------------------------------------------------------------------
def test_tp_load_matches_page_bytes():
    """modelexpress refit test: at TP_SIZE=2, rank 0 pulls INTER_PER_TP*HIDDEN*4
    bytes from the start of expert 1's up_proj source into the w3 half of
    expert 1's slot, which begins at byte 192 of the fused fp32 w13."""
    g = json.load(open(os.path.join(GOLDEN, "w13_layout.json")))
    H, I, E, G, r = g["hidden"], g["inter"], g["local_experts"], g["tp_size"], g["tp_rank"]
    Ip = I // G
    assert Ip == g["inter_per_tp"]
    # distinct sources, marked so every element names where it came from
    src = {m: (np.arange(I * H, dtype=np.float32) + 1000 * (m + 1)).reshape(I, H) for m in range(3)}
    down = np.zeros((H, I), np.float32)
    w13 = np.zeros((E, 2 * Ip, H), np.float32)
    w2 = np.zeros((E, H, Ip), np.float32)
    oracle.tp_load_expert(w13, w2, g["expert"], src[0], src[1], down, G, r)
    flat = w13.reshape(-1)
    landed = np.nonzero(flat >= 2000)[0]  # the up source's values (member 1)
    assert landed.size * g["elsize"] == g["expected_pulled_bytes"]
    assert landed.min() * g["elsize"] == g["expected_byte_offset"]
    assert (np.diff(landed) == 1).all()
    src_idx = flat[landed].astype(np.int64) - 2000
    assert src_idx.min() * g["elsize"] == g["expected_src_min_byte"]
    # the gate source fills the w1 half just below, expert 0 is untouched
    gate_landed = np.nonzero((flat >= 1000) & (flat < 2000))[0]
    assert gate_landed.min() * g["elsize"] == g["expected_byte_offset"] - Ip * H * g["elsize"]
    assert not w13[0].any()
    # rank 1 reads the next INTER_PER_TP rows of every source
    oracle.tp_load_expert(w13, w2, 0, src[0], src[1], src[2].T.copy(), G, 1)
    assert (w13[0, :Ip] == src[0][Ip:]).all() and (w13[0, Ip:] == src[1][Ip:]).all()
    assert (w2[0] == src[2].T[:, Ip:]).all()


@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_tp_ranks_sum_to_full_layer(G):
    """The ranks' outputs add up to the unsliced layer (routed experts and the
    gated shared expert), since the MLP sums over intermediate indices; a
    slice that pairs the wrong gate/up/down indices breaks the sum."""
    cfg, inp = tiny(seed=3, num_tokens=11, hidden_size=16, num_experts=6, top_k=3, intermediate_size=12,
                    shared_intermediate_size=24)
    assert "shared_w13" in inp
    full = oracle.forward(inp, cfg.top_k)["out"]
    parts = [oracle.forward(oracle.tp_slice(inp, G, r), cfg.top_k) for r in range(G)]
    total = sum(p["out"] for p in parts)
    assert np.max(np.abs(total - full)) <= 1e-12 * np.max(np.abs(full))
    # every rank routes identically (router replicated)
    for p in parts:
        assert (p["ids"] == parts[0]["ids"]).all()
    if G == 1:
        s = oracle.tp_slice(inp, 1, 0)
        for key in ("w13", "w2", "shared_w13", "shared_w2"):
            assert (s[key] == inp[key]).all()


def test_tp_rank_slices_partition_the_weights():
    """Every stored value of the full layer lands in exactly one rank, once."""
    cfg, inp = tiny(seed=4, intermediate_size=8)
    G = 4
    s = [oracle.tp_slice(inp, G, r) for r in range(G)]
    I = cfg.intermediate_size
    Ip = I // G
    gate = np.concatenate([x["w13"][:, :Ip] for x in s], axis=1)
    up = np.concatenate([x["w13"][:, Ip:] for x in s], axis=1)
    assert (gate == inp["w13"][:, :I]).all() and (up == inp["w13"][:, I:]).all()
    assert (np.concatenate([x["w2"] for x in s], axis=2) == inp["w2"]).all()


def test_tp_load_rejects_bad_shapes():
    w13 = np.zeros((2, 4, 3), np.float32)
    w2 = np.zeros((2, 3, 2), np.float32)
    src = np.zeros((4, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.tp_load_expert(w13, w2, 0, src, src, np.zeros((3, 4), np.float32), 3, 0)  # 4 % 3
    with pytest.raises(ValueError):
        oracle.tp_load_expert(w13, w2, 0, src, src, np.zeros((3, 4), np.float32), 2, 2)  # rank >= size
    with pytest.raises(ValueError):
        oracle.tp_load_expert(w13, w2, 0, src, src, np.zeros((4, 3), np.float32), 2, 0)  # down transposed
