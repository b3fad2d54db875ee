"""Pins of the oracle's dispatch plan and of its expert-parallel split.

Pinned against: the printed vectors of the ep_dispatch.rs tests, a plan derived
by hand from the same inputs, brute-force nested loops, the invariants the
Dispatcher Module implies, and the zero-input special case.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _brute_plan(ids, weights, E):
    ids = np.asarray(ids)
    T, k = ids.shape
    perm = []
    for e in range(E):
        for a in range(T * k):
            if int(ids.flat[a]) == e:
                perm.append(a)
    inv = [0] * (T * k)
    for p, a in enumerate(perm):
        inv[a] = p
    counts = [sum(1 for a in range(T * k) if int(ids.flat[a]) == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return {
        "perm": perm, "inv": inv, "counts": counts, "offsets": offsets,
        "packed_ids": [a // k for a in perm],
        "packed_w": [float(np.asarray(weights).flat[a]) for a in perm],
    }


def check_plan_invariants(plan, ids, weights, E):
    ids = np.asarray(ids)
    T, k = ids.shape
    P = T * k
    counts, offsets = plan["counts"].astype(np.int64), plan["offsets"].astype(np.int64)
    perm, inv = plan["perm"].astype(np.int64), plan["inv"].astype(np.int64)
    assert counts.sum() == P
    assert offsets[0] == 0 and offsets[E] == P
    assert (np.diff(offsets) == counts).all()
    assert (perm[inv] == np.arange(P)).all()
    assert (inv[perm] == np.arange(P)).all()
    flat = ids.reshape(-1)
    for e in range(E):
        rng = perm[offsets[e]:offsets[e + 1]]
        assert (flat[rng] == e).all()
        assert (np.diff(rng) > 0).all()  # stable: assignment order kept inside an expert
    assert (plan["packed_ids"] == perm // k).all()
    assert (plan["packed_w"] == np.asarray(weights, dtype=np.float64).reshape(-1)[perm]).all()


def test_plan_from_ep_mixed_vectors():
    g = _load("dispatch_plan_ep_mixed.json")
    plan = oracle.dispatch_plan(np.array(g["ids"]), np.array(g["weights"]), g["num_experts"])
    ex = g["expect"]
    assert plan["perm"].tolist() == ex["perm"]
    assert plan["inv"].tolist() == ex["inv"]
    assert plan["packed_ids"].tolist() == ex["packed_ids"]
    assert plan["packed_w"].tolist() == ex["packed_w"]
    nz = {str(e): int(c) for e, c in enumerate(plan["counts"]) if c}
    assert nz == ex["nonzero_counts"]
    for e, v in ex["offsets_at"].items():
        assert plan["offsets"][int(e)] == v
    check_plan_invariants(plan, np.array(g["ids"]), np.array(g["weights"]), g["num_experts"])


def test_plan_range_agrees_with_ep_local_bucket():
    """The expert range [0, 256) of the plan holds the same tokens/weights as the
    local bucket printed by test_mixed_routing (same inputs, assignment order
    coincides with expert order there)."""
    g = _load("ep_dispatch_vectors.json")
    case = [c for c in g["cases"] if c["name"] == "mixed_routing"][0]
    ids = np.array(case["indices"]).reshape(case["num_tokens"], case["top_k"])
    w = np.array(case["weights"]).reshape(ids.shape)
    plan = oracle.dispatch_plan(ids, w, 512)
    lo, hi = plan["offsets"][case["start"]], plan["offsets"][case["end"]]
    assert plan["packed_ids"][lo:hi].tolist() == case["expect"]["local_token_indices"]
    assert np.allclose(plan["packed_w"][lo:hi], case["expect"]["local_weights"])
    rest = list(range(0, lo)) + list(range(hi, len(plan["perm"])))
    got = sorted(zip(plan["packed_ids"][rest].tolist(), ids.reshape(-1)[plan["perm"][rest]].tolist()))
    exp = sorted(zip(case["expect"]["remote_token_indices"], case["expect"]["remote_expert_ids"]))
    assert got == exp


@pytest.mark.parametrize("seed", range(8))
def test_plan_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    T = int(rng.integers(0, 9))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int64)
    w = rng.random((T, k))
    plan = oracle.dispatch_plan(ids, w, E)
    ref = _brute_plan(ids, w, E)
    for key in ("perm", "inv", "counts", "offsets", "packed_ids"):
        assert plan[key].tolist() == ref[key], key
    assert plan["packed_w"].tolist() == ref["packed_w"]
    check_plan_invariants(plan, ids, w, E)


def test_plan_invariants_large_skewed():
    rng = np.random.default_rng(11)
    E, T, k = 128, 4096, 8
    pop = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    ids = np.stack([rng.choice(E, size=k, replace=False, p=pop / pop.sum()) for _ in range(T)])
    w = rng.random((T, k))
    plan = oracle.dispatch_plan(ids, w, E)
    check_plan_invariants(plan, ids, w, E)
    assert plan["perm"].tolist() == np.argsort(ids.reshape(-1), kind="stable").tolist()


def test_zero_input_plan():
    # every token picks experts 0..k-1 in slot order: expert e holds a = e, k+e, 2k+e, ...
    T, k, E = 7, 3, 5
    ids = np.tile(np.arange(k), (T, 1))
    plan = oracle.dispatch_plan(ids, np.full((T, k), 1.0 / k), E)
    assert plan["counts"].tolist() == [T] * k + [0] * (E - k)
    for e in range(k):
        rng = plan["perm"][plan["offsets"][e]:plan["offsets"][e + 1]]
        assert rng.tolist() == [e + k * t for t in range(T)]


def test_empty_and_single():
    plan = oracle.dispatch_plan(np.zeros((0, 2), np.int32), np.zeros((0, 2)), 4)
    assert plan["offsets"].tolist() == [0, 0, 0, 0, 0]
    assert plan["perm"].size == 0
    plan = oracle.dispatch_plan(np.array([[3]]), np.array([[1.0]]), 4)
    assert plan["offsets"].tolist() == [0, 0, 0, 0, 1]
    assert plan["perm"].tolist() == [0] and plan["inv"].tolist() == [0]


def test_plan_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.dispatch_plan(np.array([[0, 4]]), np.ones((1, 2)), 4)


@pytest.mark.parametrize("case", _load("ep_dispatch_vectors.json")["cases"], ids=lambda c: c["name"])
def test_ep_routing_table_printed_vectors(case):
    t = oracle.ep_routing_table(case["indices"], case["weights"], case["num_tokens"], case["top_k"],
                                case["start"], case["end"])
    ex = case["expect"]
    nl, nr = len(t["local_token_indices"]), len(t["remote_token_indices"])
    if "local_count" in ex:
        assert nl == ex["local_count"]
    if "remote_count" in ex:
        assert nr == ex["remote_count"]
    if "total_count" in ex:
        assert nl + nr == ex["total_count"]
    for key in ("local_token_indices", "local_expert_ids", "remote_token_indices", "remote_expert_ids"):
        if key in ex:
            assert t[key].tolist() == ex[key], key
    for key in ("local_weights", "remote_weights"):
        if key in ex:
            assert t[key].tolist() == np.array(ex[key], dtype=np.float32).tolist(), key


@pytest.mark.parametrize("case", _load("ep_dispatch_vectors.json")["errors"], ids=lambda c: c["name"])
def test_ep_routing_table_length_errors(case):
    with pytest.raises(ValueError, match=case["message"]):
        oracle.ep_routing_table(case["indices"], case["weights"], case["num_tokens"], case["top_k"],
                                case["start"], case["end"])


# --------------------------------------------------------------------------
# expert-parallel send counts per rank
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", _load("ep_dispatch_vectors.json")["cases"], ids=lambda c: c["name"])
def test_ep_rank_counts_match_printed_vectors(case):
    """Two ranks over 512 experts ([0, 256) and [256, 512), the ranges the
    page's tests use): the send counts are the printed local/remote counts of
    rank 0 (rank 1 for the rank-1 perspective)."""
    c = oracle.ep_rank_counts(case["indices"], 512, 2)
    assert oracle.ep_rank_ranges(512, 2) == [(0, 256), (256, 512)]
    ex = case["expect"]
    mine = 0 if case["start"] == 0 else 1
    assert c["send_counts"][mine] == ex["local_count"]
    if "remote_count" in ex:
        assert c["send_counts"][1 - mine] == ex["remote_count"]
    assert c["send_offsets"].tolist() == [0, int(c["send_counts"][0]), len(case["indices"])]


@pytest.mark.parametrize("E,G", [(128, 8), (60, 8), (7, 3), (5, 5), (9, 1), (512, 7)])
def test_ep_rank_ranges_partition_the_experts(E, G):
    r = oracle.ep_rank_ranges(E, G)
    assert r[0][0] == 0 and r[-1][1] == E
    assert all(r[i][1] == r[i + 1][0] for i in range(G - 1))
    sizes = [hi - lo for lo, hi in r]
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1


@pytest.mark.parametrize("seed", range(4))
def test_ep_rank_counts_agree_with_plan_and_table(seed):
    """The counts are the plan's offsets at the rank boundaries and each
    rank's local bucket of the routing table (two independently pinned
    functions)."""
    rng = np.random.default_rng(seed)
    E, k, T = [(128, 8, 300), (60, 4, 16), (64, 2, 513), (16, 3, 1)][seed]
    G = [8, 8, 3, 16][seed]
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    c = oracle.ep_rank_counts(ids, E, min(G, E))
    plan = oracle.dispatch_plan(ids, np.ones_like(ids, dtype=np.float64), E)
    for r, (lo, hi) in enumerate(oracle.ep_rank_ranges(E, min(G, E))):
        assert c["send_offsets"][r] == plan["offsets"][lo]
        assert c["send_counts"][r] == plan["offsets"][hi] - plan["offsets"][lo]
        t = oracle.ep_routing_table(ids.reshape(-1), np.ones(T * k), T, k, lo, hi)
        assert c["send_counts"][r] == len(t["local_token_indices"])
    assert c["send_offsets"][-1] == T * k
