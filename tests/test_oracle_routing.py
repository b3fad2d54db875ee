"""Pins of the oracle's router: logits, top-k selection and routing weights.

Each check ties the oracle to something other than itself: brute force over
all k-subsets, hand-worked cases, closed forms, a library softmax, and
textbook invariants.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
import workloads


def _brute_topk(row, k):
    """All k-subsets in lexicographic order; the first with the largest sum wins;
    slots ordered by (value descending, id ascending).  Values are exact binary
    fractions so every sum is exact."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(row)), k):
        s = sum(float(row[i]) for i in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    return sorted(best, key=lambda i: (-float(row[i]), i))


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 7))
    k = int(rng.integers(1, E + 1))
    # small integers / 4: many exact ties, every partial sum is exact
    L = rng.integers(-3, 4, size=(6, E)).astype(np.float64) / 4.0
    ids = oracle.select_topk(L, k)
    for t in range(L.shape[0]):
        assert list(ids[t]) == _brute_topk(L[t], k)


def test_topk_hand_case_with_tie():
    # logits [1,3,3,2], k=2 -> experts 1 and 2 (tie at 3 goes to the lower id first)
    L = np.array([[1.0, 3.0, 3.0, 2.0]])
    ids = oracle.select_topk(L, 2)
    assert ids.tolist() == [[1, 2]]
    w = oracle.routing_weights(L, ids, renormalize=True)
    assert w.tolist() == [[0.5, 0.5]]


def test_topk_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    ids = oracle.select_topk(L, 1)
    assert ids[:, 0].tolist() == [0, 0]


def test_zero_input_routes_to_first_experts():
    cfg = workloads.config("tiny_fp32").scaled(num_tokens=5, hidden_size=16, num_experts=6, top_k=3,
                                               intermediate_size=8)
    inp = workloads.generate(cfg, seed=3)
    x0 = np.zeros_like(inp["x"])
    L = oracle.router_logits(x0, inp["router_weight"])
    ids = oracle.select_topk(L, 3)
    assert (ids == np.arange(3)[None, :]).all()
    assert np.allclose(oracle.routing_weights(L, ids, True), 1.0 / 3, rtol=0, atol=1e-15)
    assert np.allclose(oracle.routing_weights(L, ids, False), 1.0 / 6, rtol=0, atol=1e-15)


def test_duplicate_router_rows_tie_to_lower_id():
    rng = np.random.default_rng(0)
    H = 8
    x = rng.standard_normal((4, H)).astype(np.float32)
    wr = rng.standard_normal((5, H)).astype(np.float32)
    wr[3] = wr[1]  # experts 1 and 3 always tie exactly
    L = oracle.router_logits(x, wr)
    ids = oracle.select_topk(L, 5)
    for t in range(4):
        row = list(ids[t])
        assert row.index(1) < row.index(3)


def test_two_experts_top1_closed_form():
    # E=2, k=1, no renormalisation: weight = sigmoid(l_sel - l_other)
    L = np.array([[0.3, -1.1], [2.0, 2.5], [-0.25, -0.25]])
    ids = oracle.select_topk(L, 1)
    w = oracle.routing_weights(L, ids, renormalize=False)[:, 0]
    for t in range(3):
        sel = ids[t, 0]
        d = L[t, sel] - L[t, 1 - sel]
        assert w[t] == pytest.approx(1.0 / (1.0 + math.exp(-d)), rel=1e-15)
    assert ids[:, 0].tolist() == [0, 1, 0]


def test_top1_renormalised_weight_is_one():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((10, 7))
    ids = oracle.select_topk(L, 1)
    assert (oracle.routing_weights(L, ids, True) == 1.0).all()


def test_weights_against_library_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((20, 9)) * 3
    ids = oracle.select_topk(L, 4)
    ref = scipy.special.softmax(L, axis=1)
    assert np.allclose(oracle.routing_probs(L), ref, rtol=1e-14, atol=0)
    assert np.allclose(oracle.routing_weights(L, ids, False), np.take_along_axis(ref, ids.astype(np.int64), 1),
                       rtol=1e-14, atol=0)
    # renormalised weights are the softmax over the k selected logits alone
    sel_logits = np.take_along_axis(L, ids.astype(np.int64), 1)
    assert np.allclose(oracle.routing_weights(L, ids, True), scipy.special.softmax(sel_logits, axis=1),
                       rtol=1e-14, atol=0)


def test_weights_sum_and_order():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((64, 32))
    ids = oracle.select_topk(L, 8)
    w = oracle.routing_weights(L, ids, True)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=8 * 2.0 ** -52)
    # slots in descending weight order (softmax is monotone)
    assert (np.diff(w, axis=1) <= 0).all()
    # every chosen logit is >= every unchosen logit
    for t in range(64):
        chosen = set(ids[t].tolist())
        lo = min(L[t, e] for e in chosen)
        hi = max((L[t, e] for e in range(32) if e not in chosen), default=-np.inf)
        assert lo >= hi


def test_router_logits_pure_python():
    cfg = workloads.config("tiny_fp32").scaled(num_tokens=3, hidden_size=5, num_experts=4, top_k=2,
                                               intermediate_size=8, zipf_bias=True, zero_experts=1)
    inp = workloads.generate(cfg, seed=7)
    L = oracle.router_logits(inp["x"], inp["router_weight"], inp["router_bias"])
    for t in range(3):
        for e in range(4):
            acc = 0.0
            for h in range(5):
                acc += float(inp["x"][t, h]) * float(inp["router_weight"][e, h])
            acc += float(inp["router_bias"][e])
            assert L[t, e] == pytest.approx(acc, rel=1e-12, abs=1e-12)


def test_bias_forced_experts_never_selected():
    cfg = workloads.config("qwen3_30b_a3b_prefill_zipf").scaled(num_tokens=64, hidden_size=64)
    inp = workloads.generate(cfg, seed=0)
    L = oracle.router_logits(inp["x"], inp["router_weight"], inp["router_bias"])
    ids = oracle.select_topk(L, cfg.top_k)
    zero = np.nonzero(inp["router_bias"] < -1000)[0]
    assert len(zero) == 16
    assert not np.isin(ids, zero).any()
    w = oracle.routing_weights(L, ids, True)
    assert np.isfinite(w).all()


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x3C00, 0x7F7F], dtype=np.uint16)
    vals = oracle.widen(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert math.copysign(1.0, vals[3]) == -1.0
    assert vals[4] == 3.140625  # 0x4049 = 1.5703125 * 2
    assert vals[5] == 2.0 ** -7
    assert vals[6] == (2 - 2.0 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------- group-limited
def _brute_topk_grouped(row, k, n_group, topk_group):
    """Subset formulation: the kept groups are the topk_group-subset whose
    (-score, group) pairs, sorted, are lexicographically smallest (largest
    scores first, lower groups on ties); the experts are the k-subset of the
    kept groups' experts chosen the same way on (-logit, id)."""
    E = len(row)
    gs = E // n_group
    score = [max(float(row[e]) for e in range(g * gs, (g + 1) * gs)) for g in range(n_group)]
    best_s = min(itertools.combinations(range(n_group), topk_group),
                 key=lambda S: sorted((-score[g], g) for g in S))
    allowed = [e for e in range(E) if e // gs in best_s]
    best_e = min(itertools.combinations(allowed, k), key=lambda C: sorted((-float(row[e]), e) for e in C))
    return [e for _, e in sorted((-float(row[e]), e) for e in best_e)]


@pytest.mark.parametrize("seed", range(10))
def test_topk_grouped_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n_group = int(rng.choice([2, 3, 4]))
    gs = int(rng.integers(1, 4))
    E = n_group * gs
    tg = int(rng.integers(1, n_group + 1))
    k = int(rng.integers(1, tg * gs + 1))
    L = rng.integers(-3, 4, size=(5, E)).astype(np.float64) / 4.0  # many exact ties
    ids = oracle.select_topk_grouped(L, k, n_group, tg)
    for t in range(L.shape[0]):
        assert list(ids[t]) == _brute_topk_grouped(L[t], k, n_group, tg)


def test_topk_grouped_reduces_to_plain():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((40, 32))
    for k in (1, 4, 8):
        plain = oracle.select_topk(L, k)
        assert (oracle.select_topk_grouped(L, k, 1, 1) == plain).all()
        assert (oracle.select_topk_grouped(L, k, 8, 8) == plain).all()
        assert (oracle.select_topk_grouped(L, k, 4, 4) == plain).all()


def test_topk_grouped_hand_cases():
    # groups of 2: maxima 9, 2, 8.5, 8.4 -> keep groups 0 and 2 -> experts 0, 1, 4, 5;
    # the plain top-4 would take expert 6 (8.4) instead of expert 5 (0)
    L = np.array([[9, 8.9, 1, 2, 8.5, 0, 8.4, 0]], dtype=np.float64)
    assert list(oracle.select_topk_grouped(L, 4, 4, 2)[0]) == [0, 1, 4, 5]
    assert list(oracle.select_topk(L, 4)[0]) == [0, 1, 4, 6]
    # equal group scores (5 and 5): the lower group is kept
    L = np.array([[5, 0, 0, 5, 1, 1, 2, 2]], dtype=np.float64)
    assert list(oracle.select_topk_grouped(L, 2, 4, 1)[0]) == [0, 1]


def test_topk_grouped_invariants():
    rng = np.random.default_rng(11)
    T, E, ng, tg, k = 200, 128, 8, 4, 8
    L = rng.standard_normal((T, E))
    ids = oracle.select_topk_grouped(L, k, ng, tg)
    gs = E // ng
    score = L.reshape(T, ng, gs).max(axis=2)
    for t in range(T):
        groups = set(int(e) // gs for e in ids[t])
        top_groups = set(np.argsort(-score[t], kind="stable")[:tg].tolist())
        assert groups <= top_groups and len(set(ids[t].tolist())) == k
        allowed = [e for e in range(E) if e // gs in top_groups]
        rest = [e for e in allowed if e not in set(ids[t].tolist())]
        assert L[t, ids[t]].min() >= L[t, rest].max()
        assert (np.diff(L[t, ids[t]]) <= 0).all()


def test_topk_grouped_rejects_bad_shapes():
    L = np.zeros((2, 12))
    with pytest.raises(ValueError):
        oracle.select_topk_grouped(L, 2, 5, 2)   # 5 does not divide 12
    with pytest.raises(ValueError):
        oracle.select_topk_grouped(L, 7, 4, 2)   # only 2 * 3 experts kept
    with pytest.raises(ValueError):
        oracle.select_topk_grouped(L, 2, 4, 5)   # more kept groups than groups
