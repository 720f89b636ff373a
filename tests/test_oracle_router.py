"""Pins of the oracle's routing: sqrtsoftplus closed forms, brute-force top-k,
special cases and the hash route as a table lookup (CPU)."""
import itertools
import math

import numpy as np
import pytest

import oracle


def check_sqrtsoftplus_closed_forms():
    s = oracle.sqrtsoftplus
    assert s(0.0) == pytest.approx(0.8325546111576977, rel=1e-15)       # sqrt(ln 2)
    assert s(100.0) == pytest.approx(10.0, rel=1e-15)
    assert s(-100.0) == pytest.approx(math.exp(-50.0), rel=1e-12)
    assert s(1000.0) == pytest.approx(math.sqrt(1000.0), rel=1e-15)     # naive softplus overflows in fp32
    x = np.random.default_rng(3).uniform(-30, 30, 1000)
    # softplus(x) - softplus(-x) = x
    assert np.allclose(s(x) ** 2 - s(-x) ** 2, x, rtol=1e-12, atol=1e-12)
    small = np.linspace(-20, 20, 401)
    assert np.allclose(s(small), np.sqrt(np.log(1.0 + np.exp(small))), rtol=1e-13)
    assert np.all(np.diff(s(small)) > 0)


def test_sqrtsoftplus_closed_forms():
    check_sqrtsoftplus_closed_forms()


def test_silu_special_values():
    z = np.random.default_rng(5).uniform(-20, 20, 100)
    assert oracle.silu(0.0) == 0.0
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert oracle.silu(-800.0) == 0.0 and oracle.silu(800.0) == 800.0


def _bruteforce_topk_set(key, k):
    """The unique k-subset S with key_i > key_j, or equal keys and i < j, for all i in S, j not in S."""
    E = len(key)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(key[i] > key[j] or (key[i] == key[j] and i < j) for i in S for j in rest):
            found.append(set(S))
    assert len(found) == 1
    return found[0]


def check_topk_bruteforce():
    rng = np.random.default_rng(11)
    for trial in range(60):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        logits = rng.standard_normal((1, E))
        bias = rng.standard_normal(E) * 0.1
        if trial % 3 == 0:                        # force exact ties in the key
            logits[0, :] = logits[0, 0]
            bias[:] = np.round(bias * 2) / 2
        ids, w, key, s = oracle.route_topk(logits, bias, k)
        assert set(ids[0].tolist()) == _bruteforce_topk_set(key[0], k)
        order = sorted(range(E), key=lambda e: (-key[0, e], e))[:k]
        assert ids[0].tolist() == order
        assert np.allclose(w[0], s[0, ids[0]] / s[0, ids[0]].sum(), rtol=1e-15)


def test_topk_bruteforce():
    check_topk_bruteforce()


def test_topk_zero_router_picks_lowest_indices():
    for E, k in [(16, 2), (256, 6), (7, 7)]:
        ids, w, _, _ = oracle.route_topk(np.zeros((3, E)), np.zeros(E), k)
        assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))
        assert np.allclose(w, 1.0 / k, rtol=1e-15)


def test_topk_k_equals_E_selects_all():
    rng = np.random.default_rng(2)
    ids, w, _, _ = oracle.route_topk(rng.standard_normal((4, 9)), rng.standard_normal(9), 9)
    for t in range(4):
        assert sorted(ids[t]) == list(range(9))
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)


def test_bias_ranks_but_does_not_weight():
    logits = np.zeros((1, 8))
    logits[0, 5] = 1.0
    bias = np.zeros(8)
    bias[2] = 10.0
    ids, w, _, s = oracle.route_topk(logits, bias, 2)
    assert ids[0].tolist() == [2, 5]
    assert w[0, 0] == pytest.approx(s[0, 2] / (s[0, 2] + s[0, 5]), rel=1e-15)
    assert w[0, 0] < w[0, 1]


def test_pruned_router_equals_survivor_masked_router():
    """REAP-pruned layers (alphaneural card "DeepSeek-V4-Flash-MLX-4bit",
    section "REAP-pruned builds": the router renormalizes over survivors)
    keep only the survivors' router rows. Routing over those rows, mapped
    back through the survivor list, equals routing over all experts with the
    dropped ones masked out (bias -inf): same ids in the same order, same
    weights."""
    rng = np.random.default_rng(31)
    E, k, T = 256, 6, 50
    survivors = np.sort(rng.choice(E, 192, replace=False))      # REAP25 keeps 192
    logits = rng.standard_normal((T, E))
    bias = rng.standard_normal(E) * 0.1
    ids_p, w_p, _, _ = oracle.route_topk(logits[:, survivors], bias[survivors], k)
    masked = np.full(E, -np.inf)
    masked[survivors] = bias[survivors]
    ids_m, w_m, _, _ = oracle.route_topk(logits, masked, k)
    assert np.array_equal(survivors[ids_p], ids_m)
    assert np.allclose(w_p, w_m, rtol=1e-15)
    assert np.allclose(w_p.sum(1), 1.0, rtol=1e-14)


def test_router_logits_loop():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 40))
    wr = rng.standard_normal((5, 40)).astype(np.float32)
    l = oracle.router_logits(x, wr)
    for t in range(3):
        for e in range(5):
            assert l[t, e] == pytest.approx(sum(x[t, i] * float(wr[e, i]) for i in range(40)), rel=1e-12, abs=1e-12)


def check_hash_route_lookup():
    rng = np.random.default_rng(4)
    E, d, vocab, k, T = 12, 32, 50, 3, 20
    tid2eid = rng.integers(0, E, size=(vocab, k)).astype(np.int32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    x = rng.standard_normal((T, d))
    tok = rng.integers(0, vocab, T).astype(np.int32)
    ids, w, _ = oracle.route_hash(x, wr, tid2eid, tok)
    assert np.array_equal(ids, tid2eid[tok])
    for t in range(T):
        sc = [math.sqrt(math.log1p(math.exp(float(np.dot(x[t], wr[e].astype(np.float64)))))) for e in ids[t]]
        assert np.allclose(w[t], np.array(sc) / sum(sc), rtol=1e-12)
    # ids do not depend on the activations
    ids2, _, _ = oracle.route_hash(x[::-1].copy(), wr, tid2eid, tok)
    assert np.array_equal(ids2, ids)


def test_hash_route_is_table_lookup():
    check_hash_route_lookup()


def test_hash_route_duplicates_are_separate_slots():
    E, d = 4, 8
    wr = np.ones((E, d), np.float32)
    tid2eid = np.array([[1, 1, 3]], np.int32)
    ids, w, _ = oracle.route_hash(np.ones((1, d)) * 0.1, wr, tid2eid, np.array([0], np.int32))
    assert ids[0].tolist() == [1, 1, 3]
    assert np.allclose(w[0], 1.0 / 3)


def test_hash_route_rejects_bad_ids():
    wr = np.ones((4, 8), np.float32)
    with pytest.raises(AssertionError):
        oracle.route_hash(np.ones((1, 8)), wr, np.array([[0, 1]], np.int32), np.array([1], np.int32))
    with pytest.raises(AssertionError):
        oracle.route_hash(np.ones((1, 8)), wr, np.array([[0, 4]], np.int32), np.array([0], np.int32))
