"""Pins of the oracle's routing (logits, top-k, gates) against facts that do not
come from the oracle: closed forms, brute force over all k-subsets, and
library routines (numpy argmax, scipy softmax)."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _brute_topk_set(z, k):
    """Max-sum k-subset; among equal sums the lexicographically smallest ids."""
    best = None
    for sub in itertools.combinations(range(len(z)), k):
        s = sum(z[e] for e in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    return set(best[1])


@pytest.mark.parametrize("E,k", [(1, 1), (3, 1), (4, 2), (5, 3), (6, 2), (7, 4), (7, 7)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # small integer logits force many exact ties
    z = rng.integers(-2, 3, size=(300, E)).astype(np.float64)
    idx = oracle.topk(z, k)
    for t in range(z.shape[0]):
        assert set(idx[t].tolist()) == _brute_topk_set(z[t], k)
        assert len(set(idx[t].tolist())) == k
        # slot 0 is the arg-max with the lowest id among equals (numpy's argmax rule)
        assert idx[t, 0] == int(np.argmax(z[t]))
        # slots are in non-increasing logit order
        assert all(z[t, idx[t, j]] >= z[t, idx[t, j + 1]] for j in range(k - 1))


def test_gates_match_softmax_over_chosen():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(200, 16)) * 3
    for k in (1, 2, 5, 16):
        idx = oracle.topk(z, k)
        g = oracle.gates(z, idx)
        for t in range(z.shape[0]):
            np.testing.assert_allclose(g[t], softmax(z[t, idx[t]]), rtol=1e-13, atol=0)
        assert np.all(np.abs(g.sum(1) - 1.0) < 1e-14)
        assert np.all(np.diff(g, axis=1) <= 0)


def test_k1_gate_is_exactly_one_and_kE_is_full_softmax():
    rng = np.random.default_rng(2)
    z = rng.normal(size=(50, 8))
    idx = oracle.topk(z, 1)
    assert np.all(oracle.gates(z, idx) == 1.0)
    idx = oracle.topk(z, 8)
    g = oracle.gates(z, idx)
    for t in range(50):
        np.testing.assert_allclose(g[t], softmax(z[t])[idx[t]], rtol=1e-13)
        assert sorted(idx[t].tolist()) == list(range(8))


def test_logits_fp32_chain_order_closed_form():
    # chain 0 + 2^24 -> 2^24; + 1 -> 2^24 (tie to even); - 2^24 -> 0.  Exact sum is 1;
    # the reversed order would give 1.  The sequential fp32 chain must give 0.
    x = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]], np.float32)
    w = np.ones((1, 3), np.float32)
    assert oracle.logits(x, w, None, "bf16")[0, 0] == 0.0
    assert oracle.logits(x, w, None, "exact")[0, 0] == 1.0


def test_logits_use_fused_multiply_add():
    # (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 exactly; a rounded product would lose 2^-24.
    a = 1.0 + 2.0 ** -12
    x = np.array([[-1.0, a]], np.float32)
    w = np.array([[1.0, a]], np.float32)
    assert oracle.logits(x, w, None, "f32")[0, 0] == 2.0 ** -11 + 2.0 ** -24


def test_logits_bias_is_one_fp32_add_after_the_chain():
    x = np.array([[1.0, 2.0 ** -30]], np.float32)
    w = np.array([[1.0, 1.0]], np.float32)
    b = np.array([-1.0], np.float32)
    # chain: 1 + 2^-30 -> 1 in fp32; + (-1) -> 0 (bias not folded into the chain start)
    assert oracle.logits(x, w, b, "f32")[0, 0] == 0.0


def test_logits_within_fp32_error_bound_of_exact_sum():
    rng = np.random.default_rng(3)
    d = 512
    x = rng.normal(size=(64, d)).astype(np.float32)
    w = rng.normal(size=(8, d)).astype(np.float32)
    z32 = oracle.logits(x, w, None, "f32")
    z64 = x.astype(np.float64) @ w.astype(np.float64).T
    bound = d * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T)
    assert np.all(np.abs(z32 - z64) <= bound)
    assert np.all(z32 == z32.astype(np.float32))  # values are fp32


def test_route_composes_logits_topk_gates():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(40, 32)).astype(np.float32)
    w = rng.normal(size=(6, 32)).astype(np.float32)
    b = rng.normal(size=6).astype(np.float32)
    idx, g = oracle.route(x, w, b, 3, "bf16")
    z = x.astype(np.float64) @ w.astype(np.float64).T + b
    for t in range(40):
        order = np.argsort(-z[t], kind="stable")[:3]
        assert idx[t].tolist() == order.tolist()
        np.testing.assert_allclose(g[t], softmax(z[t][order]), rtol=1e-5)


def _lexsort_topk(z, k):
    """Independent ordering: numbers before NaNs, larger logit first, lower
    id first among equals (numpy lexsort: the last key is the primary one)."""
    E = z.shape[0]
    nan = np.isnan(z)
    negz = np.where(nan, 0.0, -z)
    return np.lexsort((np.arange(E), negz, nan))[:k]


@pytest.mark.parametrize("E,k", [(4, 2), (8, 8), (7, 3), (16, 5)])
def test_topk_nan_ranks_after_every_number(E, k):
    """Reading (the pages say nothing of non-numbers): a NaN logit ranks
    after every number, -inf included; NaNs rank among themselves by id."""
    rng = np.random.default_rng(40 + E + k)
    z = rng.integers(-2, 3, size=(400, E)).astype(np.float64)
    z[rng.random(z.shape) < 0.25] = np.nan
    z[rng.random(z.shape) < 0.1] = -np.inf
    z[:5] = np.nan                    # whole rows of NaN
    idx = oracle.topk(z, k)
    for t in range(z.shape[0]):
        np.testing.assert_array_equal(idx[t], _lexsort_topk(z[t], k))
    assert np.all(idx[:5] == np.arange(k))   # an all-NaN row takes the k lowest ids


def test_gates_ignore_nan_among_unchosen_logits():
    """Gates are the softmax of the chosen logits: a NaN logit of an unchosen
    expert leaves them finite; an all-NaN row gives NaN gates."""
    rng = np.random.default_rng(3)
    z = rng.normal(size=(50, 8))
    z[:, 5] = np.nan
    idx = oracle.topk(z, 3)
    assert not np.any(idx == 5)
    g = oracle.gates(z, idx)
    for t in range(50):
        np.testing.assert_allclose(g[t], softmax(z[t, idx[t]]), rtol=1e-13, atol=0)
    zn = np.full((2, 8), np.nan)
    assert np.all(np.isnan(oracle.gates(zn, oracle.topk(zn, 2))))
