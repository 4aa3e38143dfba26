"""Pins for the oracle's draft top-K / log-sum-exp and DDTree tree
construction (CPU only).  Each pin checks the oracle against something it
does not compute itself: a hand-worked tree, scipy's logsumexp, numpy's
stable sort, brute-force enumeration of every path, or a closed form."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_golden_small_tree():
    g = json.load(open(os.path.join(HERE, "golden", "draft_tree_small.json")))
    with np.errstate(divide="ignore"):
        X = np.log(np.array(g["probs"]))
    idx, val, lse = oracle.draft_topk(X, g["K"])
    assert idx.tolist() == g["topk_idx"]
    np.testing.assert_allclose(lse, 0.0, atol=1e-12)
    parent, tok, score, depth, _ = oracle.build_tree(idx, oracle.log_probs(val, lse), g["N"], g["root_token"])
    assert parent.tolist() == g["parent"]
    assert tok.tolist() == g["tok"]
    assert depth.tolist() == g["depth"]
    np.testing.assert_allclose(np.exp(score), g["score_p"], rtol=1e-12)


def test_topk_ties_nan_and_inf_by_hand():
    X = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, np.nan],
                  [np.nan, 0.5, -np.inf, 0.5, np.inf * -1, 0.25],
                  [-np.inf] * 6], dtype=np.float32)
    idx, val, lse = oracle.draft_topk(X, 4)
    assert idx[0].tolist() == [1, 2, 4, 3]        # equal values: lower index first; NaN never chosen
    assert idx[1].tolist() == [1, 3, 5, -1]       # only three finite logits
    assert idx[2].tolist() == [-1, -1, -1, -1]
    assert np.isneginf(val[1, 3]) and np.isneginf(lse[2])
    np.testing.assert_allclose(lse[0], logsumexp([1, 3, 3, 2, 3]), rtol=1e-13)
    np.testing.assert_allclose(lse[1], logsumexp([0.5, 0.5, 0.25]), rtol=1e-13)


def test_topk_and_lse_match_library_on_random_rows():
    rng = np.random.default_rng(3)
    for dt in ("f32", "bf16"):
        X = synth.store(rng.standard_normal((5, 3001)) * 2, dt)
        x = oracle.num.f64(X)
        idx, val, lse = oracle.draft_topk(X, 8)
        for i in range(5):
            order = np.argsort(-x[i], kind="stable")[:8]   # stable: ties keep index order
            assert idx[i].tolist() == order.tolist()
            np.testing.assert_array_equal(val[i], x[i][order])
        np.testing.assert_allclose(lse, logsumexp(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("K,L", [(1, 3), (2, 3), (3, 2), (2, 4), (3, 3)])
def test_tree_equals_sort_of_all_paths(K, L):
    rng = np.random.default_rng(10 * K + L)
    for trial in range(5):
        X = rng.standard_normal((L, 12))
        if trial == 1:
            X = np.round(X)                            # many exact logit ties
        idx, val, lse = oracle.draft_topk(X, K)
        lp = oracle.log_probs(val, lse)
        total = sum(K ** d for d in range(1, L + 1))
        for N in (1, 2, 5, total + 1, total + 5):
            p, t, s, _, _ = oracle.build_tree(idx, lp, N, 99)
            pb, tb, sb = oracle.build_tree_brute(idx, lp, N, 99)
            assert p.tolist() == pb.tolist() and t.tolist() == tb.tolist()
            np.testing.assert_array_equal(s, sb)
            assert len(p) == min(N, total + 1)


def test_k1_is_a_chain_of_the_argmax_tokens():
    X = np.random.default_rng(4).standard_normal((6, 40))
    idx, val, lse = oracle.draft_topk(X, 1)
    p, t, s, d, _ = oracle.build_tree(idx, oracle.log_probs(val, lse), 22, 5)
    assert p.tolist() == [-1, 0, 1, 2, 3, 4, 5]
    assert t[1:].tolist() == np.argmax(X, axis=1).tolist() and t[0] == 5
    assert d.tolist() == list(range(7))


def test_uniform_positions_give_breadth_first_tree():
    # every candidate has the same log-probability, so scores depend on depth
    # only: all depth-1 nodes (rank order), then depth 2 in rank-sequence order
    K, L = 3, 3
    X = np.zeros((L, 20))
    idx, val, lse = oracle.draft_topk(X, K)
    lp = oracle.log_probs(val, lse)
    np.testing.assert_allclose(lp, -np.log(20.0))
    p, t, s, d, rk = oracle.build_tree(idx, lp, 1 + 3 + 5, 0)
    assert p.tolist() == [-1, 0, 0, 0, 1, 1, 1, 2, 2]
    assert d.tolist() == [0, 1, 1, 1, 2, 2, 2, 2, 2]
    assert t.tolist() == [0, 0, 1, 2, 0, 1, 2, 0, 1]   # candidates are tokens 0, 1, 2 (ties by index)


def test_dead_position_stops_the_tree():
    X = np.random.default_rng(5).standard_normal((4, 30))
    X[2, :] = np.nan                                     # position 2 has no candidate
    idx, val, lse = oracle.draft_topk(X, 2)
    p, t, s, d, _ = oracle.build_tree(idx, oracle.log_probs(val, lse), 50, 1)
    assert d.max() == 2 and len(p) == 1 + 2 + 4


def test_tree_invariants_on_realistic_draft():
    lg = synth.draft_logits(0, (7,), 16, 5000, "bf16")
    idx, val, lse = oracle.draft_topk(lg, 8)
    p, t, s, d, rk = oracle.build_tree(idx, oracle.log_probs(val, lse), 22, 3)
    assert len(p) == 22
    assert all(p[i] < i for i in range(1, 22))
    keys = [(-s[i], rk[i]) for i in range(1, 22)]
    assert keys == sorted(keys)                          # numbered in selection order
    for i in range(1, 22):
        assert d[i] == d[p[i]] + 1 and rk[i][:-1] == rk[p[i]]
        assert t[i] == idx[d[i] - 1, rk[i][-1]]
    # nothing left out scores higher than the worst node kept
    kept = set(rk)
    for r in itertools.chain.from_iterable(((x + (k,)) for k in range(8)) for x in rk):
        if r not in kept and len(r) <= 16:
            sc = sum(oracle.log_probs(val, lse)[j, r[j]] for j in range(len(r)))
            assert (-sc, r) > max(keys)
