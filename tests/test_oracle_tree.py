"""Pins for the oracle's tree bookkeeping (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def all_trees(n):
    """Every parent array with parent[i] in [0, i): (n-1)! trees."""
    for ps in itertools.product(*[range(i) for i in range(1, n)]):
        yield np.array([-1, *ps], dtype=np.int64)


def test_tiny_tree_golden():
    g = json.load(open(os.path.join(GOLD, "tiny_tree.json")))
    par = np.array(g["parent"])
    assert list(oracle.depth(par)) == g["depth"]
    assert oracle.ancestor_mask(par) == g["anc"]
    assert oracle.conv_window(par, 4).tolist() == g["win_w4"]
    assert list(synth.binary_tree(3)) == g["parent"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_brute_force_all_trees(n):
    """Ancestor masks from downward reachability (children lists, BFS) and
    windows from depth arithmetic, against the oracle's pointer chasing."""
    for par in all_trees(n):
        ch = [[] for _ in range(n)]
        for i in range(1, n):
            ch[par[i]].append(i)
        anc = [0] * n
        for j in range(n):              # j is an ancestor of everything below it
            stack = [j]
            while stack:
                u = stack.pop()
                anc[u] |= 1 << j
                stack.extend(ch[u])
        assert oracle.ancestor_mask(par) == anc
        d = oracle.depth(par)
        assert all(bin(anc[i]).count("1") == d[i] + 1 for i in range(n))
        W = 4
        win = oracle.conv_window(par, W)
        for i in range(n):
            for j in range(1, W):
                if j <= d[i]:
                    # the ancestor of i at depth d(i)-j
                    cand = [a for a in range(n) if (anc[i] >> a) & 1 and d[a] == d[i] - j]
                    assert win[i, j - 1] == cand[0] and len(cand) == 1
                else:
                    assert win[i, j - 1] == -((W - 1) - (j - d[i]) + 1)


def test_validation():
    with pytest.raises(oracle.TreeError):
        oracle.validate_tree([0, 0])
    with pytest.raises(oracle.TreeError):
        oracle.validate_tree([-1, 1])
    with pytest.raises(oracle.TreeError):
        oracle.validate_tree([-1, 0, 3, 0])
    with pytest.raises(oracle.TreeError):
        oracle.validate_tree(list(range(-1, 64)))  # 65 nodes
    with pytest.raises(oracle.TreeError):
        oracle.validate_tree([-1, 0, 1, 2], max_levels=3)
    oracle.validate_tree([-1, 0, 1, 2], max_levels=4)


def test_generator_level_cap():
    for s in range(20):
        par = synth.random_tree(synth.rng_for(s, 99), 22, 8)
        oracle.validate_tree(par, max_levels=8)
        par = synth.random_tree(synth.rng_for(s, 98), 64, 10)
        oracle.validate_tree(par, max_levels=10)
