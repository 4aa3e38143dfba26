"""Tree bookkeeping for the oracle (test infrastructure).

A draft tree is a parent-pointer array: node 0 is the root (the last
committed, not yet processed token), parent[0] = -1 and 0 <= parent[i] < i.
The root counts toward the budget (lucebox-hub README, "02 · DFlash DDtree",
budget 22; codehub lucebox-hub@main, "Server flags", --ddtree-budget).

Readings where the pages are silent:
* "levels" count the nodes on a root path (a lone root has one level), so a
  cap of L levels allows edge depth up to L-1.
* A node's conv window is the W-1 tokens before it on the sequence
  ``committed prefix ++ root path``; window slot j (1-based, j-th previous
  token) is an ancestor id when the path is long enough, else a prefix slot
  encoded as -(s+1) with prefix slot s = 0 the oldest.
"""
import numpy as np


class TreeError(ValueError):
    pass


def validate_tree(parent, max_levels=None, n_max=64):
    parent = np.asarray(parent)
    n = len(parent)
    if n < 1 or n > n_max:
        raise TreeError(f"tree size {n} outside [1, {n_max}]")
    if int(parent[0]) != -1:
        raise TreeError("parent[0] must be -1")
    for i in range(1, n):
        if not (0 <= int(parent[i]) < i):
            raise TreeError(f"parent[{i}]={int(parent[i])} not in [0,{i})")
    if max_levels is not None:
        if int(max(depth(parent))) + 1 > max_levels:
            raise TreeError("tree exceeds the level cap")


def root_path(parent, i):
    """Nodes from the root to i inclusive, by following parent pointers."""
    out = [int(i)]
    while parent[out[-1]] >= 0:
        out.append(int(parent[out[-1]]))
    return out[::-1]


def depth(parent):
    """Edge depth of every node: number of proper ancestors."""
    return np.array([len(root_path(parent, i)) - 1 for i in range(len(parent))], dtype=np.int64)


def ancestor_mask(parent):
    """Bit j of mask i is set iff node j lies on i's root path (i included)."""
    return [sum(1 << j for j in root_path(parent, i)) for i in range(len(parent))]


def conv_window(parent, W):
    """[n][W-1] table; entry j-1 names the j-th previous token of node i."""
    n = len(parent)
    win = np.zeros((n, max(W - 1, 0)), dtype=np.int64)
    for i in range(n):
        p = root_path(parent, i)
        m = len(p) - 1
        for j in range(1, W):
            if j <= m:
                win[i, j - 1] = p[m - j]
            else:
                s = (W - 1) - (j - m)
                win[i, j - 1] = -(s + 1)
    return win
