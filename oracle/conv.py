"""Tree-aware causal depthwise conv1d (oracle; test infrastructure).

The pages name a tree-mode conv for the SSM layers (lucebox-hub README,
"02 · DFlash DDtree", "Implemented here": ggml_ssm_conv_tree) without a
formula.  Reading: a plain depthwise causal conv of width W, no bias, applied
to each node as if its root path had been appended to the committed tokens;
weight tap W-1 multiplies the current token; optional SiLU.
"""
import numpy as np

from .num import f64
from .tree import root_path


def _silu(z):
    return z / (1.0 + np.exp(-z))


def tree_conv(parent, x, prefix, w, act=0, tree_off=None):
    """y[i][c] = act( sum_{t=0}^{W-1} w[c][W-1-t] * seq_i[-1-t][c] ) where
    seq_i = prefix_b ++ x[root path of i] (prefix oldest first).

    parent: concatenated local parent arrays; tree_off [B+1] (None = one tree);
    x [n][C]; prefix [B][W-1][C]; w [C][W].  Returns fp64 [n][C]."""
    parent = np.asarray(parent)
    X, P, Wt = f64(x), f64(prefix), f64(w)
    C, W = Wt.shape
    if tree_off is None:
        tree_off = [0, len(parent)]
    y = np.zeros((len(parent), C))
    for b in range(len(tree_off) - 1):
        o, e = int(tree_off[b]), int(tree_off[b + 1])
        par = parent[o:e]
        for i in range(e - o):
            path = [o + j for j in root_path(par, i)]
            seq = np.concatenate([P[b], X[path]], axis=0)  # [(W-1)+len][C]
            acc = np.zeros(C)
            for t in range(W):
                acc += Wt[:, W - 1 - t] * seq[-1 - t]
            y[o + i] = _silu(acc) if act == 1 else acc
    return y
