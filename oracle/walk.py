"""Verify argmax and greedy acceptance walk (oracle; test infrastructure).

Greedy (temperature 0) acceptance against the target's per-node argmax
(codehub lucebox-hub@main, "Run the Server", "Making requests": greedy
decoding gives the highest acceptance; "GPU draft top-K & verify-argmax
(DFlash)": the verify argmax is read from the device logits).

Readings: ties take the lowest vocabulary index; NaN never wins (treated as
-inf); among children carrying the accepted token the lowest node index is
taken.  The walk starts at the root and keeps stepping to a child whose
draft token equals the current node's argmax; it emits L = |path| tokens
(L-1 accepted drafts plus the bonus argmax of the last node).
"""
import numpy as np

from .num import f64


def argmax_rows(logits):
    X = f64(logits).copy()
    X[np.isnan(X)] = -np.inf
    return np.argmax(X, axis=1).astype(np.int64)  # first occurrence of the max


def accept_walk(parent, draft_tok, amax, tree_off=None):
    """Returns (paths: list of local node lists, L [B], bonus [B])."""
    parent = np.asarray(parent)
    if tree_off is None:
        tree_off = [0, len(parent)]
    paths, L, bonus = [], [], []
    for b in range(len(tree_off) - 1):
        o, e = int(tree_off[b]), int(tree_off[b + 1])
        path = [0]
        while True:
            cur = path[-1]
            a = int(amax[o + cur])
            nxt = [c for c in range(e - o) if int(parent[o + c]) == cur and int(draft_tok[o + c]) == a]
            if not nxt:
                break
            path.append(min(nxt))
        paths.append(path)
        L.append(len(path))
        bonus.append(int(amax[o + path[-1]]))
    return paths, np.array(L), np.array(bonus)
