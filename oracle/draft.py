"""Draft top-K, log-sum-exp and DDTree tree construction (oracle; test
infrastructure only).

What is computed (sources)
--------------------------
* The draft model's K most likely vocabulary indices (K from 1 to 8) and the
  log-sum-exp of each draft position's logits are taken on the device, from
  the logits buffer in place (codehub lucebox-hub@main, "GPU draft top-K &
  verify-argmax (DFlash)").
* DDTree turns the block-diffusion drafter's output into a tree of draft
  tokens under a node budget, which the target verifies in one pass
  (lucebox-hub README, "02 · DFlash DDtree ...", "Algorithms used"; budget
  22 under "Implemented here").  The pages give no selection rule.

Readings (the plainest ones the pages support)
----------------------------------------------
* The drafter predicts a block of L positions in one pass, so the
  distribution of position i does not depend on the tokens chosen at
  earlier positions.  The root (node 0) is the last committed token, depth
  0; a node at depth d >= 1 holds a token of draft position d-1 (0-based),
  and its candidate children are the K most likely tokens of position d.
* log p(token) = logit - LSE of its position.  A node's score is the sum of
  the log-probabilities on its root path (the root scores 0).
* The tree is the root plus the N-1 best nodes under one total order: score
  descending, then the sequence of candidate ranks along the root path,
  lexicographically ascending with a prefix before its extensions.  A
  child's score never exceeds its parent's, so the order lists every parent
  before its children: the best N-1 nodes are closed under taking parents
  (they form a tree), and they are what best-first expansion from the root
  selects.  Nodes are numbered in that order.
* Top-K ties take the lower vocabulary index.  NaN logits count as -inf;
  -inf logits are never candidates and LSE ignores them.  A position with
  no finite logit has no candidates, so the tree ends before it.  If fewer
  than N-1 nodes can be formed the tree is smaller.
"""
import heapq

import numpy as np

from .num import f64


def draft_topk(logits, K):
    """Top-K per position and log-sum-exp.

    logits: [L][V] stored values (fp32 / fp16 / bf16 bit patterns).
    Returns idx [L][K] int64, val [L][K] (the logits, fp64) and lse [L]
    (fp64).  Entries past a row's finite logits have idx -1 and val -inf."""
    X = f64(logits).copy()
    X[np.isnan(X)] = -np.inf
    L, V = X.shape
    idx = np.full((L, K), -1, dtype=np.int64)
    val = np.full((L, K), -np.inf)
    lse = np.full(L, -np.inf)
    for i in range(L):
        row = X[i]
        # ascending by (-value, index): largest first, ties to the lower index
        order = np.lexsort((np.arange(V), -row))
        for k in range(K):
            t = order[k]
            if np.isfinite(row[t]):
                idx[i, k] = t
                val[i, k] = row[t]
        fin = row[np.isfinite(row)]
        if fin.size:
            m = fin.max()
            lse[i] = m + np.log(np.exp(fin - m).sum())
    return idx, val, lse


def log_probs(val, lse):
    """log p of each top-K entry: logit - LSE of its position (-inf where absent)."""
    lp = np.full(val.shape, -np.inf)
    for i in range(val.shape[0]):
        if np.isfinite(lse[i]):
            ok = np.isfinite(val[i])
            lp[i, ok] = val[i, ok] - lse[i]
    return lp


def build_tree(idx, lp, N, root_token):
    """Best-first DDTree construction.

    idx, lp: [L][K] candidate tokens and their log-probabilities per draft
    position.  Returns parent [n] (-1 for the root), tok [n], score [n]
    (fp64), depth [n] and ranks (tuple of candidate ranks per node), n <= N."""
    L, K = idx.shape
    parent, tok, score, depth, ranks = [-1], [int(root_token)], [0.0], [0], [()]
    heap = []

    def push_children(node):
        d = depth[node]
        if d >= L:
            return
        for k in range(K):
            if np.isfinite(lp[d, k]):
                s = score[node] + lp[d, k]
                heapq.heappush(heap, (-s, ranks[node] + (k,), node, k))

    push_children(0)
    while len(parent) < N and heap:
        neg_s, rk, par, k = heapq.heappop(heap)
        d = depth[par]
        parent.append(par)
        tok.append(int(idx[d, k]))
        score.append(-neg_s)
        depth.append(d + 1)
        ranks.append(rk)
        push_children(len(parent) - 1)
    return (np.array(parent, dtype=np.int64), np.array(tok, dtype=np.int64), np.array(score),
            np.array(depth, dtype=np.int64), ranks)


def build_tree_brute(idx, lp, N, root_token):
    """The same tree by listing every candidate path and sorting them all
    (tiny K and L only); used to pin build_tree."""
    L, K = idx.shape
    paths = [((), 0.0)]
    frontier = [((), 0.0)]
    for d in range(L):
        nxt = []
        for rk, s in frontier:
            for k in range(K):
                if np.isfinite(lp[d, k]):
                    nxt.append((rk + (k,), s + lp[d, k]))
        paths += nxt
        frontier = nxt
    body = sorted(paths[1:], key=lambda p: (-p[1], p[0]))[:N - 1]
    order = [()] + [p[0] for p in body]
    num = {rk: i for i, rk in enumerate(order)}
    parent = [-1] + [num[rk[:-1]] for rk in order[1:]]
    tok = [int(root_token)] + [int(idx[len(rk) - 1, rk[-1]]) for rk in order[1:]]
    score = [0.0] + [p[1] for p in body]
    return np.array(parent, dtype=np.int64), np.array(tok, dtype=np.int64), np.array(score)
