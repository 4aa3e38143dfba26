"""Stochastic tree acceptance (oracle; test infrastructure).

Sources.  Requests that give no temperature are sampled with the model
card's settings, temperature 1.0, top_p 0.95 and top_k 20, while greedy
decoding (temperature 0) accepts the most drafts (codehub lucebox-hub@main,
"Making requests").  The pages give no rule for accepting a draft tree under
sampling.

Readings (the plainest ones the pages support)
----------------------------------------------
* Target distribution at a node, in the order temperature -> top-k -> top-p:
  the logits divided by T; the top_k tokens by logit (ties to the lower
  index; NaN counts as -inf and -inf tokens are never kept); their softmax
  p_i, in descending order; the smallest prefix whose mass reaches
  top_p * (total mass of the top_k), at least one token; renormalised.
* Sampling with the node's uniform u in [0, 1): with c_i the inclusive
  cumulative masses of the kept prefix (descending order) and R its total,
  the sample is the first kept token with c_i > u * R.
* Acceptance: at each node reached, starting at the root, draw that node's
  sample; if a child carries that token, move to the child (the lowest
  index if several do) and repeat; otherwise stop.  The last sample is the
  bonus token.  Every emitted token is then a draw from the target's own
  distribution at its prefix, so the output is distributed as plain
  sampling from the target; this is recursive rejection sampling with the
  drafts as deterministic candidates (a candidate x is accepted with
  probability p(x) given that its earlier siblings were not, as min(1,
  p/q) gives for q = 1 on x).  The tree walk is the greedy walk with the
  samples in place of the argmax (walk.accept_walk).
* The random numbers are inputs: one uniform per tree node.
"""
import numpy as np

from .num import f64


def filtered_dist(row, temperature, top_k, top_p):
    """Kept tokens (descending order, ties to the lower index) and their
    unnormalised masses exp((v - v_max) / T) for one row of logits."""
    x = f64(row).copy()
    x[np.isnan(x)] = -np.inf
    order = np.lexsort((np.arange(len(x)), -x))[:top_k]
    order = np.array([t for t in order if np.isfinite(x[t])], dtype=np.int64)
    if len(order) == 0:
        return order, np.zeros(0)
    v = x[order]
    p = np.exp((v - v[0]) / temperature)
    c = np.cumsum(p)
    m = int(np.argmax(c >= top_p * c[-1])) + 1  # smallest prefix reaching top_p of the mass
    return order[:m], p[:m]


def sample_row(row, u, temperature, top_k, top_p):
    """(token, margin): the sampled token of one row and the relative
    distance of u * R to the nearest decision boundary (cumulative mass or
    the top-p cut), so that a test can tell rounding-order ties apart.
    Token -1 when the row has no finite logit."""
    x = f64(row).copy()
    x[np.isnan(x)] = -np.inf
    order = np.lexsort((np.arange(len(x)), -x))[:top_k]
    order = np.array([t for t in order if np.isfinite(x[t])], dtype=np.int64)
    if len(order) == 0:
        return -1, np.inf
    v = x[order]
    p = np.exp((v - v[0]) / temperature)
    call = np.cumsum(p)
    thr = top_p * call[-1]
    m = int(np.argmax(call >= thr)) + 1
    c = call[:m]
    R = c[-1]
    t = u * R
    i = int(np.argmax(c > t))
    # closeness to the boundaries the decision depends on: the top-p cut
    # (every c_i >= thr test; with top_p = 1 the last one holds by
    # construction on any machine) and the cumulative masses around t
    cut = call[:-1] if top_p >= 1.0 else call
    marg = np.min(np.abs(cut - thr)) / call[-1] if len(cut) else np.inf
    marg = min(marg, np.min(np.abs(c - t)) / R)
    return int(order[i]), marg


def sample_tokens(logits, u, temperature, top_k, top_p):
    """Samples [n] (int64) and margins [n] for logits [n][V] and uniforms [n]."""
    toks, margs = [], []
    for r in range(len(logits)):
        t, mg = sample_row(logits[r], float(u[r]), temperature, top_k, top_p)
        toks.append(t)
        margs.append(mg)
    return np.array(toks, dtype=np.int64), np.array(margs)
