"""Tree gated delta-net (oracle; test infrastructure).

The pages name tree-aware gated delta-net kernels with a persisting variant
for state rollback (lucebox-hub README, "02 · DFlash DDtree", "Implemented
here").  The recurrence is the standard gated delta rule (Yang, Kautz,
Hatamizadeh, "Gated Delta Networks", 2024), per value head h:

    S_t = alpha_t * S_{t-1} @ (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t @ q_t

with S in R^{d_v x d_k} (v k^T is d_v x d_k, so o = S q is in R^{d_v}).
Readings: key head of value head h is h // (Hv // Hk) (contiguous groups);
the output reads the state after the node's own update; scale defaults to 1
(no 1/sqrt(d_k) is written in the rule).

Tree mode: a node's state is computed from its parent's state, the root's
from the committed state S_c.  By definition this must equal replaying the
node's root path from S_c.
"""
import numpy as np

from .num import f64
from .tree import root_path


def gdn_step(S, q, k, v, a, b, scale=1.0):
    """One token of the gated delta rule, literal matrix form."""
    dk = S.shape[1]
    S = a * (S @ (np.eye(dk) - b * np.outer(k, k))) + b * np.outer(v, k)
    return S, scale * (S @ q)


def gdn_chain(S0, q, k, v, alpha, beta, scale=1.0):
    """Sequential processing of a token sequence for one value head.
    q,k [L][dk], v [L][dv], alpha,beta [L]; returns (outputs [L][dv], S_L)."""
    S = np.array(S0, dtype=np.float64)
    outs = []
    for t in range(len(alpha)):
        S, o = gdn_step(S, q[t], k[t], v[t], alpha[t], beta[t], scale)
        outs.append(o)
    return np.array(outs).reshape(len(alpha), -1), S


def _prep(q, k, v, alpha, beta, S_c):
    return f64(q), f64(k), f64(v), f64(alpha), f64(beta), f64(S_c)


def tree_gdn(parent, q, k, v, alpha, beta, S_c, scale=1.0, tree_off=None, want_states=False):
    """Per-node outputs (and states) by replaying each node's root path.

    q,k [n][Hk][dk]; v [n][Hv][dv]; alpha,beta [n][Hv]; S_c [B][Hv][dv][dk].
    Returns out [n][Hv][dv] (and states [n][Hv][dv][dk])."""
    parent = np.asarray(parent)
    Q, K, Vv, A, Bt, S0 = _prep(q, k, v, alpha, beta, S_c)
    n, Hk, dk = Q.shape
    Hv, dv = Vv.shape[1], Vv.shape[2]
    grp = Hv // Hk
    if tree_off is None:
        tree_off = [0, n]
    out = np.zeros((n, Hv, dv))
    states = np.zeros((n, Hv, dv, dk)) if want_states else None
    for b in range(len(tree_off) - 1):
        o, e = int(tree_off[b]), int(tree_off[b + 1])
        par = parent[o:e]
        for i in range(e - o):
            path = [o + j for j in root_path(par, i)]
            for h in range(Hv):
                g = h // grp
                ys, S = gdn_chain(S0[b, h], Q[path, g], K[path, g], Vv[path, h],
                                  A[path, h], Bt[path, h], scale)
                out[o + i, h] = ys[-1]
                if want_states:
                    states[o + i, h] = S
    return (out, states) if want_states else out


def tree_gdn_recurrent(parent, q, k, v, alpha, beta, S_c, scale=1.0, tree_off=None):
    """Same quantity computed node by node from the parent's state (index
    order is topological because parent[i] < i).  Performs exactly the
    operations of the path replay, so the two agree bitwise."""
    parent = np.asarray(parent)
    Q, K, Vv, A, Bt, S0 = _prep(q, k, v, alpha, beta, S_c)
    n, Hk, dk = Q.shape
    Hv, dv = Vv.shape[1], Vv.shape[2]
    grp = Hv // Hk
    if tree_off is None:
        tree_off = [0, n]
    out = np.zeros((n, Hv, dv))
    states = np.zeros((n, Hv, dv, dk))
    for b in range(len(tree_off) - 1):
        o, e = int(tree_off[b]), int(tree_off[b + 1])
        for i in range(e - o):
            p = int(parent[o + i])
            for h in range(Hv):
                g = h // grp
                Sp = S0[b, h] if p < 0 else states[o + p, h]
                S, y = gdn_step(Sp, Q[o + i, g], K[o + i, g], Vv[o + i, h],
                                A[o + i, h], Bt[o + i, h], scale)
                states[o + i, h] = S
                out[o + i, h] = y
    return out, states
