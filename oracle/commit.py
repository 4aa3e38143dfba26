"""Commit of the accepted path (oracle; test infrastructure).

After the walk the accepted node's linear-attention state becomes the
committed state (the pages' "tree-aware SSM state rollback", lucebox-hub
README, "02 · DFlash DDtree", "Implemented here"), the conv prefix advances
over the accepted tokens and their K/V enter the cache.

Readings: the root (last committed token) is processed in this step, so the
path's L tokens (root included) are appended at positions T..T+L-1 and T
grows by L; the bonus token becomes the next step's root.
"""
import numpy as np

from .gdn import gdn_chain
from .num import f64


def commit_gdn_state(S_c, q, k, v, alpha, beta, path_global, b, scale=1.0):
    """New committed state [Hv][dv][dk] of sequence b: replay of the path."""
    Q, K, Vv, A, Bt, S0 = f64(q), f64(k), f64(v), f64(alpha), f64(beta), f64(S_c)
    Hk, Hv = Q.shape[1], Vv.shape[1]
    grp = Hv // Hk
    p = list(path_global)
    out = np.zeros(S0.shape[1:])
    for h in range(Hv):
        g = h // grp
        _, S = gdn_chain(S0[b, h], Q[p, g], K[p, g], Vv[p, h], A[p, h], Bt[p, h], scale)
        out[h] = S
    return out


def commit_conv_prefix(prefix, x, path_global, b):
    """New prefix [W-1][C]: the last W-1 rows of prefix_b ++ x[path]."""
    P, X = f64(prefix), f64(x)
    W1 = P.shape[1]
    seq = np.concatenate([P[b], X[list(path_global)]], axis=0)
    return seq[len(seq) - W1:]


def commit_kv(Kp, Vp, page_table, T, Kt, Vt, path_global, b):
    """Copies of the pools with the path's draft K/V written at T_b..T_b+L-1
    of sequence b (values copied bit for bit), and the new length."""
    Kp, Vp = Kp.copy(), Vp.copy()
    PAGE = Kp.shape[2]
    t0 = int(np.atleast_1d(T)[b])
    for r, node in enumerate(path_global):
        t = t0 + r
        page = (t // PAGE) if page_table is None else int(np.asarray(page_table)[b][t // PAGE])
        Kp[page, :, t % PAGE, :] = Kt[node]
        Vp[page, :, :, t % PAGE] = Vt[node]
    return Kp, Vp, t0 + len(path_global)
