"""Fused input stage of a linear-attention layer feeding the tree gated
delta-net (oracle; test infrastructure).

Sources.  The pages list a tree-mode short conv and tree gated delta-net
kernels side by side (lucebox-hub README, "02 · DFlash DDtree",
"Implemented here": ssm_conv_tree, gated_delta_net_tree and its _persist
variant) and run a whole forward pass in one persistent dispatch with no
host round trips between layers (same README, "01 · Megakernel").  How the
conv output becomes the delta rule's q, k and v is the Gated DeltaNet
layer (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024): a short
causal conv with SiLU over the projected q, k and v, L2-normalised q and k,
then the gated delta rule.

Readings (the pages give none of these):
* The conv channels are [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)], each part
  head-major (channel h*d + j is entry j of head h), so C = 2*Hk*dk + Hv*dv
  (8192 = 2*16*128 + 32*128 for the 27B layer shape).
* SiLU follows the conv on every channel; no bias.
* q and k are L2-normalised per head as x / sqrt(sum x^2 + eps) with
  eps = 1e-6 (a zero vector stays zero); v is not normalised.
* The gates alpha, beta are inputs (a model computes them from its own
  projections); the output scale is an argument, as for the delta-net alone.
"""
import numpy as np

from .conv import tree_conv
from .gdn import tree_gdn

L2_EPS = 1e-6


def qkv_split_norm(y, Hk, Hv, dk, dv, eps=L2_EPS):
    """Conv output rows [n][C] -> q, k [n][Hk][dk] (L2-normalised per head)
    and v [n][Hv][dv], all fp64."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[0]
    assert y.shape[1] == 2 * Hk * dk + Hv * dv
    q = y[:, :Hk * dk].reshape(n, Hk, dk)
    k = y[:, Hk * dk:2 * Hk * dk].reshape(n, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(n, Hv, dv).copy()

    def l2n(a):
        out = np.empty_like(a)
        for i in range(a.shape[0]):
            for h in range(a.shape[1]):
                out[i, h] = a[i, h] / np.sqrt(np.sum(a[i, h] ** 2) + eps)
        return out

    return l2n(q), l2n(k), v


def tree_conv_gdn(parent, x, prefix, w, alpha, beta, S_c, Hk, Hv, dk, dv, scale=1.0,
                  tree_off=None, want_states=False):
    """The fused layer over a tree: tree conv with SiLU, split and
    normalisation, then the tree gated delta rule.

    x [n][C]; prefix [B][W-1][C]; w [C][W]; alpha, beta [n][Hv];
    S_c [B][Hv][dv][dk].  Returns (out [n][Hv][dv], q, k, v) and, with
    want_states, the node states [n][Hv][dv][dk] after them."""
    y = tree_conv(parent, x, prefix, w, act=1, tree_off=tree_off)
    q, k, v = qkv_split_norm(y, Hk, Hv, dk, dv)
    r = tree_gdn(parent, q, k, v, alpha, beta, S_c, scale=scale, tree_off=tree_off,
                 want_states=want_states)
    if want_states:
        return r[0], q, k, v, r[1]
    return r, q, k, v
