"""Pins for the oracle's fused conv -> SiLU -> split -> L2 norm -> delta-net
layer (CPU only)."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth

SHAPE = dict(Hk=2, Hv=4, dk=8, dv=8)  # C = 2*2*8 + 4*8 = 64


def _C(Hk, Hv, dk, dv):
    return 2 * Hk * dk + Hv * dv


def test_split_norm_matches_torch_normalize():
    Hk, Hv, dk, dv = 3, 2, 16, 8
    n = 5
    y = synth.rng_for(7, 1).standard_normal((n, _C(Hk, Hv, dk, dv)))
    y[2, Hk * dk:Hk * dk + dk] = 0.0          # one all-zero key head
    q, k, v = oracle.qkv_split_norm(y, Hk, Hv, dk, dv)
    t = torch.tensor(y)
    # library normalisation; eps = 1e-6 under the root moves unit vectors of
    # these norms by far less than 1e-6
    qr = F.normalize(t[:, :Hk * dk].reshape(n, Hk, dk), dim=-1).numpy()
    kr = F.normalize(t[:, Hk * dk:2 * Hk * dk].reshape(n, Hk, dk), dim=-1).numpy()
    np.testing.assert_allclose(q, qr, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(k, kr, rtol=1e-6, atol=1e-9)
    np.testing.assert_array_equal(k[2, 0], np.zeros(dk))       # zero stays zero, no NaN
    np.testing.assert_array_equal(v, y[:, 2 * Hk * dk:].reshape(n, Hv, dv))  # v untouched
    nq = np.linalg.norm(q, axis=-1)
    assert np.all(np.abs(nq - 1.0) < 1e-6)


def _library_chain(inp, Hk, Hv, dk, dv, scale):
    """The layer on a chain from library routines: torch depthwise conv1d
    over prefix ++ x, torch SiLU, head-major split, torch L2 normalisation,
    then the (separately pinned) delta rule chain per value head."""
    x = np.asarray(oracle.num.f64(inp["x"]))
    pre = np.asarray(oracle.num.f64(inp["prefix"]))[0]
    w = np.asarray(oracle.num.f64(inp["w"]))
    n, C = x.shape
    seq = torch.tensor(np.concatenate([pre, x], 0).T[None])
    y = F.conv1d(seq, torch.tensor(w)[:, None, :], groups=C)[0].T
    y = F.silu(y)
    q = F.normalize(y[:, :Hk * dk].reshape(n, Hk, dk), dim=-1).numpy()
    k = F.normalize(y[:, Hk * dk:2 * Hk * dk].reshape(n, Hk, dk), dim=-1).numpy()
    v = y[:, 2 * Hk * dk:].reshape(n, Hv, dv).numpy()
    out = np.zeros((n, Hv, dv))
    S = np.asarray(inp["S_c"], dtype=np.float64)
    for h in range(Hv):
        g = h // (Hv // Hk)
        o, _ = oracle.gdn_chain(S[0, h], q[:, g], k[:, g], v[:, h], inp["alpha"][:, h].astype(np.float64),
                                inp["beta"][:, h].astype(np.float64), scale)
        out[:, h] = o
    return out, q, k, v


def test_chain_matches_library_pipeline():
    n, W = 9, 4
    inp = synth.fused_inputs(0, (5,), n, W=W, dtype="f32", **SHAPE)
    out, q, k, v = oracle.tree_conv_gdn(synth.chain(n), inp["x"], inp["prefix"], inp["w"], inp["alpha"],
                                        inp["beta"], inp["S_c"], scale=0.5, **SHAPE)
    ro, rq, rk, rv = _library_chain(inp, scale=0.5, **SHAPE)
    np.testing.assert_allclose(q, rq, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(k, rk, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(v, rv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, ro, rtol=1e-5, atol=1e-6 * np.abs(ro).max())


def test_tree_node_equals_its_chain_and_states():
    n, W = 14, 4
    par = synth.random_tree(synth.rng_for(6, 2), n, 6)
    inp = synth.fused_inputs(6, (6,), n, W=W, dtype="bf16", **SHAPE)
    out, q, k, v, st = oracle.tree_conv_gdn(par, inp["x"], inp["prefix"], inp["w"], inp["alpha"], inp["beta"],
                                            inp["S_c"], want_states=True, **SHAPE)
    for i in range(n):
        path = oracle.root_path(par, i)
        oc, qc, kc, vc, sc = oracle.tree_conv_gdn(
            synth.chain(len(path)), inp["x"][path], inp["prefix"], inp["w"], inp["alpha"][path],
            inp["beta"][path], inp["S_c"], want_states=True, **SHAPE)
        np.testing.assert_array_equal(out[i], oc[-1])
        np.testing.assert_array_equal(k[i], kc[-1])
        np.testing.assert_array_equal(st[i], sc[-1])


def test_batched_sequences_use_their_own_prefix_and_state():
    trees = [synth.random_tree(synth.rng_for(8, b), nb, 4) for b, nb in enumerate([4, 6])]
    par, off = synth.concat_trees(trees)
    inp = synth.fused_inputs(8, (8,), len(par), W=4, dtype="f32", B=2, **SHAPE)
    out, q, k, v = oracle.tree_conv_gdn(par, inp["x"], inp["prefix"], inp["w"], inp["alpha"], inp["beta"],
                                        inp["S_c"], tree_off=off, **SHAPE)
    for b in range(2):
        o, e = off[b], off[b + 1]
        ob, qb, kb, vb = oracle.tree_conv_gdn(par[o:e], inp["x"][o:e], inp["prefix"][b:b + 1], inp["w"],
                                              inp["alpha"][o:e], inp["beta"][o:e], inp["S_c"][b:b + 1],
                                              **SHAPE)
        np.testing.assert_array_equal(out[o:e], ob)
        np.testing.assert_array_equal(v[o:e], vb)
