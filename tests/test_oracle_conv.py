"""Pins for the oracle's tree conv (CPU only)."""
import numpy as np
import torch

import oracle
import synth


def _chain_torch(prefix, x, w):
    # depthwise causal conv1d over prefix ++ x via torch (cross-correlation:
    # out[t] = sum_k w[k] in[t+k], so tap W-1 meets the newest token)
    C, W = w.shape
    seq = torch.tensor(np.concatenate([prefix, x], 0).T[None])          # [1][C][L]
    out = torch.nn.functional.conv1d(seq, torch.tensor(w)[:, None, :], groups=C)
    return out[0].T.numpy()                                              # [n][C]


def test_chain_equals_torch_conv1d():
    n, C, W = 9, 24, 4
    inp = synth.conv_inputs(0, (1,), n, C, W, "f32")
    y = oracle.tree_conv(synth.chain(n), inp["x"], inp["prefix"], inp["w"])
    ref = _chain_torch(inp["prefix"][0].astype(np.float64), inp["x"].astype(np.float64),
                       inp["w"].astype(np.float64))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_identity_and_oldest_taps():
    par = synth.random_tree(synth.rng_for(1, 2), 12, 5)
    C, W = 8, 4
    inp = synth.conv_inputs(1, (2,), 12, C, W, "f32")
    w = np.zeros((C, W), np.float32)
    w[:, W - 1] = 1
    np.testing.assert_array_equal(oracle.tree_conv(par, inp["x"], inp["prefix"], w), inp["x"])
    w = np.zeros((C, W), np.float32)
    w[:, 0] = 1            # tap 0: the token W-1 steps back; for the root that is the oldest prefix slot
    y = oracle.tree_conv(par, inp["x"], inp["prefix"], w)
    np.testing.assert_array_equal(y[0], inp["prefix"][0, 0])


def test_tree_node_equals_its_chain_and_silu():
    n, C, W = 16, 8, 4
    par = synth.random_tree(synth.rng_for(3, 3), n, 6)
    inp = synth.conv_inputs(3, (3,), n, C, W, "bf16")
    y = oracle.tree_conv(par, inp["x"], inp["prefix"], inp["w"])
    ys = oracle.tree_conv(par, inp["x"], inp["prefix"], inp["w"], act=1)
    np.testing.assert_allclose(ys, torch.nn.functional.silu(torch.tensor(y)).numpy(), rtol=1e-12)
    for i in range(n):
        path = oracle.root_path(par, i)
        yc = oracle.tree_conv(synth.chain(len(path)), inp["x"][path], inp["prefix"], inp["w"])
        np.testing.assert_array_equal(y[i], yc[-1])


def test_batched_offsets():
    trees = [synth.random_tree(synth.rng_for(4, b), nb, 4) for b, nb in enumerate([3, 7, 1])]
    par, off = synth.concat_trees(trees)
    C, W = 8, 4
    inp = synth.conv_inputs(4, (4,), len(par), C, W, "f32", B=3)
    y = oracle.tree_conv(par, inp["x"], inp["prefix"], inp["w"], tree_off=off)
    for b in range(3):
        o, e = off[b], off[b + 1]
        yb = oracle.tree_conv(par[o:e], inp["x"][o:e], inp["prefix"][b:b + 1], inp["w"])
        np.testing.assert_array_equal(y[o:e], yb)
