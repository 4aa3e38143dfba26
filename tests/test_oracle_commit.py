"""Pins for the oracle's commit: committing a path and then processing one
more token must equal processing the whole sequence as a chain (CPU only)."""
import numpy as np

import oracle
import synth
from oracle.num import f64


def _path_and_next(par):
    # the deepest node's path, then a fresh node appended as its child
    d = oracle.depth(par)
    last = int(np.argmax(d))
    return oracle.root_path(par, last)


def test_gdn_commit_then_step_equals_chain():
    n = 14
    par = synth.random_tree(synth.rng_for(0, 1), n, 6)
    inp = synth.gdn_inputs(0, (3,), n + 1, 2, 4, 8, 8, "f32")
    path = _path_and_next(par)
    S_new = oracle.commit.commit_gdn_state(inp["S_c"], inp["q"], inp["k"], inp["v"],
                                           inp["alpha"], inp["beta"], path, 0)
    nxt = n   # the extra generated node plays the next step's root
    one = {k: v[[nxt]] for k, v in inp.items() if k != "S_c"}
    o1 = oracle.tree_gdn([-1], **one, S_c=S_new[None])
    seq = path + [nxt]
    sub = {k: v[seq] for k, v in inp.items() if k != "S_c"}
    oc = oracle.tree_gdn(synth.chain(len(seq)), **sub, S_c=inp["S_c"])
    np.testing.assert_allclose(o1[0], oc[-1], rtol=1e-11, atol=1e-12)
    # L = 1 (root only) is one chain step
    S1 = oracle.commit.commit_gdn_state(inp["S_c"], inp["q"], inp["k"], inp["v"],
                                        inp["alpha"], inp["beta"], [0], 0)
    _, st = oracle.tree_gdn([-1], **{k: v[[0]] for k, v in inp.items() if k != "S_c"},
                            S_c=inp["S_c"], want_states=True)
    np.testing.assert_array_equal(S1, st[0])


def test_conv_commit_then_step_equals_chain():
    n, C, W = 14, 8, 4
    par = synth.random_tree(synth.rng_for(1, 1), n, 6)
    inp = synth.conv_inputs(1, (3,), n + 1, C, W, "bf16")
    for path in (_path_and_next(par), [0], [0, int(np.nonzero(par == 0)[0][0])]):
        pre = oracle.commit.commit_conv_prefix(inp["prefix"], inp["x"], path, 0)
        y1 = oracle.tree_conv([-1], inp["x"][[n]], pre[None], inp["w"])
        seq = path + [n]
        yc = oracle.tree_conv(synth.chain(len(seq)), inp["x"][seq], inp["prefix"], inp["w"])
        np.testing.assert_allclose(y1[0], yc[-1], rtol=1e-12, atol=1e-12)


def test_kv_commit_then_step_equals_chain():
    n, T, Hq, Hkv, D = 12, 29, 4, 2, 16
    par = synth.random_tree(synth.rng_for(2, 1), n, 6)
    pt, P = synth.page_layout(2, (4,), [T], [n + 1])
    K, V = synth.kv_pool(2, (4,), P, Hkv, D, "f16")
    a = synth.attn_inputs(2, (4,), n + 1, Hq, Hkv, D, "f16")
    path = _path_and_next(par)
    K2, V2, T2 = oracle.commit.commit_kv(K, V, pt, [T], a["Kt"], a["Vt"], path, 0)
    assert T2 == T + len(path)
    o1 = oracle.tree_attn([-1], a["q"][[n]], K2, V2, [T2], a["Kt"][[n]], a["Vt"][[n]], page_table=pt)
    seq = path + [n]
    oc = oracle.tree_attn(synth.chain(len(seq)), a["q"][seq], K, V, [T], a["Kt"][seq], a["Vt"][seq],
                          page_table=pt)
    np.testing.assert_allclose(o1[0], oc[-1], rtol=1e-11, atol=1e-13)
    # the appended values are the draft values, bit for bit
    for r, node in enumerate(path):
        t = T + r
        assert np.array_equal(K2[pt[0][t // 16], :, t % 16], a["Kt"][node])
        assert np.array_equal(V2[pt[0][t // 16], :, :, t % 16], a["Vt"][node])
