"""Pins for the oracle's tree gated delta-net (CPU only)."""
import numpy as np

import oracle
import synth
from oracle.num import f64


def _inp(n, Hk=2, Hv=4, d=8, seed=0, dtype="f32"):
    return synth.gdn_inputs(seed, (7,), n, Hk, Hv, d, d, dtype)


def test_tree_recurrence_equals_path_replay_bitwise():
    n = 22
    par = synth.random_tree(synth.rng_for(0, 5), n, 8)
    inp = _inp(n, dtype="bf16")
    a, sa = oracle.tree_gdn(par, **inp, want_states=True)
    b, sb = oracle.tree_gdn_recurrent(par, **inp)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_gates_identity():
    # alpha = 1, beta = 0: the state never changes, o = scale S_c q
    n = 7
    par = synth.binary_tree(3)
    inp = _inp(n)
    inp["alpha"][:] = 1
    inp["beta"][:] = 0
    out, st = oracle.tree_gdn(par, **inp, scale=0.5, want_states=True)
    S = f64(inp["S_c"])[0]
    q = f64(inp["q"])
    for i in range(n):
        for h in range(4):
            np.testing.assert_array_equal(st[i, h], S[h])
            np.testing.assert_allclose(out[i, h], 0.5 * S[h] @ q[i, h // 2], rtol=1e-13)


def test_delta_rule_writes_value_under_key():
    # beta = 1 and a unit key: the new state maps k to v for any alpha
    rng = np.random.default_rng(0)
    d = 16
    S = rng.standard_normal((d, d))
    k = rng.standard_normal(d)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(d)
    for a in (0.1, 0.7, 1.0):
        Sn, _ = oracle.gdn.gdn_step(S, k, k, v, a, 1.0)
        np.testing.assert_allclose(Sn @ k, v, rtol=1e-12, atol=1e-12)


def test_single_node_from_zero_state():
    inp = _inp(1)
    inp["S_c"][:] = 0
    out = oracle.tree_gdn([-1], **inp)
    q, k, v, b = f64(inp["q"])[0], f64(inp["k"])[0], f64(inp["v"])[0], f64(inp["beta"])[0]
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(out[0, h], b[h] * (k[g] @ q[g]) * v[h], rtol=1e-12)


def test_row_form_independent():
    # row-by-row delta update u = beta (v - alpha S k); S <- alpha S + u k^T
    n = 10
    par = synth.random_tree(synth.rng_for(2, 5), n, 5)
    inp = _inp(n, Hk=1, Hv=2, d=16, seed=2)
    out, st = oracle.tree_gdn(par, **inp, want_states=True)
    q, k, v, A, Bt, S0 = (f64(inp[x]) for x in ("q", "k", "v", "alpha", "beta", "S_c"))
    for i in range(n):
        for h in range(2):
            S = S0[0, h].copy()
            for t in oracle.root_path(par, i):
                kk = k[t, 0]
                for r in range(S.shape[0]):
                    u = Bt[t, h] * (v[t, h, r] - A[t, h] * (S[r] @ kk))
                    S[r] = A[t, h] * S[r] + u * kk
            np.testing.assert_allclose(st[i, h], S, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(out[i, h], S @ q[i, 0], rtol=1e-10, atol=1e-12)


def test_gqa_head_groups():
    # value heads 0,1 read key head 0 and 2,3 read key head 1: swapping the
    # key heads must swap which value-head pairs change
    n = 5
    par = synth.random_tree(synth.rng_for(3, 5), n, 4)
    inp = _inp(n, Hk=2, Hv=4, seed=3)
    out = oracle.tree_gdn(par, **inp)
    sw = dict(inp)
    sw["q"] = inp["q"][:, ::-1].copy()
    sw["k"] = inp["k"][:, ::-1].copy()
    sw["S_c"] = inp["S_c"][:, [2, 3, 0, 1]].copy()
    sw["v"] = inp["v"][:, [2, 3, 0, 1]].copy()
    sw["alpha"] = inp["alpha"][:, [2, 3, 0, 1]].copy()
    sw["beta"] = inp["beta"][:, [2, 3, 0, 1]].copy()
    out2 = oracle.tree_gdn(par, **sw)
    np.testing.assert_array_equal(out2, out[:, [2, 3, 0, 1]])


def test_batched_sequences_use_their_own_state():
    trees = [synth.random_tree(synth.rng_for(4, b), nb, 4) for b, nb in enumerate([4, 6])]
    par, off = synth.concat_trees(trees)
    inp = synth.gdn_inputs(4, (8,), len(par), 1, 2, 8, 8, "f32", B=2)
    out = oracle.tree_gdn(par, **inp, tree_off=off)
    for b in range(2):
        o, e = off[b], off[b + 1]
        sub = {k: (v[o:e] if k != "S_c" else v[b:b + 1]) for k, v in inp.items()}
        np.testing.assert_array_equal(out[o:e], oracle.tree_gdn(par[o:e], **sub))
