"""Pins for the oracle's tree attention (CPU only)."""
import numpy as np
import torch

import oracle
import synth
from oracle.num import f64


def _setup(seed, n, T, Hq=4, Hkv=2, D=16, par=None, shuffle=True):
    par = synth.random_tree(synth.rng_for(seed, 1), n, 5) if par is None else par
    pt, P = synth.page_layout(seed, (2,), [T], [n], shuffle=shuffle)
    K, V = synth.kv_pool(seed, (2,), P, Hkv, D, "f32")
    a = synth.attn_inputs(seed, (2,), n, Hq, Hkv, D, "f32")
    return par, pt, K, V, a


def _sdpa_chain(q, Kc, Vc, Kt, Vt, grp):
    """torch SDPA for a chain: row i sees the cache and chain tokens 0..i."""
    n, Hq, D = q.shape
    T = Kc.shape[1]
    keys = torch.cat([torch.tensor(Kc), torch.tensor(Kt).permute(1, 0, 2)], 1)   # [Hkv][T+n][D]
    vals = torch.cat([torch.tensor(Vc), torch.tensor(Vt).permute(1, 0, 2)], 1)
    keys = keys.repeat_interleave(grp, 0)
    vals = vals.repeat_interleave(grp, 0)
    mask = torch.ones(n, T + n, dtype=torch.bool)
    mask[:, T:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).permute(1, 0, 2), keys, vals, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


def test_chain_without_cache_is_causal_sdpa():
    n, Hq, Hkv, D = 9, 4, 2, 16
    par, pt, K, V, a = _setup(0, n, 0, Hq, Hkv, D, par=synth.chain(n))
    o = oracle.tree_attn(par, a["q"], K, V, [0], a["Kt"], a["Vt"], page_table=pt)
    ref = _sdpa_chain(f64(a["q"]), np.zeros((Hkv, 0, D)), np.zeros((Hkv, 0, D)),
                      f64(a["Kt"]), f64(a["Vt"]), Hq // Hkv)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_chain_with_cache_is_masked_sdpa():
    n, T, Hq, Hkv, D = 6, 37, 6, 2, 16
    par, pt, K, V, a = _setup(1, n, T, Hq, Hkv, D, par=synth.chain(n))
    o = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt)
    Kc = np.stack([oracle.gather_cache(K, V, pt, 0, g, T)[0] for g in range(Hkv)])
    Vc = np.stack([oracle.gather_cache(K, V, pt, 0, g, T)[1] for g in range(Hkv)])
    ref = _sdpa_chain(f64(a["q"]), Kc, Vc, f64(a["Kt"]), f64(a["Vt"]), Hq // Hkv)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_page_gather_reads_the_right_slots():
    # write token t's key as the constant t; the gather must return t in order
    T, Hkv, D = 53, 2, 4
    pt, P = synth.page_layout(5, (3,), [T], [0], shuffle=True)
    K = np.zeros((P, Hkv, 16, D), np.float32)
    V = np.zeros((P, Hkv, D, 16), np.float32)
    for t in range(T):
        K[pt[0][t // 16], :, t % 16, :] = t
        V[pt[0][t // 16], :, :, t % 16] = -t
    for g in range(Hkv):
        Kc, Vc = oracle.gather_cache(K, V, pt, 0, g, T)
        np.testing.assert_array_equal(Kc[:, 0], np.arange(T))
        np.testing.assert_array_equal(Vc[:, 3], -np.arange(T))


def test_single_node_no_cache_returns_its_value():
    par, pt, K, V, a = _setup(2, 1, 0, par=np.array([-1]))
    o = oracle.tree_attn(par, a["q"], K, V, [0], a["Kt"], a["Vt"], page_table=pt)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], f64(a["Vt"])[0, h // 2], rtol=1e-14)


def test_equal_keys_average_visible_values():
    n, T = 7, 20
    par, pt, K, V, a = _setup(3, n, T, par=synth.binary_tree(3))
    K[:] = 0.25
    a["Kt"][:] = 0.25
    o = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt)
    for i in range(n):
        path = oracle.root_path(par, i)
        for h in range(4):
            g = h // 2
            Vc = oracle.gather_cache(K, V, pt, 0, g, T)[1]
            allv = np.concatenate([Vc, f64(a["Vt"])[path, g]], 0)
            np.testing.assert_allclose(o[i, h], allv.mean(0), rtol=1e-12)


def test_permutation_invariances():
    n, T = 10, 45
    par, pt, K, V, a = _setup(4, n, T, shuffle=False)
    o = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt)
    o_none = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=None)
    np.testing.assert_array_equal(o, o_none)            # consecutive pages == no table
    perm = np.random.default_rng(0).permutation(K.shape[0])
    K2, V2 = np.empty_like(K), np.empty_like(V)
    K2[perm], V2[perm] = K, V                            # page p moves to perm[p]
    o2 = oracle.tree_attn(par, a["q"], K2, V2, [T], a["Kt"], a["Vt"], page_table=perm[pt])
    np.testing.assert_array_equal(o2, o)
    # permuting the committed tokens themselves leaves the result unchanged
    Kc = np.stack([oracle.gather_cache(K, V, pt, 0, g, T)[0] for g in range(2)])
    Vc = np.stack([oracle.gather_cache(K, V, pt, 0, g, T)[1] for g in range(2)])
    tp = np.random.default_rng(1).permutation(T)
    K3, V3 = K.copy(), V.copy()
    for t in range(T):
        K3[pt[0][t // 16], :, t % 16] = Kc[:, tp[t]]
        V3[pt[0][t // 16], :, :, t % 16] = Vc[:, tp[t]]
    o3 = oracle.tree_attn(par, a["q"], K3, V3, [T], a["Kt"], a["Vt"], page_table=pt)
    np.testing.assert_allclose(o3, o, rtol=1e-12, atol=1e-14)


def test_tree_node_equals_its_chain():
    n, T = 12, 30
    par, pt, K, V, a = _setup(5, n, T)
    o = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt)
    for i in range(n):
        path = oracle.root_path(par, i)
        oc = oracle.tree_attn(synth.chain(len(path)), a["q"][path], K, V, [T],
                              a["Kt"][path], a["Vt"][path], page_table=pt)
        np.testing.assert_allclose(o[i], oc[-1], rtol=1e-12, atol=1e-14)


def test_row_subset():
    n, T = 8, 19
    par, pt, K, V, a = _setup(6, n, T)
    full = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt)
    rows = [(3, 1), (7, 2)]
    sub = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], page_table=pt, rows=rows)
    for i, h in rows:
        np.testing.assert_allclose(sub[i, h], full[i, h], rtol=1e-13)


# ---- 8-bit cache (dequantisation in front of the same attention)
def test_q8_dequant_hand_values():
    """Codes times a power-of-two scale are exact; 3 * fp16(0.1) lies exactly
    halfway between two fp16 neighbours and rounds to the even one."""
    Kq = np.array([-127, -1, 0, 1, 127], np.int8).reshape(1, 1, 1, 5)
    Ksc = np.array([0.5], np.float16).reshape(1, 1, 1)
    Vq = np.array([3], np.int8).reshape(1, 1, 1, 1)
    Vsc = np.array([0.1], np.float16).reshape(1, 1, 1)  # 0.0999755859375
    K, V = oracle.dequant_q8(Kq, Ksc, Vq, Vsc)
    assert K.dtype == np.float16 and V.dtype == np.float16
    assert K.ravel().tolist() == [-63.5, -0.5, 0.0, 0.5, 63.5]
    # 3 * 0.0999755859375 = 0.2999267578125 = 1228.5 * 2**-12: ties to 1228 * 2**-12
    assert float(V.ravel()[0]) == 1228 * 2.0 ** -12


def test_q8_dequant_scales_follow_tokens():
    """One scale per token: K row t and V column t of a page take token t's
    scale (distinct powers of two, so every product is exact)."""
    P, H, D = 2, 2, 4
    Kq = np.arange(P * H * 16 * D).reshape(P, H, 16, D).astype(np.int64) % 7 - 3
    Vq = np.arange(P * H * D * 16).reshape(P, H, D, 16).astype(np.int64) % 5 - 2
    Ksc = (2.0 ** -(np.arange(P * H * 16).reshape(P, H, 16) % 8)).astype(np.float16)
    Vsc = (2.0 ** -((np.arange(P * H * 16).reshape(P, H, 16) + 3) % 8)).astype(np.float16)
    K, V = oracle.dequant_q8(Kq.astype(np.int8), Ksc, Vq.astype(np.int8), Vsc)
    for p in range(P):
        for h in range(H):
            for t in range(16):
                assert (K[p, h, t, :].astype(np.float64) == Kq[p, h, t, :] * float(Ksc[p, h, t])).all()
                assert (V[p, h, :, t].astype(np.float64) == Vq[p, h, :, t] * float(Vsc[p, h, t])).all()
