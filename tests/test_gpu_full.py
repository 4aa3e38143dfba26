"""Parity at the workloads' full sizes, on sampled outputs.

- The 128K stack (48 gated delta-net + conv layers, 16 attention layers,
  T = 131,072, 22-node tree) is built and stepped exactly as the benchmark
  does (same class, same context headroom, hence the same attention split
  configuration).  The first and last delta-net / conv layers are checked
  in full, attention rows are sampled in the first and last attention
  layers, the walk in full, and the commit on the checked layers.
- The batched workload (8 sequences, budgets from {8, 16, 22, 32, 64}, up to
  10 levels, contexts in [2048, 65536] over a shuffled paged cache) runs one
  layer of each kind, the walk over all trees and the commit; delta-net
  value heads 0 and 31 and two attention rows per sequence are checked.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import TOL, banner, dev, host, rel_err

pytestmark = pytest.mark.gpu


def u16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def hostin(t):
    return u16(t) if t.dtype == torch.bfloat16 else host(t)


def test_stack_128k_full_size_sampled(gpu):
    import bench
    banner("stack 48 gdn+conv / 16 attn, T=131072, N=22: sampled parity")
    st = bench.Stack(gpu, seed=0, headroom_steps=bench.headroom())  # the benchmark's default
    c = st.c
    N = c["N"]
    chk_g = [0, c["n_gdn"] - 1]
    chk_a = [0, c["n_attn"] - 1]
    pre = {l: dict(S_c=host(st.gdn[l]["S_c"]).copy(), prefix=u16(st.conv[l]["prefix"]).copy())
           for l in chk_g}
    T0 = int(st.T.item())
    st.step()
    torch.cuda.synchronize()
    assert not host(st.tb.status).any()
    par = st.parent
    ins = {}
    for l in chk_g:
        g = {k: hostin(v) for k, v in st.gdn[l].items()}
        g["S_c"] = pre[l]["S_c"]
        x = {k: u16(v) for k, v in st.conv[l].items()}
        x["prefix"] = pre[l]["prefix"]
        ins[l] = (g, x)
        assert rel_err(host(st.conv_out[l]), oracle.tree_conv(par, x["x"], x["prefix"], x["w"]), (0,)) < TOL
        assert rel_err(host(st.gdn_out[l]), oracle.tree_gdn(par, **g), (0, 1)) < TOL
    rng = np.random.default_rng(1)
    for l in chk_a:
        rows = [(int(i), int(h)) for i, h in zip(rng.integers(0, N, 6), rng.integers(0, c["Hq"], 6))]
        rows += [(N - 1, c["Hq"] - 1)]
        K, V = st.kv[l]
        a = {k: host(v) for k, v in st.attn[l].items()}
        # the commit only writes positions >= T0, so the first T0 are the inputs
        ref = oracle.tree_attn(par, a["q"], host(K), host(V), [T0], a["Kt"], a["Vt"], rows=rows)
        idx = tuple(np.array(rows).T)
        assert rel_err(host(st.attn_out[l])[idx], ref[idx], (0,)) < TOL
    am = oracle.argmax_rows(u16(st.logits))
    assert np.array_equal(host(st.amax), am)
    paths, L, bonus = oracle.accept_walk(par, host(st.tok), am)
    assert int(host(st.L)[0]) == L[0] and int(host(st.bonus)[0]) == bonus[0]
    assert list(host(st.path)[0][:L[0]]) == list(paths[0])
    assert int(st.T.item()) == T0 + L[0]
    pg = list(paths[0])
    for l in chk_g:
        g, x = ins[l]
        S_ref = oracle.commit_gdn_state(g["S_c"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], pg, 0)
        assert rel_err(host(st.gdn[l]["S_c"])[0], S_ref, (0,)) < TOL
        pre_ref = oracle.commit_conv_prefix(x["prefix"], x["x"], pg, 0)
        assert np.array_equal(oracle.num.f64(u16(st.conv[l]["prefix"]))[0], pre_ref)
    for l in chk_a:
        K, V = st.kv[l]
        a = st.attn[l]
        for r, node in enumerate(pg):
            t = T0 + r
            assert torch.equal(K[t // 16, :, t % 16, :], a["Kt"][node])
            assert torch.equal(V[t // 16, :, :, t % 16], a["Vt"][node])


def test_stack_128k_fused_full_size_sampled(gpu):
    """The benchmark's headline step: each linear-attention layer as one
    fused conv -> delta-net call, at full size; sampled layers against the
    fused oracle, the walk, and the commit of their state and prefix."""
    import bench
    banner("stack 48 fused conv->gdn / 16 attn, T=131072, N=22 (the benchmark's step): sampled parity")
    st = bench.Stack(gpu, seed=0, headroom_steps=bench.headroom())
    st.setup_fused()
    st.fused_step = True
    c = st.c
    chk_g = [0, c["n_gdn"] - 1]
    pre = {l: dict(S_c=host(st.gdn[l]["S_c"]).copy(), prefix=u16(st.conv[l]["prefix"]).copy())
           for l in chk_g}
    T0 = int(st.T.item())
    st.step()
    torch.cuda.synchronize()
    assert not host(st.tb.status).any()
    par = st.parent
    refs = {}
    for l in chk_g:
        x = {k: u16(v) for k, v in st.conv[l].items()}
        x["prefix"] = pre[l]["prefix"]
        f = st.fz[l]
        al, be = host(f["alpha"]), host(f["beta"])
        out, q, k, v = oracle.tree_conv_gdn(par, x["x"], x["prefix"], x["w"], al, be, pre[l]["S_c"],
                                            c["Hk"], c["Hv"], c["dk"], c["dv"])
        assert rel_err(host(st.gdn_out[l]), out, (0, 1)) < TOL
        assert rel_err(host(f["k"]), k, (0, 1)) < TOL  # the keys handed to the commit
        refs[l] = (x, q, k, v, al, be)
    am = oracle.argmax_rows(u16(st.logits))
    assert np.array_equal(host(st.amax), am)
    paths, L, bonus = oracle.accept_walk(par, host(st.tok), am)
    assert int(host(st.L)[0]) == L[0] and int(host(st.bonus)[0]) == bonus[0]
    assert int(st.T.item()) == T0 + L[0]
    pg = list(paths[0])
    for l in chk_g:
        x, q, k, v, al, be = refs[l]
        S_ref = oracle.commit_gdn_state(pre[l]["S_c"], q, k, v, al, be, pg, 0)
        assert rel_err(host(st.gdn[l]["S_c"])[0], S_ref, (0,)) < TOL
        pre_ref = oracle.commit_conv_prefix(x["prefix"], x["x"], pg, 0)
        assert np.array_equal(oracle.num.f64(u16(st.conv[l]["prefix"]))[0], pre_ref)


def test_batched_full_size_sampled(gpu):
    banner("batched 8 sequences, paged, budgets {8..64}, T in [2K, 64K]: sampled parity")
    cfg = synth.BATCHED
    trees, T = synth.batched_trees(0)
    par, off = synth.concat_trees(trees)
    n, B = len(par), len(trees)
    sizes = [len(t) for t in trees]
    tb = ddt.TreeBatch(par, off, cfg["W"], gpu)
    ddt.ddt_tree_plan(tb, cfg["levels"])
    Hk, Hv, dk, C, W = cfg["Hk"], cfg["Hv"], cfg["dk"], cfg["C"], cfg["W"]
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    gi = synth.gdn_inputs(0, (4, 1), n, Hk, Hv, dk, cfg["dv"], "bf16", B=B)
    ci = synth.conv_inputs(0, (4, 2), n, C, W, "bf16", B=B)
    pt, P = synth.page_layout(0, (4, 3), T, sizes)
    Kp, Vp = synth.kv_pool(0, (4, 3), P, Hkv, D, "f16")
    ai = synth.attn_inputs(0, (4, 4), n, Hq, Hkv, D, "f16")
    lg, tok = [], []
    for b, t in enumerate(trees):
        l_, t_ = synth.logits_and_draft(0, (4, 5, b), t, synth.VOCAB, "bf16", p_match=0.8)
        lg.append(l_)
        tok.append(t_)
    lg, tok = np.concatenate(lg), np.concatenate(tok).astype(np.int32)
    g = {k: dev(v) for k, v in gi.items()}
    x = {k: dev(v) for k, v in ci.items()}
    a = {k: dev(v) for k, v in ai.items()}
    K, V, ptd = dev(Kp), dev(Vp), dev(pt)
    Td = dev(T.astype(np.int32))
    T_max = int(T.max())
    y = torch.empty(n, C, dtype=torch.float32, device=gpu)
    o = torch.empty(n, Hv, cfg["dv"], dtype=torch.float32, device=gpu)
    nu = torch.empty_like(o)
    oa = torch.empty(n, Hq, D, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_conv(tb, x["x"], x["prefix"], x["w"], 0, y)
    ddt.ddt_tree_gdn(tb, g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S_c"], 1.0, o, None, nu)
    ws = torch.empty(ddt.ddt_tree_attn_workspace(tb, Hq, Hkv, D, T_max), dtype=torch.uint8, device=gpu)
    ddt.ddt_tree_attn(tb, a["q"], K, V, ptd, Td, T_max, a["Kt"], a["Vt"], oa, ws)
    wws = torch.empty(ddt.ddt_accept_walk_workspace(tb, synth.VOCAB), dtype=torch.uint8, device=gpu)
    i32 = dict(dtype=torch.int32, device=gpu)
    am, path, L, bonus = (torch.empty(n, **i32), torch.empty(B, tb.n_max, **i32), torch.empty(B, **i32),
                          torch.empty(B, **i32))
    ddt.ddt_accept_walk(tb, dev(lg), dev(tok), am, path, L, bonus, wws)
    gl = [ddt.GdnLayer(q=g["q"].data_ptr(), k=g["k"].data_ptr(), v=g["v"].data_ptr(),
                       alpha=g["alpha"].data_ptr(), beta=g["beta"].data_ptr(), S_c=g["S_c"].data_ptr(),
                       node_u=nu.data_ptr(), x=x["x"].data_ptr(), prefix=x["prefix"].data_ptr())]
    al = [ddt.AttnLayer(a["Kt"].data_ptr(), a["Vt"].data_ptr(), K.data_ptr(), V.data_ptr())]
    ddt.ddt_commit_state(tb, path, L, ddt.DDT_COMMIT_UPDATE, ddt.layer_table(gl, gpu), 1, Hk, Hv, dk,
                         cfg["dv"], ddt.DDT_BF16, C, ddt.DDT_BF16, ddt.layer_table(al, gpu), 1, Hkv, D,
                         ddt.DDT_F16, ptd, Td)
    torch.cuda.synchronize()
    assert not host(tb.status).any()
    # layer outputs
    assert rel_err(host(y), oracle.tree_conv(par, ci["x"], ci["prefix"], ci["w"], tree_off=off), (0,)) < TOL
    heads, kheads = [0, Hv - 1], [0, (Hv - 1) // (Hv // Hk)]
    sub = dict(q=gi["q"][:, kheads], k=gi["k"][:, kheads], v=gi["v"][:, heads], alpha=gi["alpha"][:, heads],
               beta=gi["beta"][:, heads], S_c=gi["S_c"][:, heads])
    assert rel_err(host(o)[:, heads], oracle.tree_gdn(par, **sub, tree_off=off), (0, 1)) < TOL
    rng = np.random.default_rng(2)
    rows = []
    for b in range(B):
        for _ in range(2):
            rows.append((int(off[b] + rng.integers(0, sizes[b])), int(rng.integers(0, Hq))))
    ref = oracle.tree_attn(par, ai["q"], Kp, Vp, T, ai["Kt"], ai["Vt"], page_table=pt, tree_off=off, rows=rows)
    idx = tuple(np.array(rows).T)
    assert rel_err(host(oa)[idx], ref[idx], (0,)) < TOL
    # walk
    amr = oracle.argmax_rows(lg)
    assert np.array_equal(host(am), amr)
    paths, Lr, br = oracle.accept_walk(par, tok, amr, tree_off=off)
    assert np.array_equal(host(L), Lr) and np.array_equal(host(bonus), br)
    assert np.array_equal(host(Td), T + Lr)
    # commit
    S_new = host(g["S_c"])
    pre_new = oracle.num.f64(u16(x["prefix"]))
    Kh, Vh = host(K), host(V)
    for b in range(B):
        pgl = [off[b] + j for j in paths[b]]
        S_ref = oracle.commit_gdn_state(sub["S_c"], sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"],
                                        pgl, b)
        assert rel_err(S_new[b][heads], S_ref, (0,)) < TOL
        assert np.array_equal(pre_new[b], oracle.commit_conv_prefix(ci["prefix"], ci["x"], pgl, b))
        for r, node in enumerate(pgl):
            t = int(T[b]) + r
            page = int(pt[b][t // 16])
            assert np.array_equal(Kh[page, :, t % 16, :].view(np.uint16), ai["Kt"][node].view(np.uint16))
            assert np.array_equal(Vh[page, :, :, t % 16].view(np.uint16), ai["Vt"][node].view(np.uint16))
