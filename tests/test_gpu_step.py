"""A whole verify step on the GPU through the C ABI -- plan, conv, gated
delta-net, attention, accept walk, commit -- checked against the oracle,
including REPLAY == SELECT bitwise and commit-then-next-step semantics."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import TOL, banner, dev, host, rel_err

pytestmark = pytest.mark.gpu

Hk, Hv, dk, C, W = 2, 4, 128, 256, 4
Hq, Hkv, D = 12, 2, 256
V = 5000


def build_step(gpu, seed, sizes, T, n_gdn=2, n_attn=1):
    trees = [synth.random_tree(synth.rng_for(seed, 80, b), s, 10) for b, s in enumerate(sizes)]
    par, off = synth.concat_trees(trees)
    n, B = len(par), len(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    st = dict(trees=trees, par=par, off=off, tb=tb, n=n, B=B, T=np.asarray(T, np.int64))
    st["gdn"] = [synth.gdn_inputs(seed, (81, l), n, Hk, Hv, dk, dk, "bf16", B=B) for l in range(n_gdn)]
    st["conv"] = [synth.conv_inputs(seed, (82, l), n, C, W, "bf16", B=B) for l in range(n_gdn)]
    pt, P = synth.page_layout(seed, (83,), T, sizes)
    st["pt"] = pt
    st["kv"] = [synth.kv_pool(seed, (84, l), P, Hkv, D, "f16") for l in range(n_attn)]
    st["attn"] = [synth.attn_inputs(seed, (85, l), n, Hq, Hkv, D, "f16") for l in range(n_attn)]
    lg, tok = [], []
    for b, t in enumerate(trees):
        l_, t_ = synth.logits_and_draft(seed, (86, b), t, V, "bf16", p_match=0.9)
        lg.append(l_)
        tok.append(t_)
    st["logits"], st["tok"] = np.concatenate(lg), np.concatenate(tok).astype(np.int32)
    return st


def run_step(gpu, st, mode):
    tb, n, B = st["tb"], st["n"], st["B"]
    d = {}
    d["gdn"] = [{k: dev(v) for k, v in g.items()} for g in st["gdn"]]
    d["conv"] = [{k: dev(v) for k, v in c.items()} for c in st["conv"]]
    d["kv"] = [(dev(K), dev(Vv)) for K, Vv in st["kv"]]
    d["attn"] = [{k: dev(v) for k, v in a.items()} for a in st["attn"]]
    pt = dev(st["pt"])
    T = dev(st["T"].astype(np.int32))
    T_max = int(st["T"].max())
    ddt.ddt_tree_plan(tb, 10)
    outs = dict(conv=[], gdn=[], attn=[])
    ns = []
    for l, (g, c) in enumerate(zip(d["gdn"], d["conv"])):
        y = torch.empty(n, C, dtype=torch.float32, device=gpu)
        ddt.ddt_tree_conv(tb, c["x"], c["prefix"], c["w"], 0, y)
        o = torch.empty(n, Hv, dk, dtype=torch.float32, device=gpu)
        nsl = (torch.empty(n, Hv, dk, dk, dtype=torch.float32, device=gpu)
               if mode == ddt.DDT_COMMIT_SELECT else None)
        nul = torch.empty(n, Hv, dk, dtype=torch.float32, device=gpu) if mode == ddt.DDT_COMMIT_UPDATE else None
        ddt.ddt_tree_gdn(tb, g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S_c"], 1.0, o, nsl, nul)
        outs["conv"].append(y)
        outs["gdn"].append(o)
        ns.append((nsl, nul))
    ws = torch.empty(ddt.ddt_tree_attn_workspace(tb, Hq, Hkv, D, T_max), dtype=torch.uint8, device=gpu)
    for (K, Vv), a in zip(d["kv"], d["attn"]):
        o = torch.empty(n, Hq, D, dtype=torch.float32, device=gpu)
        ddt.ddt_tree_attn(tb, a["q"], K, Vv, pt, T, T_max, a["Kt"], a["Vt"], o, ws)
        outs["attn"].append(o)
    wws = torch.empty(ddt.ddt_accept_walk_workspace(tb, V), dtype=torch.uint8, device=gpu)
    am = torch.empty(n, dtype=torch.int32, device=gpu)
    path = torch.empty(B, tb.n_max, dtype=torch.int32, device=gpu)
    L = torch.empty(B, dtype=torch.int32, device=gpu)
    bonus = torch.empty(B, dtype=torch.int32, device=gpu)
    ddt.ddt_accept_walk(tb, dev(st["logits"]), dev(st["tok"]), am, path, L, bonus, wws)
    ptr = lambda t: t.data_ptr() if t is not None else None
    gl = [ddt.GdnLayer(q=g["q"].data_ptr(), k=g["k"].data_ptr(), v=g["v"].data_ptr(),
                       alpha=g["alpha"].data_ptr(), beta=g["beta"].data_ptr(), S_c=g["S_c"].data_ptr(),
                       node_states=ptr(ns[l][0]), node_u=ptr(ns[l][1]), x=c["x"].data_ptr(),
                       prefix=c["prefix"].data_ptr())
          for l, (g, c) in enumerate(zip(d["gdn"], d["conv"]))]
    al = [ddt.AttnLayer(a["Kt"].data_ptr(), a["Vt"].data_ptr(), K.data_ptr(), Vv.data_ptr())
          for (K, Vv), a in zip(d["kv"], d["attn"])]
    gt, at = ddt.layer_table(gl, gpu), ddt.layer_table(al, gpu)
    ddt.ddt_commit_state(tb, path, L, mode, gt, len(gl), Hk, Hv, dk, dk, ddt.DDT_BF16, C, ddt.DDT_BF16,
                         at, len(al), Hkv, D, ddt.DDT_F16, pt, T)
    torch.cuda.synchronize()
    return d, outs, dict(am=host(am), path=host(path), L=host(L), bonus=host(bonus), T=host(T),
                         status=host(tb.status))


@pytest.mark.parametrize("seed,mode", [(0, 0), (1, 2)])
def test_step_against_oracle(gpu, seed, mode):
    banner(f"step seed={seed} commit mode={mode}")
    sizes = [22, 8, 33]
    T = [700, 1000, 64]
    st = build_step(gpu, seed, sizes, T)
    d, outs, res = run_step(gpu, st, mode)
    par, off = st["par"], st["off"]
    assert not res["status"].any()
    for l in range(len(st["gdn"])):
        c = st["conv"][l]
        assert rel_err(host(outs["conv"][l]), oracle.tree_conv(par, c["x"], c["prefix"], c["w"], tree_off=off), (0,)) < TOL
        assert rel_err(host(outs["gdn"][l]), oracle.tree_gdn(par, **st["gdn"][l], tree_off=off), (0, 1)) < TOL
    for l, ((K, Vv), a) in enumerate(zip(st["kv"], st["attn"])):
        ref = oracle.tree_attn(par, a["q"], K, Vv, st["T"], a["Kt"], a["Vt"], page_table=st["pt"], tree_off=off)
        assert rel_err(host(outs["attn"][l]), ref, (0, 1)) < TOL
    am = oracle.argmax_rows(st["logits"])
    assert np.array_equal(res["am"], am)
    paths, L, bonus = oracle.accept_walk(par, st["tok"], am, tree_off=off)
    assert np.array_equal(res["L"], L) and np.array_equal(res["bonus"], bonus)
    assert np.array_equal(res["T"], st["T"] + L)
    # committed state, prefix and cache of every sequence
    for b in range(st["B"]):
        pg = [off[b] + j for j in paths[b]]
        for l in range(len(st["gdn"])):
            g = st["gdn"][l]
            S_ref = oracle.commit_gdn_state(g["S_c"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], pg, b)
            assert rel_err(host(d["gdn"][l]["S_c"])[b], S_ref, (0,)) < TOL
            c = st["conv"][l]
            pre = oracle.commit_conv_prefix(c["prefix"], c["x"], pg, b)
            assert np.array_equal(oracle.num.f64(host(d["conv"][l]["prefix"].view(torch.int16)).view(np.uint16))[b], pre)
        for l, ((K, Vv), a) in enumerate(zip(st["kv"], st["attn"])):
            K2, V2, _ = oracle.commit_kv(K, Vv, st["pt"], st["T"], a["Kt"], a["Vt"], pg, b)
            K, Vv = K2, V2
            st["kv"][l] = (K, Vv)
    for l in range(len(st["kv"])):
        assert np.array_equal(host(d["kv"][l][0]).view(np.uint16), st["kv"][l][0].view(np.uint16))
        assert np.array_equal(host(d["kv"][l][1]).view(np.uint16), st["kv"][l][1].view(np.uint16))


def test_commit_modes_agree_bitwise(gpu):
    banner("commit replay == select == update")
    st = build_step(gpu, 3, [22, 64, 5], [300, 40, 999])
    d1, _, r1 = run_step(gpu, st, ddt.DDT_COMMIT_REPLAY)
    d2, _, r2 = run_step(gpu, st, ddt.DDT_COMMIT_SELECT)
    d3, _, r3 = run_step(gpu, st, ddt.DDT_COMMIT_UPDATE)
    assert np.array_equal(r1["L"], r2["L"]) and np.array_equal(r1["L"], r3["L"]) and (r1["L"] >= 1).all()
    assert (r1["L"] > 1).any()
    for l in range(len(st["gdn"])):
        assert torch.equal(d1["gdn"][l]["S_c"], d2["gdn"][l]["S_c"])
        assert torch.equal(d1["gdn"][l]["S_c"], d3["gdn"][l]["S_c"])
        assert torch.equal(d1["conv"][l]["prefix"], d2["conv"][l]["prefix"])


def test_step_is_deterministic_and_batch_independent(gpu):
    banner("step determinism / batch independence")
    st = build_step(gpu, 4, [22, 16], [500, 2000])
    _, o1, r1 = run_step(gpu, st, 0)
    _, o2, r2 = run_step(gpu, st, 0)
    for k in ("conv", "gdn", "attn"):
        for a, b in zip(o1[k], o2[k]):
            assert torch.equal(a, b)
    # sequence 1 alone gives the same outputs as inside the batch
    solo = build_step(gpu, 4, [22, 16], [500, 2000])
    o, e = solo["off"][1], solo["off"][2]
    tree1 = solo["trees"][1]
    one = dict(solo)
    one["trees"] = [tree1]
    one["par"], one["off"] = synth.concat_trees([tree1])
    one["tb"] = ddt.TreeBatch(one["par"], one["off"], W, gpu)
    one["n"], one["B"] = len(tree1), 1
    one["T"] = solo["T"][1:]
    one["gdn"] = [{k: (v[o:e] if k != "S_c" else v[1:2]) for k, v in g.items()} for g in solo["gdn"]]
    one["conv"] = [{k: (v[o:e] if k == "x" else (v[1:2] if k == "prefix" else v)) for k, v in c.items()}
                   for c in solo["conv"]]
    one["attn"] = [{k: v[o:e] for k, v in a.items()} for a in solo["attn"]]
    one["pt"] = solo["pt"][1:2]
    one["logits"], one["tok"] = solo["logits"][o:e], solo["tok"][o:e]
    _, o3, r3 = run_step(gpu, one, 0)
    for k in ("conv", "gdn"):
        for a, b in zip(o1[k], o3[k]):
            assert torch.equal(a[o:e], b)
    # attention: in a batch the sequences share a pool of context splits,
    # dealt in proportion to each one's tiles, so sequence 1's split bounds
    # depend on its neighbour and its rows agree with the solo run to the
    # rounding of the split merge (fp16 partials), not bit for bit
    for a, b in zip(o1["attn"], o3["attn"]):
        assert torch.isfinite(b).all()
        assert rel_err(host(b), host(a[o:e]), (0, 1)) < TOL
    assert r3["L"][0] == r1["L"][1]


@pytest.mark.parametrize("W,cdt", [(8, "f32"), (2, "bf16"), (1, "bf16")])
def test_commit_deep_path_and_conv_widths(gpu, W, cdt):
    """UPDATE and SELECT over a 40-node accepted chain (several ancestor
    batches of the UPDATE) and a short path in a second tree; conv prefixes of
    width W over C = 2056 channels (column groups with a ragged tail): the two
    modes bitwise equal, the oracle's state within tolerance, its prefix
    exactly."""
    banner(f"commit deep path, conv W={W} {cdt}")
    C2, d2 = 2056, 64
    trees = [synth.chain(40), synth.random_tree(synth.rng_for(7, 87), 12, 5)]
    par, off = synth.concat_trees(trees)
    n, B = len(par), len(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    ddt.ddt_tree_plan(tb, 64)
    paths = [oracle.root_path(t, int(np.argmax(oracle.depth(t)))) for t in trees]
    assert len(paths[0]) == 40
    ph = np.full((B, tb.n_max), -1, np.int32)
    for b, p in enumerate(paths):
        ph[b, :len(p)] = p
    Lh = np.array([len(p) for p in paths], np.int32)
    g = synth.gdn_inputs(7, (88,), n, Hk, Hv, d2, d2, "bf16", B=B)
    c = synth.conv_inputs(7, (89,), n, C2, W, cdt, B=B)
    res = {}
    for mode in (ddt.DDT_COMMIT_UPDATE, ddt.DDT_COMMIT_SELECT):
        dg = {k: dev(v) for k, v in g.items()}
        dc = {k: dev(v) for k, v in c.items()}
        o = torch.empty(n, Hv, d2, dtype=torch.float32, device=gpu)
        ns = torch.empty(n, Hv, d2, d2, dtype=torch.float32, device=gpu) if mode == ddt.DDT_COMMIT_SELECT else None
        nu = torch.empty(n, Hv, d2, dtype=torch.float32, device=gpu) if mode == ddt.DDT_COMMIT_UPDATE else None
        ddt.ddt_tree_gdn(tb, dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"], dg["S_c"], 1.0, o, ns, nu)
        gl = [ddt.GdnLayer(q=dg["q"].data_ptr(), k=dg["k"].data_ptr(), v=dg["v"].data_ptr(),
                           alpha=dg["alpha"].data_ptr(), beta=dg["beta"].data_ptr(), S_c=dg["S_c"].data_ptr(),
                           node_states=ns.data_ptr() if ns is not None else None,
                           node_u=nu.data_ptr() if nu is not None else None, x=dc["x"].data_ptr(),
                           prefix=dc["prefix"].data_ptr())]
        T = dev(np.array([5, 5], np.int32))
        ddt.ddt_commit_state(tb, dev(ph), dev(Lh), mode, ddt.layer_table(gl, gpu), 1, Hk, Hv, d2, d2,
                             ddt.DDT_BF16, C2, ddt.DDT_F32 if cdt == "f32" else ddt.DDT_BF16, None, 0, 1, 64,
                             ddt.DDT_F16, None, T)
        torch.cuda.synchronize()
        assert not host(tb.status).any()
        res[mode] = (dg, dc)
    (ug, uc), (sg, sc) = res[ddt.DDT_COMMIT_UPDATE], res[ddt.DDT_COMMIT_SELECT]
    assert torch.equal(ug["S_c"], sg["S_c"])
    assert torch.equal(uc["prefix"], sc["prefix"])
    for b in range(B):
        pg = [off[b] + j for j in paths[b]]
        S_ref = oracle.commit_gdn_state(g["S_c"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], pg, b)
        assert rel_err(host(ug["S_c"])[b], S_ref, (0,)) < TOL
        if W > 1:
            pre = oracle.commit_conv_prefix(c["prefix"], c["x"], pg, b)
            p = uc["prefix"]
            got = host(p)[b] if cdt == "f32" else host(p.view(torch.int16)).view(np.uint16)[b]
            assert np.array_equal(oracle.num.f64(got), pre)


def _commit_case(gpu, trees, paths, T, page_table, n_pages, cache_pages=None, seed=12):
    """One UPDATE commit of explicit paths over one delta-net + conv layer and
    one attention layer; returns the host inputs and the device buffers."""
    par, off = synth.concat_trees(trees)
    n, B = len(par), len(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    ddt.ddt_tree_plan(tb, 64)
    ph = np.full((B, tb.n_max), -1, np.int32)
    for b, p in enumerate(paths):
        ph[b, :len(p)] = p
    Lh = np.array([len(p) for p in paths], np.int32)
    g = synth.gdn_inputs(seed, (90,), n, Hk, Hv, dk, dk, "bf16", B=B)
    c = synth.conv_inputs(seed, (91,), n, C, W, "bf16", B=B)
    K, Vv = synth.kv_pool(seed, (92,), n_pages, Hkv, D, "f16")
    a = synth.attn_inputs(seed, (93,), n, Hq, Hkv, D, "f16")
    dg, dc = {k: dev(v) for k, v in g.items()}, {k: dev(v) for k, v in c.items()}
    dK, dV, da = dev(K), dev(Vv), {k: dev(v) for k, v in a.items()}
    o = torch.empty(n, Hv, dk, dtype=torch.float32, device=gpu)
    nu = torch.empty(n, Hv, dk, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_gdn(tb, dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"], dg["S_c"], 1.0, o, None, nu)
    gl = [ddt.GdnLayer(q=dg["q"].data_ptr(), k=dg["k"].data_ptr(), v=dg["v"].data_ptr(),
                       alpha=dg["alpha"].data_ptr(), beta=dg["beta"].data_ptr(), S_c=dg["S_c"].data_ptr(),
                       node_u=nu.data_ptr(), x=dc["x"].data_ptr(), prefix=dc["prefix"].data_ptr())]
    al = [ddt.AttnLayer(da["Kt"].data_ptr(), da["Vt"].data_ptr(), dK.data_ptr(), dV.data_ptr())]
    dT = dev(np.asarray(T, np.int32))
    pt = dev(page_table) if page_table is not None else None
    ddt.ddt_commit_state(tb, dev(ph), dev(Lh), ddt.DDT_COMMIT_UPDATE, ddt.layer_table(gl, gpu), 1, Hk, Hv,
                         dk, dk, ddt.DDT_BF16, C, ddt.DDT_BF16, ddt.layer_table(al, gpu), 1, Hkv, D,
                         ddt.DDT_F16, pt, dT, cache_pages=cache_pages)
    torch.cuda.synchronize()
    return dict(par=par, off=off, g=g, c=c, K=K, V=Vv, a=a, dg=dg, dc=dc, dK=dK, dV=dV, T=dT,
                status=host(tb.status))


def _u16(t):
    return host(t.view(torch.int16)).view(np.uint16)


def test_commit_refuses_a_sequence_its_cache_cannot_hold(gpu):
    """A sequence whose accepted tokens do not fit its pages is not committed
    at all (state, conv prefix, cache and T untouched, DDT_ST_CTX set); the
    other sequence of the batch is committed as usual."""
    banner("commit capacity: paged batch, one sequence refused")
    trees = [synth.random_tree(synth.rng_for(5, 94, b), 22, 8) for b in range(2)]
    paths = [oracle.root_path(t, int(np.argmax(oracle.depth(t))))[:4] for t in trees]
    n_pages = 40
    pt = np.arange(2 * 16, dtype=np.int32).reshape(2, 16)[:, ::-1].copy()  # 16 pages per sequence
    pt[1] = pt[1] + 8                                                        # shared pool of 40 pages
    T = [100, 16 * 16 - 2]   # sequence 1: 254 + 4 > 256 slots of its table
    r = _commit_case(gpu, trees, paths, T, pt, n_pages)
    assert r["status"][0] == 0 and r["status"][1] == ddt.DDT_ST_CTX
    assert list(host(r["T"])) == [100 + 4, T[1]]
    off = r["off"]
    # sequence 1 untouched, bit for bit
    S = host(r["dg"]["S_c"])
    assert np.array_equal(S[1], r["g"]["S_c"][1])
    assert np.array_equal(_u16(r["dc"]["prefix"])[1], r["c"]["prefix"][1])
    # sequence 0 committed: state, prefix and its four cache slots
    pg = [off[0] + j for j in paths[0]]
    g = r["g"]
    S_ref = oracle.commit_gdn_state(g["S_c"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], pg, 0)
    assert rel_err(S[0], S_ref, (0,)) < TOL
    assert np.array_equal(oracle.num.f64(_u16(r["dc"]["prefix"])[0]),
                          oracle.commit_conv_prefix(r["c"]["prefix"], r["c"]["x"], pg, 0))
    K2, V2, _ = oracle.commit_kv(r["K"], r["V"], pt, np.asarray(T), r["a"]["Kt"], r["a"]["Vt"], pg, 0)
    # no slot of sequence 1's pages changed: the whole pool equals sequence 0's commit alone
    assert np.array_equal(host(r["dK"]).view(np.uint16), K2.view(np.uint16))
    assert np.array_equal(host(r["dV"]).view(np.uint16), V2.view(np.uint16))


@pytest.mark.parametrize("room", [2, 3])
def test_commit_contiguous_cache_capacity(gpu, room):
    """A contiguous cache of 8 pages (128 tokens) and a 3-token path: with 2
    free slots the commit is refused whole; with 3 it fills the last slots."""
    banner(f"commit capacity: contiguous cache, {room} free slots")
    tree = synth.random_tree(synth.rng_for(6, 95), 22, 8)
    path = oracle.root_path(tree, int(np.argmax(oracle.depth(tree))))[:3]
    T0 = 128 - room
    r = _commit_case(gpu, [tree], [path], [T0], None, 8, cache_pages=8)
    S = host(r["dg"]["S_c"])
    if room < 3:
        assert r["status"][0] == ddt.DDT_ST_CTX and int(host(r["T"])[0]) == T0
        assert np.array_equal(S, r["g"]["S_c"])
        assert np.array_equal(_u16(r["dc"]["prefix"]), r["c"]["prefix"])
        assert np.array_equal(host(r["dK"]).view(np.uint16), r["K"].view(np.uint16))
        assert np.array_equal(host(r["dV"]).view(np.uint16), r["V"].view(np.uint16))
    else:
        assert r["status"][0] == 0 and int(host(r["T"])[0]) == 128
        g = r["g"]
        S_ref = oracle.commit_gdn_state(g["S_c"], g["q"], g["k"], g["v"], g["alpha"], g["beta"], path, 0)
        assert rel_err(S[0], S_ref, (0,)) < TOL
        K2, V2, _ = oracle.commit_kv(r["K"], r["V"], None, np.array([T0]), r["a"]["Kt"], r["a"]["Vt"], path, 0)
        assert np.array_equal(host(r["dK"]).view(np.uint16), K2.view(np.uint16))
        assert np.array_equal(host(r["dV"]).view(np.uint16), V2.view(np.uint16))
