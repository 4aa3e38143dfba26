"""GPU parity of the fused conv -> SiLU -> split -> L2 norm -> gated delta-net
layer (ddt_tree_conv_gdn) against the oracle, through the C ABI, and the
commit of fused layers."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import TOL, banner, dev, host, rel_err

pytestmark = pytest.mark.gpu

CASES = {
    "small_bf16": dict(sizes=[12], Hk=2, Hv=4, dk=32, dv=32, W=4, dt="bf16"),
    "d16_w8_f32_batch": dict(sizes=[9, 17], Hk=1, Hv=2, dk=16, dv=16, W=8, dt="f32"),
    "d64_w1_gqa": dict(sizes=[13], Hk=1, Hv=4, dk=64, dv=32, W=1, dt="bf16"),
    "w2_d128": dict(sizes=[15], Hk=2, Hv=2, dk=128, dv=16, W=2, dt="f32"),
    "layer_bf16": dict(sizes=[22], Hk=16, Hv=32, dk=128, dv=128, W=4, dt="bf16"),
    "max_tree_d128": dict(sizes=[64], Hk=2, Hv=4, dk=128, dv=128, W=4, dt="bf16", levels=12),
    "batch_mixed": dict(sizes=[8, 64, 22, 1], Hk=2, Hv=4, dk=128, dv=64, W=4, dt="bf16"),
    "deep_chain": dict(chain=40, Hk=1, Hv=2, dk=64, dv=16, W=4, dt="f32"),
}


def make_batch(trees, W, gpu, max_levels=64):
    par, off = synth.concat_trees(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    ddt.ddt_tree_plan(tb, max_levels)
    return tb, par, off


def run_fused(gpu, tb, d, c, n, with_extras=True):
    o = torch.full((n, c["Hv"], c["dv"]), np.nan, dtype=torch.float32, device=gpu)
    ex = {}
    if with_extras:
        ex = dict(q_out=torch.full((n, c["Hk"], c["dk"]), np.nan, dtype=torch.float32, device=gpu),
                  k_out=torch.full((n, c["Hk"], c["dk"]), np.nan, dtype=torch.float32, device=gpu),
                  v_out=torch.full((n, c["Hv"], c["dv"]), np.nan, dtype=torch.float32, device=gpu),
                  node_states=torch.full((n, c["Hv"], c["dv"], c["dk"]), np.nan, dtype=torch.float32,
                                         device=gpu),
                  node_u=torch.full((n, c["Hv"], c["dv"]), np.nan, dtype=torch.float32, device=gpu))
    ddt.ddt_tree_conv_gdn(tb, d["x"], d["prefix"] if c["W"] > 1 else None, d["w"], d["alpha"], d["beta"],
                          d["S_c"], c["Hk"], c["dk"], 1.0, o, **ex)
    return o, ex


@pytest.mark.parametrize("case", list(CASES))
def test_fused_layer(gpu, case):
    banner(f"fused conv->gdn {case}")
    c = CASES[case]
    if "chain" in c:
        trees = [synth.chain(c["chain"])]
    else:
        trees = [synth.random_tree(synth.rng_for(9, 90, b), s, c.get("levels", 10))
                 for b, s in enumerate(c["sizes"])]
    tb, par, off = make_batch(trees, c["W"], gpu)
    n, B = len(par), len(trees)
    inp = synth.fused_inputs(9, (91,), n, c["Hk"], c["Hv"], c["dk"], c["dv"], c["W"], c["dt"], B=B)
    d = {k: dev(v) for k, v in inp.items()}
    o1, _ = run_fused(gpu, tb, d, c, n, with_extras=False)
    o2, ex = run_fused(gpu, tb, d, c, n)
    torch.cuda.synchronize()
    assert not host(tb.status).any()
    assert torch.equal(o1, o2)  # the optional outputs do not change the result
    ref, q, k, v, states = oracle.tree_conv_gdn(par, inp["x"], inp["prefix"], inp["w"], inp["alpha"],
                                                inp["beta"], inp["S_c"], c["Hk"], c["Hv"], c["dk"], c["dv"],
                                                tree_off=off, want_states=True)
    assert rel_err(host(o2), ref, (0, 1)) < TOL
    assert rel_err(host(ex["q_out"]), q, (0, 1)) < TOL
    assert rel_err(host(ex["k_out"]), k, (0, 1)) < TOL
    assert rel_err(host(ex["v_out"]), v, (0, 1)) < TOL
    assert rel_err(host(ex["node_states"]), states, (0, 1)) < TOL
    # saved u_j = beta_j (v_j - alpha_j S_parent k_j) from the oracle's states and normalised keys
    a64, b64, S64 = oracle.num.f64(inp["alpha"]), oracle.num.f64(inp["beta"]), oracle.num.f64(inp["S_c"])
    grp = c["Hv"] // c["Hk"]
    u_ref = np.empty((n, c["Hv"], c["dv"]))
    for bb in range(B):
        for j in range(off[bb], off[bb + 1]):
            for hh in range(c["Hv"]):
                Sp = S64[bb, hh] if par[j] < 0 else states[off[bb] + par[j], hh]
                u_ref[j, hh] = b64[j, hh] * (v[j, hh] - a64[j, hh] * (Sp @ k[j, hh // grp]))
    assert rel_err(host(ex["node_u"]), u_ref, (0, 1)) < TOL


def test_fused_scale_and_determinism(gpu):
    banner("fused scale, determinism")
    c = dict(Hk=2, Hv=4, dk=64, dv=32, W=4)
    trees = [synth.random_tree(synth.rng_for(10, 92), 20, 6)]
    tb, par, off = make_batch(trees, 4, gpu)
    n = len(par)
    inp = synth.fused_inputs(10, (92,), n, c["Hk"], c["Hv"], c["dk"], c["dv"], 4, "bf16")
    d = {k: dev(v) for k, v in inp.items()}
    outs = []
    for _ in range(3):
        o = torch.empty(n, c["Hv"], c["dv"], dtype=torch.float32, device=gpu)
        ddt.ddt_tree_conv_gdn(tb, d["x"], d["prefix"], d["w"], d["alpha"], d["beta"], d["S_c"], c["Hk"],
                              c["dk"], 0.25, o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref, _, _, _ = oracle.tree_conv_gdn(par, inp["x"], inp["prefix"], inp["w"], inp["alpha"], inp["beta"],
                                        inp["S_c"], c["Hk"], c["Hv"], c["dk"], c["dv"], scale=0.25)
    assert rel_err(host(outs[0]), ref, (0, 1)) < TOL


def _commit(gpu, tb, layers, path, L, mode, c, T):
    gl = [ddt.GdnLayer(q=l["q_out"].data_ptr(), k=l["k_out"].data_ptr(), v=l["v_out"].data_ptr(),
                       alpha=l["alpha"].data_ptr(), beta=l["beta"].data_ptr(), S_c=l["S_c"].data_ptr(),
                       node_states=l["node_states"].data_ptr(), node_u=l["node_u"].data_ptr(),
                       x=l["x"].data_ptr(), prefix=l["prefix"].data_ptr()) for l in layers]
    gt = ddt.layer_table(gl, gpu)
    C = 2 * c["Hk"] * c["dk"] + c["Hv"] * c["dv"]
    ddt.ddt_commit_state(tb, path, L, mode, gt, len(gl), c["Hk"], c["Hv"], c["dk"], c["dv"], ddt.DDT_F32, C,
                         ddt.DDT_BF16, None, 0, 1, 64, ddt.DDT_F16, None, T)


def test_fused_layers_commit(gpu):
    """Fused layers committed from their k_out / node_u (UPDATE) or node
    states (SELECT): bitwise the same state, the oracle's replay of the
    accepted path within tolerance, REPLAY within tolerance, conv prefix
    advanced over the path."""
    banner("fused commit update == select, vs oracle")
    c = dict(Hk=2, Hv=4, dk=128, dv=64, W=4)
    trees = [synth.random_tree(synth.rng_for(11, 93, b), s, 8) for b, s in enumerate([22, 9])]
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    # accepted path of each tree: the root path of its deepest node
    paths = []
    for t in trees:
        dep = oracle.depth(t)
        paths.append(oracle.root_path(t, int(np.argmax(dep))))
    ph = np.full((B, tb.n_max), -1, np.int32)
    for b, p in enumerate(paths):
        ph[b, :len(p)] = p
    Lh = np.array([len(p) for p in paths], np.int32)
    inps = [synth.fused_inputs(11, (94, l), n, c["Hk"], c["Hv"], c["dk"], c["dv"], 4, "bf16", B=B) for l in range(2)]
    res = {}
    for mode in (ddt.DDT_COMMIT_UPDATE, ddt.DDT_COMMIT_SELECT, ddt.DDT_COMMIT_REPLAY):
        layers = []
        for inp in inps:
            d = {k: dev(v) for k, v in inp.items()}
            o, ex = run_fused(gpu, tb, d, c, n)
            d.update(ex)
            layers.append(d)
        T = dev(np.array([100, 7], np.int32))
        _commit(gpu, tb, layers, dev(ph), dev(Lh), mode, c, T)
        torch.cuda.synchronize()
        assert not host(tb.status).any()
        assert np.array_equal(host(T), [100, 7])  # T is the KV length: no attention layer, no advance
        res[mode] = layers
    for l, inp in enumerate(inps):
        up, se, rp = (res[m][l] for m in (ddt.DDT_COMMIT_UPDATE, ddt.DDT_COMMIT_SELECT, ddt.DDT_COMMIT_REPLAY))
        assert torch.equal(up["S_c"], se["S_c"])
        assert rel_err(host(rp["S_c"]), host(se["S_c"]), (0, 1)) < TOL
        _, q, k, v = oracle.tree_conv_gdn(par, inp["x"], inp["prefix"], inp["w"], inp["alpha"], inp["beta"],
                                          inp["S_c"], c["Hk"], c["Hv"], c["dk"], c["dv"], tree_off=off)
        for b in range(B):
            pg = [off[b] + j for j in paths[b]]
            S_ref = oracle.commit_gdn_state(inp["S_c"], q, k, v, inp["alpha"], inp["beta"], pg, b)
            assert rel_err(host(up["S_c"])[b], S_ref, (0,)) < TOL
            pre = oracle.commit_conv_prefix(inp["prefix"], inp["x"], pg, b)
            got = oracle.num.f64(host(up["prefix"].view(torch.int16)).view(np.uint16))[b]
            assert np.array_equal(got, pre)
