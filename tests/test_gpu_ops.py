"""GPU parity of each entry point against the CPU oracle, through the C ABI.

Sizes span several tiles and ragged tails while the oracle still finishes in
seconds; integer outputs are compared bit for bit, floating-point outputs to
max relative error 2e-3 per slice."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import TOL, banner, dev, host, rel_err

pytestmark = pytest.mark.gpu


def make_batch(trees, W, gpu, max_levels=64):
    par, off = synth.concat_trees(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    ddt.ddt_tree_plan(tb, max_levels)
    return tb, par, off


# ------------------------------------------------------------------ plan
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_device_matches_host_and_oracle(gpu, seed):
    banner(f"plan seed={seed}")
    sizes = [22, 64, 1, 7, 33, 2, 16]
    trees = [synth.random_tree(synth.rng_for(seed, 30, b), s, 10) for b, s in enumerate(sizes)]
    trees += [synth.chain(64), synth.binary_tree(6)]
    for W in (4, 1, 8):
        tb, par, off = make_batch(trees, W, gpu)
        torch.cuda.synchronize()
        n = len(par)
        W1 = max(W - 1, 1)
        h = dict(depth=np.zeros(n, np.int32), anc=np.zeros(n, np.uint64),
                 win=np.zeros(n * W1, np.int32), status=np.zeros(len(trees), np.int32))
        st = ddt.plan_struct(len(trees), n, tb.n_max, W, off, par, h["depth"], h["anc"], h["win"],
                             h["status"])
        assert ddt.ddt_tree_plan_host(st, 64) == 0
        assert np.array_equal(host(tb.depth), h["depth"])
        assert np.array_equal(host(tb.anc).view(np.uint64), h["anc"])
        assert np.array_equal(host(tb.win), h["win"])
        assert not host(tb.status).any()
        for b, t in enumerate(trees):
            o, e = off[b], off[b + 1]
            assert list(host(tb.depth)[o:e]) == list(oracle.depth(t))
            assert [int(x) for x in host(tb.anc).view(np.uint64)[o:e]] == oracle.ancestor_mask(t)
            if W > 1:
                np.testing.assert_array_equal(host(tb.win)[o * (W - 1):e * (W - 1)].reshape(e - o, W - 1),
                                              oracle.conv_window(t, W))


def test_plan_flags_malformed_trees(gpu):
    banner("plan malformed")
    good = synth.random_tree(synth.rng_for(0, 31), 22, 8)
    bad1 = good.copy(); bad1[5] = 9          # parent after child
    bad2 = good.copy(); bad2[0] = 0          # root with a parent
    deep = synth.chain(12)                   # 12 levels > cap 8
    par, off = synth.concat_trees([good, bad1, bad2, deep])
    tb = ddt.TreeBatch(par, off, 4, gpu)
    ddt.ddt_tree_plan(tb, 8)
    st = host(tb.status)
    assert st[0] == 0
    assert st[1] & ddt.DDT_ST_TREE and st[2] & ddt.DDT_ST_TREE
    assert st[3] == ddt.DDT_ST_LEVELS
    # the stand-in plan of a flagged tree stays in bounds for the later kernels:
    # a node's mask holds itself and lower ids only, depth = mask size - 1, and
    # window entries are lower node ids or prefix slots -1..-3
    depth, anc, win = host(tb.depth), host(tb.anc).view(np.uint64), host(tb.win).reshape(-1, 3)
    for b in range(4):
        o, e = off[b], off[b + 1]
        for i in range(e - o):
            a = int(anc[o + i])
            assert a >> i & 1 and a >> (i + 1) == 0 and a & 1
            assert depth[o + i] == bin(a).count("1") - 1
            assert all(-3 <= v < i or (i == 0 and v < 0) for v in win[o + i])


# ------------------------------------------------------------------ conv
@pytest.mark.parametrize("case", ["tiny_f32", "layer_bf16", "batch_silu_bf16"])
def test_conv(gpu, case):
    banner(f"conv {case}")
    if case == "tiny_f32":
        trees, C, W, dt, act = [synth.binary_tree(3)], 64, 4, "f32", 0
    elif case == "layer_bf16":
        trees, C, W, dt, act = [synth.random_tree(synth.rng_for(1, 40), 22, 8)], 8192, 4, "bf16", 0
    else:
        trees = [synth.random_tree(synth.rng_for(2, 41, b), s, 10) for b, s in enumerate([8, 64, 22])]
        C, W, dt, act = 1024, 4, "bf16", 1
    tb, par, off = make_batch(trees, W, gpu)
    inp = synth.conv_inputs(3, (42,), len(par), C, W, dt, B=len(trees))
    y = torch.empty(len(par), C, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_conv(tb, dev(inp["x"]), dev(inp["prefix"]), dev(inp["w"]), act, y)
    ref = oracle.tree_conv(par, inp["x"], inp["prefix"], inp["w"], act=act, tree_off=off)
    assert rel_err(host(y), ref, (0,)) < TOL


# ------------------------------------------------------------------ gated delta-net
GDN_CASES = {
    "tiny_f32": dict(sizes=[7], Hk=2, Hv=2, d=16, dt="f32", binary=True),
    "layer_bf16": dict(sizes=[22], Hk=16, Hv=32, d=128, dt="bf16"),
    "batch_bf16": dict(sizes=[8, 64, 22, 1], Hk=2, Hv=4, d=128, dt="bf16"),
    "gqa_d64_f32": dict(sizes=[13, 5], Hk=1, Hv=4, d=64, dt="f32"),
}


@pytest.mark.parametrize("case", list(GDN_CASES))
def test_gdn(gpu, case):
    banner(f"gdn {case}")
    c = GDN_CASES[case]
    if c.get("binary"):
        trees = [synth.binary_tree(3)]
    else:
        trees = [synth.random_tree(synth.rng_for(4, 50, b), s, 10) for b, s in enumerate(c["sizes"])]
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    inp = synth.gdn_inputs(5, (51,), n, c["Hk"], c["Hv"], c["d"], c["d"], c["dt"], B=B)
    d = {k: dev(v) for k, v in inp.items()}
    out = torch.empty(n, c["Hv"], c["d"], dtype=torch.float32, device=gpu)
    out2 = torch.empty_like(out)
    ns = torch.empty(n, c["Hv"], c["d"], c["d"], dtype=torch.float32, device=gpu)
    nu = torch.empty(n, c["Hv"], c["d"], dtype=torch.float32, device=gpu)
    ddt.ddt_tree_gdn(tb, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_c"], 1.0, out)
    ddt.ddt_tree_gdn(tb, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_c"], 1.0, out2, ns, nu)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # persisting states does not change the outputs
    if c["Hv"] * c["d"] ** 2 * n <= 32 * 128 * 128 * 22:
        ref, states = oracle.tree_gdn(par, **inp, tree_off=off, want_states=True)
        assert rel_err(host(ns), states, (0, 1)) < TOL
        # saved u_i = beta_i (v_i - alpha_i S_parent k_i), from the oracle's states
        f = oracle.num.f64
        k64, v64, a64, b64, S64 = f(inp["k"]), f(inp["v"]), f(inp["alpha"]), f(inp["beta"]), f(inp["S_c"])
        grp = c["Hv"] // c["Hk"]
        u_ref = np.empty((n, c["Hv"], c["d"]))
        for bb in range(B):
            for j in range(off[bb], off[bb + 1]):
                for hh in range(c["Hv"]):
                    Sp = S64[bb, hh] if par[j] < 0 else states[off[bb] + par[j], hh]
                    u_ref[j, hh] = b64[j, hh] * (v64[j, hh] - a64[j, hh] * (Sp @ k64[j, hh // grp]))
        assert rel_err(host(nu), u_ref, (0, 1)) < TOL
    else:
        ref = oracle.tree_gdn(par, **inp, tree_off=off)
    assert rel_err(host(out), ref, (0, 1)) < TOL


def test_gdn_scale(gpu):
    banner("gdn scale")
    trees = [synth.random_tree(synth.rng_for(6, 52), 10, 5)]
    tb, par, off = make_batch(trees, 4, gpu)
    inp = synth.gdn_inputs(6, (52,), len(par), 2, 4, 32, 32, "bf16")
    d = {k: dev(v) for k, v in inp.items()}
    out = torch.empty(len(par), 4, 32, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_gdn(tb, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_c"], 0.125, out)
    ref = oracle.tree_gdn(par, **inp, scale=0.125)
    assert rel_err(host(out), ref, (0, 1)) < TOL


# ------------------------------------------------------------------ attention
def attn_case(gpu, trees, T, Hq, Hkv, D, dt, seed, paged=True, nan_fill=False, n_splits=0,
              rows=None, plant=None):
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    T = np.asarray(T)
    pt, P = synth.page_layout(seed, (60,), T, [len(t) for t in trees], shuffle=paged)
    K, V = synth.kv_pool(seed, (60,), P, Hkv, D, dt)
    if nan_fill:  # slots past T must never influence the result
        for b in range(B):
            for t in range(int(T[b]), int(np.ceil((T[b] + len(trees[b])) / 16)) * 16):
                K[pt[b][t // 16], :, t % 16, :] = np.nan
                V[pt[b][t // 16], :, :, t % 16] = np.nan
    a = synth.attn_inputs(seed, (61,), n, Hq, Hkv, D, dt)
    if plant is not None:  # edits the inputs in place (both sides see the same values)
        plant(K, a, pt, off)
    use_pt = paged or B > 1
    ptd = dev(pt) if use_pt else None
    Td = dev(T.astype(np.int32))
    T_max = int(T.max())
    ws_bytes = ddt.ddt_tree_attn_workspace(tb, Hq, Hkv, D, T_max, n_splits)
    # all-ones bytes (NaN floats): slots of splits a sequence leaves unused must never be read
    # into its result
    ws = torch.full((max(ws_bytes, 1),), 255, dtype=torch.uint8, device=gpu)
    out = torch.full((n, Hq, D), np.nan, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_attn(tb, dev(a["q"]), dev(K), dev(V), ptd, Td, T_max, dev(a["Kt"]), dev(a["Vt"]),
                      out, ws, n_splits=n_splits)
    torch.cuda.synchronize()
    ref = oracle.tree_attn(par, a["q"], K, V, T, a["Kt"], a["Vt"],
                           page_table=pt if use_pt else None, tree_off=off, rows=rows)
    got = host(out)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        return rel_err(got[idx], ref[idx], (0,)), tb
    assert np.isfinite(got).all()
    return rel_err(got, ref, (0, 1)), tb


def test_attn_tiny_f32(gpu):
    banner("attn tiny f32 D=16")
    err, _ = attn_case(gpu, [synth.binary_tree(3)], [64], 2, 1, 16, "f32", 0, paged=False)
    assert err < TOL


@pytest.mark.parametrize("T", [0, 5, 32, 100, 1000, 4133])
def test_attn_mfma_contiguous(gpu, T):
    banner(f"attn mfma D=256 N=22 T={T}")
    tree = synth.random_tree(synth.rng_for(7, 62), 22, 8)
    err, _ = attn_case(gpu, [tree], [T], 24, 4, 256, "f16", 7, paged=False)
    assert err < TOL


@pytest.mark.parametrize("n_splits", [1, 3, 0])
def test_attn_mfma_paged_nan_tail(gpu, n_splits):
    banner(f"attn mfma paged nan-tail splits={n_splits}")
    trees = [synth.random_tree(synth.rng_for(8, 63, b), s, 10) for b, s in enumerate([22, 8, 64])]
    err, _ = attn_case(gpu, trees, [1500, 37, 3001], 24, 4, 256, "f16", 8, paged=True,
                       nan_fill=True, n_splits=n_splits)
    assert err < TOL


def test_attn_mfma_d128_and_chain(gpu):
    banner("attn mfma D=128")
    trees = [synth.chain(16), synth.random_tree(synth.rng_for(9, 64), 32, 10)]
    err, _ = attn_case(gpu, trees, [777, 2048], 16, 2, 128, "f16", 9)
    assert err < TOL


def test_attn_full_context_32k_sampled(gpu):
    banner("attn mfma T=32768 N=22 sampled rows")
    tree = synth.random_tree(synth.rng_for(10, 65), 22, 8)
    rng = np.random.default_rng(10)
    rows = [(int(i), int(h)) for i, h in zip(rng.integers(0, 22, 12), rng.integers(0, 24, 12))]
    rows += [(21, 23), (0, 0)]
    err, _ = attn_case(gpu, [tree], [32768], 24, 4, 256, "f16", 10, paged=False, rows=rows)
    assert err < TOL


# Tree sizes that give 1, 2 and 3 row blocks (16 query rows each) per
# wavefront, with and without padding blocks; contiguous and paged caches,
# NaN in unused page slots, batches, both head sizes, fixed and automatic
# split counts.
ATTN_SHAPES = {
    #  name: (tree sizes, T, Hq, Hkv, D, paged, nan_fill, n_splits)
    "1_block": ([1], [100], 24, 4, 256, False, False, 0),
    "2_blocks_batch": ([5, 3], [40, 700], 24, 4, 256, True, True, 0),
    "4_blocks": ([10], [1000], 24, 4, 256, True, False, 5),
    "6_blocks_batch": ([16, 9], [2100, 333], 24, 4, 256, True, True, 0),
    "8_blocks": ([20], [1234], 24, 4, 256, False, False, 1),
    "10_blocks": ([26], [3000], 24, 4, 256, True, True, 0),
    "11_blocks": ([27], [3000], 24, 4, 256, True, True, 0),
    "d128_6_blocks": ([8, 12], [777, 1500], 16, 2, 128, True, False, 0),
    "d128_10_blocks": ([20], [2500], 16, 2, 128, True, True, 3),
    # one sequence whose last round has 1 or 2 blocks: shared by pairs of waves
    "5_blocks_shared": ([12], [1500], 24, 4, 256, False, False, 0),
    "6_blocks_shared": ([16], [2222], 24, 4, 256, True, False, 0),
    "9_blocks_shared_ragged": ([22], [4133], 24, 4, 256, True, True, 3),
    # more splits than one combine batch holds (64), some of them left empty
    "many_splits": ([22], [40000], 6, 1, 256, False, False, 100),
    "many_splits_batch": ([22, 7], [30000, 900], 12, 2, 256, True, True, 90),
    # a batch shares the splits of a (KV head, row group): fewer splits asked
    # for than sequences (raised to one each), an empty context, a row group
    # that only some sequences reach, more sequences than a wavefront's lanes
    "pool_below_batch": ([3, 5, 2, 7], [500, 0, 2000, 64], 24, 4, 256, True, True, 2),
    "pool_uneven_rows": ([40, 2, 30], [3000, 5000, 100], 24, 4, 256, True, True, 0),
    "pool_70_seqs": ([1 + b % 8 for b in range(70)], [(b * 397) % 3001 for b in range(70)],
                     24, 4, 256, True, False, 0),
}


@pytest.mark.parametrize("case", list(ATTN_SHAPES))
def test_attn_mfma_shapes(gpu, case):
    sizes, T, Hq, Hkv, D, paged, nan_fill, ns = ATTN_SHAPES[case]
    banner(f"attn mfma {case}: sizes {sizes} T {T} Hq {Hq} Hkv {Hkv} D {D} splits {ns}")
    trees = [synth.random_tree(synth.rng_for(15, 68, b), n, 10) for b, n in enumerate(sizes)]
    err, _ = attn_case(gpu, trees, T, Hq, Hkv, D, "f16", 15, paged=paged, nan_fill=nan_fill,
                       n_splits=ns)
    assert err < TOL


def test_attn_mfma_batch_above_split_limit(gpu):
    # every sequence of a batch needs a split of its own, and a (KV head, row
    # group) has at most 1024: a larger batch is refused before any launch
    banner("attn mfma batch of 1025 one-node sequences: shape error")
    tb, par, off = make_batch([synth.chain(1)] * 1025, 4, gpu)
    n = len(par)
    q = torch.zeros(n, 24, 256, dtype=torch.float16, device=gpu)
    kv = torch.zeros(n, 4, 256, dtype=torch.float16, device=gpu)
    cache = torch.zeros(1, 4, 16, 256, dtype=torch.float16, device=gpu)
    pt = torch.zeros(1025, 1, dtype=torch.int32, device=gpu)
    T = torch.zeros(1025, dtype=torch.int32, device=gpu)
    out = torch.zeros(n, 24, 256, dtype=torch.float32, device=gpu)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=gpu)
    with pytest.raises(ddt.DDTError) as e:
        ddt.ddt_tree_attn(tb, q, cache, cache, pt, T, 0, kv, kv, out, ws)
    assert e.value.code == -3  # DDT_E_SHAPE


# ---- 8-bit cache: the same attention over fp16(code * token scale)
Q8_SCALES = {
    "default": {},
    # V scales over 16 binades (2^-12 .. 2^4) in token order: later tiles hold
    # scales far above and below the first tile's, K scales up to 0.06
    "wide": dict(ksc=(-10.0, -4.0), vsc=(-12.0, 4.0), log2=True),
}


def attn_q8_case(gpu, trees, T, Hq, Hkv, D, seed, paged=True, n_splits=0, scales="default"):
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    T = np.asarray(T)
    pt, P = synth.page_layout(seed, (70,), T, [len(t) for t in trees], shuffle=paged)
    c = synth.kv_pool_q8(seed, (70,), P, Hkv, D, **Q8_SCALES[scales])
    a = synth.attn_inputs(seed, (71,), n, Hq, Hkv, D, "f16")
    use_pt = paged or B > 1
    T_max = int(T.max())
    ws = torch.full((max(ddt.ddt_tree_attn_workspace(tb, Hq, Hkv, D, T_max, n_splits), 1),), 255,
                    dtype=torch.uint8, device=gpu)
    out = torch.full((n, Hq, D), np.nan, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_attn_q8(tb, dev(a["q"]), dev(c["Kq"]), dev(c["Ksc"]), dev(c["Vq"]), dev(c["Vsc"]),
                         dev(pt) if use_pt else None, dev(T.astype(np.int32)), T_max, dev(a["Kt"]),
                         dev(a["Vt"]), out, ws, n_splits=n_splits)
    torch.cuda.synchronize()
    K, V = oracle.dequant_q8(c["Kq"], c["Ksc"], c["Vq"], c["Vsc"])
    ref = oracle.tree_attn(par, a["q"], K, V, T, a["Kt"], a["Vt"], page_table=pt if use_pt else None,
                           tree_off=off)
    got = host(out)
    assert np.isfinite(got).all()
    return rel_err(got, ref, (0, 1))


ATTN_Q8 = {
    #  name: (tree sizes, T, Hq, Hkv, D, paged, n_splits)
    "tree_only": ([22], [0], 24, 4, 256, False, 0),
    "one_tile": ([22], [32], 24, 4, 256, False, 0),
    "three_tiles": ([22], [100], 24, 4, 256, False, 0),
    "ragged_4133": ([22], [4133], 24, 4, 256, False, 0),
    "batch_paged": ([22, 8, 64], [1500, 37, 3001], 24, 4, 256, True, 0),
    "d128": ([16, 32], [777, 2048], 16, 2, 128, True, 3),
    "many_splits": ([22], [40000], 6, 1, 256, False, 100),
    "ragged_tiny_splits": ([5], [75], 24, 4, 256, False, 4),
    "wide_scales": ([22], [4133], 24, 4, 256, False, 0, "wide"),
    "wide_scales_d128_paged": ([16, 9], [3000, 517], 16, 2, 128, True, 5, "wide"),
    "pool_uneven_rows": ([40, 2, 30], [3000, 5000, 100], 24, 4, 256, True, 0),
}


@pytest.mark.parametrize("case", list(ATTN_Q8))
def test_attn_q8(gpu, case):
    sizes, T, Hq, Hkv, D, paged, ns, *sc = ATTN_Q8[case]
    sc = sc[0] if sc else "default"
    banner(f"attn q8 {case}: sizes {sizes} T {T} Hq {Hq} Hkv {Hkv} D {D} splits {ns} scales {sc}")
    trees = [synth.random_tree(synth.rng_for(16, 72, b), n, 10) for b, n in enumerate(sizes)]
    assert attn_q8_case(gpu, trees, T, Hq, Hkv, D, 16, paged=paged, n_splits=ns, scales=sc) < TOL


def test_attn_q8_full_context_128k_sampled(gpu):
    """The 8-bit call at the size and launch configuration the benchmark
    times (T = 131,072, one 22-node tree, 24 q / 4 KV heads, D = 256,
    contiguous cache, default split count); sampled rows against the oracle."""
    n, Hq, Hkv, D, T = 22, 24, 4, 256, 131072
    banner(f"attn q8 full size: T {T} N {n} Hq {Hq} Hkv {Hkv} D {D}, sampled rows")
    tree = synth.random_tree(synth.rng_for(16, 73, 0), n, 10)
    tb, par, off = make_batch([tree], 4, gpu)
    Ta = np.array([T])
    _, P = synth.page_layout(17, (74,), Ta, [n], shuffle=False)
    c = synth.kv_pool_q8(17, (74,), P, Hkv, D)
    a = synth.attn_inputs(17, (75,), n, Hq, Hkv, D, "f16")
    ws = torch.full((ddt.ddt_tree_attn_workspace(tb, Hq, Hkv, D, T),), 255, dtype=torch.uint8, device=gpu)
    out = torch.full((n, Hq, D), np.nan, dtype=torch.float32, device=gpu)
    ddt.ddt_tree_attn_q8(tb, dev(a["q"]), dev(c["Kq"]), dev(c["Ksc"]), dev(c["Vq"]), dev(c["Vsc"]), None,
                         dev(Ta.astype(np.int32)), T, dev(a["Kt"]), dev(a["Vt"]), out, ws)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    K, V = oracle.dequant_q8(c["Kq"], c["Ksc"], c["Vq"], c["Vsc"])
    rng = np.random.default_rng(3)
    rows = [(int(i), int(h)) for i, h in zip(rng.integers(0, n, 6), rng.integers(0, Hq, 6))]
    rows += [(0, 0), (n - 1, Hq - 1)]
    ref = oracle.tree_attn(par, a["q"], K, V, [T], a["Kt"], a["Vt"], rows=rows)
    idx = tuple(np.array(rows).T)
    assert rel_err(got[idx], ref[idx], (0,)) < TOL


def _plant_cache(t):
    """Key at cache position t of sequence 0, KV head 0 := 4 q of node 0,
    q head 0: that row's score there is ~4|q|^2, about 90 binades (at scale
    1/16) above anything in the first tile of its split."""
    def f(K, a, pt, off):
        page = pt[0][t // 16]
        K[page, 0, t % 16, :] = (4.0 * a["q"][off[0], 0].astype(np.float32)).astype(K.dtype)
    return f


def _plant_tree(K, a, pt, off):
    """Draft key of node 0 (seen by every node), KV head 0 := 4 q of node 0."""
    a["Kt"][off[0], 0] = (4.0 * a["q"][off[0], 0].astype(np.float32)).astype(a["Kt"].dtype)


@pytest.mark.parametrize("where,size", [("cache", 22), ("tree", 22), ("cache", 64), ("tree", 64)])
def test_attn_redo_after_overflow(gpu, where, size):
    """A score far above its row's reference (fixed by the first tile) makes
    the split run again against the true maxima; the result must still be
    the plain softmax.  Size 64 also spreads the rows over two workgroups."""
    banner(f"attn overflow redo: planted {where} key, tree size {size}")
    tree = synth.random_tree(synth.rng_for(16, 69), size, 8)
    plant = _plant_cache(2960) if where == "cache" else _plant_tree
    err, _ = attn_case(gpu, [tree], [3000], 24, 4, 256, "f16", 16, paged=True, plant=plant)
    assert err < TOL


def test_attn_deterministic(gpu):
    banner("attn determinism")
    tree = synth.random_tree(synth.rng_for(11, 66), 22, 8)
    tb, par, off = make_batch([tree], 4, gpu)
    pt, P = synth.page_layout(11, (67,), [3000], [22])
    K, V = synth.kv_pool(11, (67,), P, 4, 256, "f16")
    a = synth.attn_inputs(11, (67,), 22, 24, 4, 256, "f16")
    args = [dev(a["q"]), dev(K), dev(V), dev(pt), dev(np.array([3000], np.int32)), 3000,
            dev(a["Kt"]), dev(a["Vt"])]
    ws = torch.empty(ddt.ddt_tree_attn_workspace(tb, 24, 4, 256, 3000), dtype=torch.uint8, device=gpu)
    o1 = torch.empty(22, 24, 256, dtype=torch.float32, device=gpu)
    o2 = torch.empty_like(o1)
    ddt.ddt_tree_attn(tb, *args, o1, ws)
    ddt.ddt_tree_attn(tb, *args, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------------------------ accept walk
@pytest.mark.parametrize("case", ["planted_bf16", "ties_bf16", "f32_ragged_vocab", "batch"])
def test_accept_walk(gpu, case):
    banner(f"walk {case}")
    V = 151936
    if case == "planted_bf16":
        trees, dt, plant, pm = [synth.random_tree(synth.rng_for(12, 70), 22, 8)], "bf16", True, 0.8
    elif case == "ties_bf16":
        trees, dt, plant, pm = [synth.random_tree(synth.rng_for(13, 71), 22, 8)], "bf16", False, 0
    elif case == "f32_ragged_vocab":
        trees, dt, plant, pm, V = [synth.binary_tree(3)], "f32", True, 0.9, 1001
    else:
        trees = [synth.random_tree(synth.rng_for(14, 72, b), s, 10) for b, s in enumerate([8, 64, 22, 1, 32])]
        dt, plant, pm = "bf16", True, 0.9
    logits, toks = [], []
    for b, t in enumerate(trees):
        lg, tk = synth.logits_and_draft(15, (73, b), t, V, dt, p_match=pm, plant=plant)
        logits.append(lg)
        toks.append(tk)
    lg = np.concatenate(logits)
    tok = np.concatenate(toks).astype(np.int32)
    if case == "ties_bf16":
        # unplanted bf16 rows tie at their maximum; force one more explicit
        # tie, then let every other node carry its parent's argmax so the walk
        # runs deep through tie-decided choices
        X = oracle.num.f64(lg)
        lg[5, 100:110] = lg[5, int(np.argmax(X[5]))]
        am = oracle.argmax_rows(lg)
        par0 = trees[0]
        for i in range(1, len(par0)):
            if i % 3:
                tok[i] = am[par0[i]]
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    ws = torch.empty(ddt.ddt_accept_walk_workspace(tb, V), dtype=torch.uint8, device=gpu)
    am = torch.empty(n, dtype=torch.int32, device=gpu)
    path = torch.empty(B, tb.n_max, dtype=torch.int32, device=gpu)
    L = torch.empty(B, dtype=torch.int32, device=gpu)
    bonus = torch.empty(B, dtype=torch.int32, device=gpu)
    ddt.ddt_accept_walk(tb, dev(lg), dev(tok), am, path, L, bonus, ws)
    torch.cuda.synchronize()
    ref_am = oracle.argmax_rows(lg)
    assert np.array_equal(host(am), ref_am)
    paths, rL, rb = oracle.accept_walk(par, tok, ref_am, tree_off=off)
    assert np.array_equal(host(L), rL) and np.array_equal(host(bonus), rb)
    hp = host(path)
    for b in range(B):
        assert list(hp[b, :rL[b]]) == paths[b] and (hp[b, rL[b]:] == -1).all()
    assert not host(tb.status).any()
    if case == "planted_bf16":
        assert rL[0] >= 1


def test_accept_walk_nan_and_bad_tokens(gpu):
    banner("walk NaN + bad tokens")
    V = 4096
    tree = synth.chain(6)
    lg = np.random.default_rng(0).standard_normal((6, V)).astype(np.float32)
    lg[0, :] = np.nan
    lg[1, 7] = np.nan
    lg[1, 9] = 50.0
    lg[2, :] = -np.inf
    lg[3, [4, 8]] = [0.0, -0.0]
    lg[3, :4] = -1
    lg[3, 5:8] = -1
    lg[3, 9:] = -1
    tok = np.array([0, 0, 9, 0, V + 5, -3], dtype=np.int32)
    tb, par, off = make_batch([tree], 4, gpu)
    ws = torch.empty(ddt.ddt_accept_walk_workspace(tb, V), dtype=torch.uint8, device=gpu)
    am = torch.empty(6, dtype=torch.int32, device=gpu)
    path = torch.empty(1, 6, dtype=torch.int32, device=gpu)
    L = torch.empty(1, dtype=torch.int32, device=gpu)
    bonus = torch.empty(1, dtype=torch.int32, device=gpu)
    ddt.ddt_accept_walk(tb, dev(lg), dev(tok), am, path, L, bonus, ws)
    torch.cuda.synchronize()
    ref = oracle.argmax_rows(lg)
    assert np.array_equal(host(am), ref)
    assert host(tb.status)[0] == ddt.DDT_ST_TOKEN
    paths, rL, rb = oracle.accept_walk(par, tok, ref)
    assert host(L)[0] == rL[0] and host(bonus)[0] == rb[0]


def walk_batch(gpu, dt, seed, V=4096):
    trees = [synth.random_tree(synth.rng_for(seed, 95, b), s, 10) for b, s in enumerate([22, 64, 1, 8])]
    lgs, toks = [], []
    for b, t in enumerate(trees):
        lg, tk = synth.logits_and_draft(seed, (96, b), t, V, dt, p_match=0.9, plant=(b % 2 == 0))
        lgs.append(lg)
        toks.append(tk)
    lg, tok = np.concatenate(lgs), np.concatenate(toks).astype(np.int32)
    lg[3, :] = lg[3, 0]                        # a whole row tied
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    outs = dict(am=torch.empty(n, dtype=torch.int32, device=gpu),
                path=torch.empty(B, tb.n_max, dtype=torch.int32, device=gpu),
                L=torch.empty(B, dtype=torch.int32, device=gpu), bonus=torch.empty(B, dtype=torch.int32, device=gpu))
    ws = torch.empty(ddt.ddt_accept_walk_workspace(tb, V), dtype=torch.uint8, device=gpu)
    return tb, par, off, lg, tok, outs, ws


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_accept_walk_host_equals_device(gpu, dt):
    # the host walk (the fall-back) gives the device walk's outputs bit for bit
    banner(f"walk host == device {dt}")
    tb, par, off, lg, tok, o, ws = walk_batch(gpu, dt, 4)
    ddt.ddt_accept_walk(tb, dev(lg), dev(tok), o["am"], o["path"], o["L"], o["bonus"], ws)
    torch.cuda.synchronize()
    h = [np.empty(tuple(t.shape), np.int32) for t in (o["am"], o["path"], o["L"], o["bonus"])]
    ddt.ddt_accept_walk_host(tb.struct_host, lg, tok, *h)
    for t, a in zip((o["am"], o["path"], o["L"], o["bonus"]), h):
        assert np.array_equal(host(t), a)
    assert np.array_equal(h[0], oracle.argmax_rows(lg))


def test_accept_walk_fallback_from_status(gpu):
    banner("walk fall-back from the status word")
    tb, par, off, lg, tok, o, ws = walk_batch(gpu, "bf16", 5)
    args = (dev(lg), dev(tok), o["am"], o["path"], o["L"], o["bonus"], ws)
    st, ran = ddt.accept_walk_with_fallback(tb, *args)
    assert not ran and not st.any()
    ref = [host(t) for t in (o["am"], o["path"], o["L"], o["bonus"])]
    # a failed device check, set from the host: the host walk takes over and
    # writes the same outputs
    tb.status[2] = ddt.DDT_ST_ARGMAX
    st, ran = ddt.accept_walk_with_fallback(tb, *args)
    assert ran and st[2] & ddt.DDT_ST_ARGMAX
    for t, r in zip((o["am"], o["path"], o["L"], o["bonus"]), ref):
        assert np.array_equal(host(t), r)
