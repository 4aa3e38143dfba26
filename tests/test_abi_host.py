"""C-ABI checks that need no GPU: exports, the host-side plan, and argument
validation (every call below returns before any kernel is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import tree_verification_ddtree_amd as ddt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "ddtree.h")).read()
    names = set(re.findall(r"\b(ddt_\w+)\s*\(", hdr))
    assert len(names) >= 12
    L = ddt.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert ddt.ddt_version() == 2


def test_library_reports_the_sources_it_was_built_from():
    from tree_verification_ddtree_amd import build
    h = ddt.ddt_source_hash()
    assert re.fullmatch(r"[0-9a-f]{64}", h), h
    assert h == build.source_hash(), "libddtree.so was built from other sources: rebuild it"


def host_plan(trees, W=4, max_levels=64, n_max=None):
    par, off = synth.concat_trees(trees)
    n = len(par)
    out = dict(depth=np.zeros(n, np.int32), anc=np.zeros(n, np.uint64),
               win=np.zeros(n * max(W - 1, 1), np.int32), status=np.zeros(len(trees), np.int32))
    nm = n_max or max(len(t) for t in trees)
    st = ddt.plan_struct(len(trees), n, nm, W, off, par, out["depth"], out["anc"], out["win"],
                         out["status"])
    rc = ddt.ddt_tree_plan_host(st, max_levels)
    return rc, par, off, out


@pytest.mark.parametrize("seed", range(6))
def test_host_plan_matches_oracle(seed):
    sizes = [22, 64, 1, 7, 33, 2]
    trees = [synth.random_tree(synth.rng_for(seed, 20, b), s, 10 if s > 22 else 8)
             for b, s in enumerate(sizes)]
    trees.append(synth.chain(40))
    trees.append(synth.binary_tree(5))   # 31 nodes
    for W in (4, 1, 8):
        rc, par, off, out = host_plan(trees, W=W)
        assert rc == 0
        W1 = max(W - 1, 1)
        for b, t in enumerate(trees):
            o, e = off[b], off[b + 1]
            n = e - o
            assert list(out["depth"][o:e]) == list(oracle.depth(t))
            assert [int(x) for x in out["anc"][o:e]] == oracle.ancestor_mask(t)
            if W > 1:
                np.testing.assert_array_equal(out["win"][o * W1:e * W1].reshape(n, W1),
                                              oracle.conv_window(t, W))
            assert out["status"][b] == 0


def test_host_plan_all_small_trees():
    import itertools
    for n in range(1, 7):
        for ps in itertools.product(*[range(i) for i in range(1, n)]):
            t = np.array([-1, *ps], dtype=np.int32)
            rc, par, off, out = host_plan([t], W=3)
            assert rc == 0
            assert [int(x) for x in out["anc"]] == oracle.ancestor_mask(t)
            assert list(out["depth"]) == list(oracle.depth(t))
            np.testing.assert_array_equal(out["win"].reshape(n, 2), oracle.conv_window(t, 3))


def test_host_plan_rejects_malformed_trees():
    assert host_plan([np.array([0, 0], np.int32)])[0] == -2
    assert host_plan([np.array([-1, 1], np.int32)])[0] == -2
    assert host_plan([np.array([-1, 0, 5], np.int32)])[0] == -2
    assert host_plan([synth.chain(10)], max_levels=9)[0] == -5       # 10 levels > 9
    assert host_plan([synth.chain(10)], max_levels=10)[0] == 0
    assert host_plan([synth.chain(8)], n_max=7)[0] in (-2, -3)         # tree larger than n_max
    assert host_plan([synth.chain(3)], W=9)[0] == -3                    # W > DDT_MAX_W


def _dummy_plan(B=1, n=4, n_max=4, W=4):
    z = np.zeros(64, np.int64)
    return ddt.plan_struct(B, n, n_max, W, z, z, z, z, z, z)


def test_device_entry_points_validate_before_launch():
    L = ddt.lib()
    P = _dummy_plan()
    bp = ctypes.byref(P)
    one = ctypes.c_void_p(16)
    # gated delta-net: Hv not a multiple of Hk; unsupported dk; dtype
    assert L.ddt_tree_gdn(bp, one, one, one, one, one, one, 3, 4, 128, 128, 1.0, 2, one, None, None, None) == -3
    assert L.ddt_tree_gdn(bp, one, one, one, one, one, one, 2, 4, 96, 128, 1.0, 2, one, None, None, None) == -3
    assert L.ddt_tree_gdn(bp, one, one, one, one, one, one, 2, 4, 128, 128, 1.0, 1, one, None, None, None) == -4
    assert L.ddt_tree_gdn(bp, None, one, one, one, one, one, 2, 4, 128, 128, 1.0, 2, one, None, None, None) == -1
    # conv: channels not a multiple of 8, bad activation
    assert L.ddt_tree_conv(bp, one, one, one, 12, 0, 2, one, None) == -3
    assert L.ddt_tree_conv(bp, one, one, one, 16, 2, 2, one, None) == -1
    # attention: GQA mismatch, small workspace, paged without table for B > 1
    assert L.ddt_tree_attn(bp, one, one, one, None, 0, one, 100, one, one, 6, 4, 256, 0.1, 1, 0,
                           one, one, 0, None) == -3
    assert L.ddt_tree_attn(bp, one, one, one, None, 0, one, 100, one, one, 24, 4, 256, 0.1, 1, 0,
                           one, one, 16, None) == -6
    P2 = _dummy_plan(B=2)
    assert L.ddt_tree_attn(ctypes.byref(P2), one, one, one, None, 0, one, 100, one, one, 24, 4, 256,
                           0.1, 1, 0, one, one, 1 << 30, None) == -1
    assert ddt.ddt_tree_attn_workspace(P, 24, 4, 256, 131072) > 0
    # a batch shares at most 1024 context splits and needs one per sequence
    P3 = _dummy_plan(B=1025)
    assert L.ddt_tree_attn(ctypes.byref(P3), one, one, one, one, 4, one, 100, one, one, 24, 4, 256,
                           0.1, 1, 0, one, one, 1 << 30, None) == -3
    # 8-bit cache attention: head size outside {128, 256}, null scales, small workspace
    q8 = L.ddt_tree_attn_q8
    assert q8(bp, one, one, one, one, one, None, 0, one, 100, one, one, 24, 4, 64, 0.1, 0, one, one,
              1 << 30, None) == -3
    assert q8(bp, one, one, None, one, one, None, 0, one, 100, one, one, 24, 4, 256, 0.1, 0, one, one,
              1 << 30, None) == -1
    assert q8(bp, one, one, one, one, one, None, 0, one, 100, one, one, 24, 4, 256, 0.1, 0, one, one,
              16, None) == -6
    # walk: workspace, dtype
    assert L.ddt_accept_walk(bp, one, 2, 1000, one, one, one, one, one, one, 0, None) == -6
    assert L.ddt_accept_walk(bp, one, 1, 1000, one, one, one, one, one, one, 1 << 20, None) == -4
    # allocation-free walk: more nodes than its static scratch holds, dtype
    big = _dummy_plan(n=4097)
    assert L.ddt_accept_walk_noalloc(ctypes.byref(big), one, 2, 1000, one, one, one, one, one, None) == -3
    assert L.ddt_accept_walk_noalloc(bp, one, 1, 1000, one, one, one, one, one, None) == -4
    assert L.ddt_accept_walk_noalloc(bp, None, 2, 1000, one, one, one, one, one, None) == -1
    # plan struct itself
    assert L.ddt_tree_plan(ctypes.byref(_dummy_plan(n_max=65)), 8, None) == -3
    assert L.ddt_tree_plan(ctypes.byref(_dummy_plan(W=0)), 8, None) == -3
    # commit: bad mode, SELECT/REPLAY shapes
    assert L.ddt_commit_state(bp, one, one, 7, one, 1, 16, 32, 128, 128, 2, 8192, 2, None, 0, 4,
                              256, 1, None, 0, None, None) == -1
    assert L.ddt_commit_state(bp, one, one, 0, one, 1, 16, 30, 128, 128, 2, 8192, 2, None, 0, 4,
                              256, 1, None, 0, None, None) == -3
    # commit with attention layers: the cache's capacity must be given, for a
    # contiguous cache (no page table) as for a paged one
    assert L.ddt_commit_state(bp, one, one, 2, one, 1, 16, 32, 128, 128, 2, 8192, 2, one, 1, 4,
                              256, 1, None, 0, one, None) == -3
    assert L.ddt_commit_state(bp, one, one, 2, one, 1, 16, 32, 128, 128, 2, 8192, 2, one, 1, 4,
                              256, 1, one, 0, one, None) == -3
    assert L.ddt_commit_state(bp, one, one, 2, one, 1, 16, 32, 128, 128, 2, 8192, 2, one, 1, 4,
                              256, 1, None, 4, None, None) == -1   # attention layers need T
    # draft top-K: K outside 1..8, dtype, workspace; tree build: L > 16, N > 64, null output
    ws = ddt.ddt_draft_topk_workspace(1, 16, 151936, 8)
    assert ws > 0 and ddt.ddt_draft_topk_workspace(1, 16, 151936, 9) == 0
    assert L.ddt_draft_topk(one, 1, 16, 151936, 2, 9, one, one, one, one, 1 << 30, None) == -3
    assert L.ddt_draft_topk(one, 1, 16, 151936, 1, 8, one, one, one, one, 1 << 30, None) == -4
    assert L.ddt_draft_topk(one, 1, 16, 151936, 2, 8, one, one, one, one, ws - 1, None) == -6
    assert L.ddt_draft_topk(None, 1, 16, 151936, 2, 8, one, one, one, one, ws, None) == -1
    assert L.ddt_tree_build(one, one, one, 1, 17, 8, 22, one, one, one, one, one, None) == -3
    assert L.ddt_tree_build(one, one, one, 1, 16, 8, 65, one, one, one, one, one, None) == -3
    assert L.ddt_tree_build(one, one, one, 1, 16, 8, 22, one, one, one, one, None, None) == -1
    # fused conv -> delta-net: GQA mismatch, dk, dtype, null gate; LDS of the largest tree fits
    f = L.ddt_tree_conv_gdn
    assert f(bp, one, one, one, 2, one, one, one, 3, 4, 128, 128, 1.0, one, None, None, None, None, None,
             None) == -3
    assert f(bp, one, one, one, 2, one, one, one, 2, 4, 96, 128, 1.0, one, None, None, None, None, None,
             None) == -3
    assert f(bp, one, one, one, 2, one, one, one, 2, 4, 128, 120, 1.0, one, None, None, None, None, None,
             None) == -3
    assert f(bp, one, one, one, 3, one, one, one, 2, 4, 128, 128, 1.0, one, None, None, None, None, None,
             None) == -4
    assert f(bp, one, one, one, 2, None, one, one, 2, 4, 128, 128, 1.0, one, None, None, None, None, None,
             None) == -1
    # ... head counts and d_v travel in 16 bits each
    assert f(bp, one, one, one, 2, one, one, one, 1, 65536, 128, 128, 1.0, one, None, None, None, None, None,
             None) == -3
    assert f(bp, one, one, one, 2, one, one, one, 2, 4, 128, 65552, 1.0, one, None, None, None, None, None,
             None) == -3
    assert 0 < ddt.ddt_tree_conv_gdn_lds(64, 128) <= 160 * 1024
    assert ddt.ddt_tree_conv_gdn_lds(65, 128) == 0 and ddt.ddt_tree_conv_gdn_lds(22, 96) == 0
    # sampled acceptance: temperature, top_k, top_p, dtype, workspace
    sw = ddt.ddt_accept_sample_workspace(P, 151936, 20)
    assert sw > 0 and ddt.ddt_accept_sample_workspace(P, 151936, 33) == 0
    sa = L.ddt_accept_sample
    assert sa(bp, one, 2, 151936, one, one, 0.0, 20, 0.95, one, one, one, one, one, sw, None) == -5
    assert sa(bp, one, 2, 151936, one, one, 1.0, 33, 0.95, one, one, one, one, one, sw, None) == -3
    assert sa(bp, one, 2, 151936, one, one, 1.0, 20, 1.5, one, one, one, one, one, sw, None) == -5
    assert sa(bp, one, 2, 151936, one, one, 1.0, 20, 0.0, one, one, one, one, one, sw, None) == -5
    assert sa(bp, one, 1, 151936, one, one, 1.0, 20, 0.95, one, one, one, one, one, sw, None) == -4
    assert sa(bp, one, 2, 151936, one, one, 1.0, 20, 0.95, one, one, one, one, one, sw - 1, None) == -6
    assert sa(bp, one, 2, 151936, one, None, 1.0, 20, 0.95, one, one, one, one, one, sw, None) == -1
    for c in (-1, -2, -3, -4, -5, -6, -7, 0):
        assert ddt.status_str(c)


def test_q8_binding_rejects_wrong_dtypes():
    import torch
    P = _dummy_plan()
    h = lambda *s, dt=torch.float16: torch.zeros(s, dtype=dt)
    q, Kt, Vt, out = h(1, 24, 128), h(1, 4, 128), h(1, 4, 128), h(1, 24, 128, dt=torch.float32)
    Kq, Vq = h(1, 4, 16, 128, dt=torch.int8), h(1, 4, 128, 16, dt=torch.int8)
    Ks, Vs = h(1, 4, 16), h(1, 4, 16)
    T = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError):
        ddt.ddt_tree_attn_q8(P, q, Kq.half(), Ks, Vq, Vs, None, T, 16, Kt, Vt, out, None)
    with pytest.raises(TypeError):
        ddt.ddt_tree_attn_q8(P, q, Kq, Ks.float(), Vq, Vs, None, T, 16, Kt, Vt, out, None)
    with pytest.raises(TypeError):
        ddt.ddt_tree_attn_q8(P, q, Kq, Ks, Vq, Vs, None, T, 16, Kt, Vt, out.half(), None)


# ---- the host acceptance walk (the fall-back of the validated device walk)
def host_walk(trees, lg, tok):
    par, off = synth.concat_trees(trees)
    B, n = len(trees), len(par)
    n_max = max(len(t) for t in trees)
    status = np.zeros(B, np.int32)
    st = ddt.plan_struct(B, n, n_max, 4, off, par, None, None, None, status)
    am, path = np.empty(n, np.int32), np.empty((B, n_max), np.int32)
    L, bonus = np.empty(B, np.int32), np.empty(B, np.int32)
    ddt.ddt_accept_walk_host(st, lg, tok, am, path, L, bonus)
    return par, off, am, path, L, bonus, status


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_host_walk_matches_oracle(dt):
    trees = [synth.random_tree(synth.rng_for(3, 93, b), s, 10) for b, s in enumerate([22, 64, 1, 8])]
    V = 2048
    lgs, toks = [], []
    for b, t in enumerate(trees):
        lg, tk = synth.logits_and_draft(3, (94, b), t, V, dt, p_match=0.9, plant=(b != 1))
        lgs.append(lg)
        toks.append(tk)
    lg, tok = np.concatenate(lgs), np.concatenate(toks).astype(np.int32)
    tok[30] = V + 1   # never matches; flagged
    par, off, am, path, L, bonus, status = host_walk(trees, lg, tok)
    ref_am = oracle.argmax_rows(lg)
    assert np.array_equal(am, ref_am)
    paths, rL, rb = oracle.accept_walk(par, tok, ref_am, tree_off=off)
    assert np.array_equal(L, rL) and np.array_equal(bonus, rb)
    for b in range(len(trees)):
        assert list(path[b, :rL[b]]) == paths[b] and (path[b, rL[b]:] == -1).all()
    assert list(status) == [0, 4, 0, 0]   # node 30 is in the second tree


def test_host_walk_refuses_bad_arguments():
    trees = [synth.chain(4)]
    lg = np.zeros((4, 8), np.float32)
    tok = np.zeros(4, np.int32)
    with pytest.raises(TypeError):
        host_walk(trees, lg.astype(np.float64), tok)
    with pytest.raises(TypeError):
        host_walk(trees, lg, tok.astype(np.int64))
    bad = [np.array([-1, 0, 2, 1], np.int32)]
    with pytest.raises(ddt.DDTError) as e:
        host_walk(bad, lg, tok)
    assert e.value.code == -2   # DDT_E_TREE
    with pytest.raises(ddt.DDTError) as e:
        host_walk(trees, np.zeros((4, 0), np.float32), tok)
    assert e.value.code == -3   # DDT_E_SHAPE
