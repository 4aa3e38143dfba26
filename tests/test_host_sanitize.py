"""The library's host-side code (csrc/host.cpp: the plan fields check, the
host tree plan and the host acceptance walk) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on arrays of exactly the stated sizes, so
that any read or write past one, and any undefined operation, stops the
driver.  Its outputs are compared with the oracle; malformed trees must be
refused without a read out of bounds."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_verification_ddtree_amd", "csrc")
DDT_E_TREE, DDT_E_RANGE, DDT_E_SHAPE, DDT_E_DTYPE = -2, -5, -3, -4


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("host") / "host_driver")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "host_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, text):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stdout.split("\n")


def ints(a):
    return " ".join(str(int(x)) for x in np.asarray(a).ravel())


def plan_case(par, off, n_max, W, max_levels, n_total=None):
    n_total = len(par) if n_total is None else n_total
    return f"plan {len(off) - 1} {n_total} {n_max} {W} {max_levels}\n{ints(off)}\n{ints(par)}\n"


def walk_case(par, off, n_max, V, lg, tok):
    if lg.dtype == np.uint16:
        dt, bits = 2, lg
    else:
        dt, bits = 0, lg.astype(np.float32).view(np.uint32)
    return (f"walk {len(off) - 1} {len(par)} {n_max} {V} {dt}\n{ints(off)}\n{ints(par)}\n{ints(tok)}\n"
            f"{ints(bits)}\n")


def test_host_plan_under_sanitizers(driver):
    cases, expect = [], []
    for seed in range(4):
        sizes = [1, 7, 22, 64][: seed + 1] + [33]
        trees = [synth.random_tree(synth.rng_for(seed, 90, b), s, 10) for b, s in enumerate(sizes)]
        par, off = synth.concat_trees(trees)
        for W in (1, 4, 8):
            cases.append(plan_case(par, off, 64, W, 64))
            expect.append(("ok", trees, W))
    chain = synth.chain(12)
    cases.append(plan_case(chain, [0, 12], 12, 4, 11))       # 12 levels over a cap of 11
    expect.append(("rc", DDT_E_RANGE))
    bad = np.array(synth.chain(8)); bad[0] = 0
    cases.append(plan_case(bad, [0, 8], 8, 4, 64))          # root with a parent
    expect.append(("rc", DDT_E_TREE))
    bad = np.array(synth.chain(8)); bad[5] = 5
    cases.append(plan_case(bad, [0, 8], 8, 4, 64))          # parent not before the node
    expect.append(("rc", DDT_E_TREE))
    two = np.concatenate([synth.chain(5), synth.chain(3)])
    cases.append(plan_case(two, [0, 7, 8], 64, 4, 64))      # second tree starts inside the first
    expect.append(("rc", DDT_E_TREE))
    cases.append(plan_case(two, [0, 10, 8], 64, 4, 64))     # first tree runs past n_total
    expect.append(("rc", DDT_E_TREE))
    # ... with parents that are valid up to the last node: a check that only
    # looked at the parents would read past the array
    cases.append(plan_case(synth.chain(8), [0, 10, 8], 64, 4, 64))
    expect.append(("rc", DDT_E_TREE))
    cases.append(plan_case(two, [0, 5, 8], 4, 4, 64))       # a tree above n_max
    expect.append(("rc", DDT_E_TREE))
    cases.append(plan_case(two, [0, 5, 8], 65, 4, 64))      # n_max above the node limit
    expect.append(("rc", DDT_E_SHAPE))
    out = run(driver, "".join(cases))
    k = 0
    for e in expect:
        rc = int(out[k].split()[1])
        k += 1
        if e[0] == "rc":
            assert rc == e[1]
            continue
        assert rc == 0
        _, trees, W = e
        W1 = max(W - 1, 1)
        depth = np.array(out[k].split(), np.int64)
        anc = np.array(out[k + 1].split(), np.uint64)
        win = np.array(out[k + 2].split(), np.int64).reshape(-1, W1)
        k += 3
        o = 0
        for t in trees:
            n = len(t)
            assert list(depth[o:o + n]) == list(oracle.depth(t))
            assert list(anc[o:o + n]) == [int(a) for a in oracle.ancestor_mask(t)]
            if W > 1:
                assert np.array_equal(win[o:o + n], oracle.conv_window(t, W))
            o += n


def walk_inputs(seed, trees, V, dt):
    lgs, toks = [], []
    for b, t in enumerate(trees):
        lg, tk = synth.logits_and_draft(seed, (91, b), t, V, dt, p_match=0.8, plant=(b % 2 == 0))
        lgs.append(lg)
        toks.append(tk)
    return np.concatenate(lgs), np.concatenate(toks).astype(np.int32)


def test_host_walk_under_sanitizers(driver):
    cases, expect = [], []
    for seed, (V, dt) in enumerate([(50, "bf16"), (1001, "f32"), (3000, "bf16"), (7, "f32")]):
        sizes = [22, 1, 64, 8][: 2 + seed % 3]
        trees = [synth.random_tree(synth.rng_for(seed, 92, b), s, 10) for b, s in enumerate(sizes)]
        par, off = synth.concat_trees(trees)
        lg, tok = walk_inputs(seed, trees, V, dt)
        if seed == 1:   # NaN rows and entries, -0 against +0, out-of-range tokens
            lg[0, :] = np.nan
            lg[1, 3] = np.nan
            lg[2, :] = -1.0
            lg[2, [4, 9]] = [0.0, -0.0]
            tok[3] = V
            tok[4] = -2
        cases.append(walk_case(par, off, max(sizes), V, lg, tok))
        expect.append((par, off, lg, tok, V))
    tree = synth.chain(4)
    cases.append(walk_case(tree, [0, 4], 4, 0, np.zeros((4, 0), np.float32), np.zeros(4, np.int32)))
    expect.append(("rc", DDT_E_SHAPE))
    bad = np.array(synth.chain(4)); bad[2] = 3
    cases.append(walk_case(bad, [0, 4], 4, 5, np.zeros((4, 5), np.float32), np.zeros(4, np.int32)))
    expect.append(("rc", DDT_E_TREE))
    out = run(driver, "".join(cases))
    k = 0
    for e in expect:
        rc = int(out[k].split()[1])
        k += 1
        if isinstance(e[0], str):
            assert rc == e[1]
            continue
        assert rc == 0
        par, off, lg, tok, V = e
        B, n_max = len(off) - 1, int(np.diff(off).max())
        am = np.array(out[k].split(), np.int64)
        path = np.array(out[k + 1].split(), np.int64).reshape(B, n_max)
        rows = [list(map(int, out[k + 2 + b].split())) for b in range(B)]
        k += 2 + B
        ref_am = oracle.argmax_rows(lg)
        assert np.array_equal(am, ref_am)
        paths, rL, rb = oracle.accept_walk(par, tok, ref_am, tree_off=off)
        for b in range(B):
            L, bonus, st = rows[b]
            assert (L, bonus) == (rL[b], rb[b])
            assert list(path[b, :L]) == paths[b] and (path[b, L:] == -1).all()
            o, e_ = off[b], off[b + 1]
            bad_tok = any(not (0 <= tok[c] < V) for c in range(o + 1, e_))
            assert st == (4 if bad_tok else 0)
