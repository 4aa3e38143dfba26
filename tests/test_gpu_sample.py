"""GPU parity of stochastic tree acceptance (ddt_accept_sample) against the
oracle, through the C ABI.  Samples must equal the oracle's exactly except
where the oracle's decision lies within 1e-5 (relative) of a boundary (a
cumulative mass or the top-p cut): there the GPU's fp32 evaluation may pick
the neighbouring kept token.  The walk must equal the oracle's walk over the
GPU's samples, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sample as S
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import banner, dev, host

pytestmark = pytest.mark.gpu
MARGIN = 1e-5


def make_batch(trees, W, gpu, max_levels=64):
    par, off = synth.concat_trees(trees)
    tb = ddt.TreeBatch(par, off, W, gpu)
    ddt.ddt_tree_plan(tb, max_levels)
    return tb, par, off


def run(gpu, trees, V, dt, seed, T, k, p, lg=None, tok=None, u=None):
    tb, par, off = make_batch(trees, 4, gpu)
    n, B = len(par), len(trees)
    if lg is None:
        ls, ts = [], []
        for b, t in enumerate(trees):
            l_, t_ = synth.logits_and_draft(seed, (110, b), t, V, dt, p_match=0.8)
            ls.append(l_)
            ts.append(t_)
        lg, tok = np.concatenate(ls), np.concatenate(ts).astype(np.int32)
    if u is None:
        u = synth.uniforms(seed, (111,), n)
    i32 = dict(dtype=torch.int32, device=gpu)
    sample = torch.full((n,), -7, **i32)
    path = torch.empty(B, tb.n_max, **i32)
    L, bonus = torch.empty(B, **i32), torch.empty(B, **i32)
    ws = torch.empty(ddt.ddt_accept_sample_workspace(tb, V, k), dtype=torch.uint8, device=gpu)
    ddt.ddt_accept_sample(tb, dev(lg), dev(tok), dev(u), T, k, p, sample, path, L, bonus, ws)
    torch.cuda.synchronize()
    return tb, par, off, lg, tok, u, host(sample), host(path), host(L), host(bonus)


def check(par, off, lg, tok, u, T, k, p, y, path, L, bonus):
    y_ref, marg = S.sample_tokens(lg, u, T, k, p)
    for r in range(len(y)):
        if y_ref[r] < 0:
            assert y[r] == 0  # no finite logit: flagged, token 0
            continue
        if y[r] != y_ref[r]:
            assert marg[r] < MARGIN, (r, y[r], y_ref[r], marg[r])
            order, _ = S.filtered_dist(lg[r], T, k, 1.0)
            assert y[r] in set(order.tolist()), (r, y[r])
    paths, L_ref, b_ref = oracle.accept_walk(par, tok, y.astype(np.int64), tree_off=off)
    assert np.array_equal(L, L_ref) and np.array_equal(bonus, b_ref)
    for b in range(len(L)):
        assert list(path[b][:L[b]]) == list(paths[b])
        assert (path[b][L[b]:] == -1).all()
    return int((y == y_ref).sum())


CASES = {
    "vocab3001_bf16": dict(sizes=[22], V=3001, dt="bf16", T=1.0, k=20, p=0.95),
    "full_vocab_bf16": dict(sizes=[22], V=synth.VOCAB, dt="bf16", T=1.0, k=20, p=0.95),
    "f32_ragged_batch": dict(sizes=[9, 22, 1], V=5003, dt="f32", T=0.7, k=32, p=1.0),
    "bf16_batch_k8_hot": dict(sizes=[16, 30], V=20000, dt="bf16", T=1.6, k=8, p=0.8),
}


@pytest.mark.parametrize("case", list(CASES))
def test_sample_walk(gpu, case):
    c = CASES[case]
    banner(f"sample {case}")
    trees = [synth.random_tree(synth.rng_for(12, 112, b), s, 8) for b, s in enumerate(c["sizes"])]
    tb, par, off, lg, tok, u, y, path, L, bonus = run(gpu, trees, c["V"], c["dt"], 12, c["T"], c["k"], c["p"])
    assert not host(tb.status).any()
    same = check(par, off, lg, tok, u, c["T"], c["k"], c["p"], y, path, L, bonus)
    assert same >= len(y) - 1  # at most a rare boundary case differs
    assert (L >= 1).all()


def test_top_k_one_is_the_greedy_walk(gpu):
    banner("sample top_k 1 == greedy")
    trees = [synth.random_tree(synth.rng_for(13, 113), 22, 8)]
    tb, par, off, lg, tok, u, y, path, L, bonus = run(gpu, trees, synth.VOCAB, "bf16", 13, 1.0, 1, 0.95)
    n = len(par)
    i32 = dict(dtype=torch.int32, device=gpu)
    am = torch.empty(n, **i32)
    p2 = torch.empty(1, tb.n_max, **i32)
    L2, b2 = torch.empty(1, **i32), torch.empty(1, **i32)
    ws = torch.empty(ddt.ddt_accept_walk_workspace(tb, synth.VOCAB), dtype=torch.uint8, device=gpu)
    ddt.ddt_accept_walk(tb, dev(lg), dev(tok), am, p2, L2, b2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y, host(am))
    assert np.array_equal(path, host(p2)) and np.array_equal(L, host(L2)) and np.array_equal(bonus, host(b2))


def test_flat_nan_and_dead_rows(gpu):
    """Flat rows (every logit tied: the lowest indices fill the top-k), rows
    with NaN and -inf, and a row with no finite logit (flagged)."""
    banner("sample flat / NaN / dead rows")
    V = 4096
    trees = [synth.random_tree(synth.rng_for(14, 114, b), s, 8) for b, s in enumerate([12, 10])]
    par, off = synth.concat_trees(trees)
    n = len(par)
    r = synth.rng_for(14, 115)
    lg = r.standard_normal((n, V)).astype(np.float32)
    lg[0, :] = 0.25                        # flat
    lg[1, ::3] = np.nan                    # NaN never kept
    lg[2, :] = -np.inf
    lg[2, 77] = 1.0                        # one finite logit
    lg[3, 100:] = -np.inf                  # fewer finite logits than k after the first chunk
    lg[off[1] + 4, :] = -np.inf            # dead row in the second tree
    tok = r.integers(0, V, n).astype(np.int32)
    u = synth.uniforms(14, (116,), n)
    tb, par, off, lg, tok, u, y, path, L, bonus = run(gpu, trees, V, "f32", 14, 1.0, 20, 0.9, lg=lg, tok=tok, u=u)
    st = host(tb.status)
    assert st[0] == 0 and st[1] & ddt.DDT_ST_ARGMAX
    assert y[0] < 20 and y[2] == 77
    check(par, off, lg, tok, u, 1.0, 20, 0.9, y, path, L, bonus)


def test_cold_and_sharp_limits(gpu):
    """A tiny temperature or a tiny top_p leaves only the argmax."""
    banner("sample tiny temperature / top_p")
    trees = [synth.random_tree(synth.rng_for(15, 117), 22, 8)]
    for T, p in ((1e-3, 0.95), (1.0, 1e-6)):
        tb, par, off, lg, tok, u, y, path, L, bonus = run(gpu, trees, 3001, "bf16", 15, T, 20, p)
        assert np.array_equal(y, oracle.argmax_rows(lg))
