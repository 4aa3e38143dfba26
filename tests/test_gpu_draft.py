"""Draft top-K / log-sum-exp and DDTree construction on the GPU against the
oracle, through the C ABI.

Integer results (indices, parents, tokens, node counts) must be equal.  The
top-K logits are copies of stored values and must be equal too; the
log-sum-exp is a float reduction (fp32 against fp64) held to 1e-5.  The
tree's order is decided by float sums: the GPU adds log-probabilities in
fp32, the oracle in fp64, so where two candidates' oracle scores lie within
fp32 rounding of each other either order is correct.  Where every gap that
decides the tree exceeds that margin the trees must be identical; otherwise
the GPU tree must be a valid tree of the same size whose scores (recomputed
in fp64) match the oracle's selection within the margin."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import banner, dev, host

pytestmark = pytest.mark.gpu

MARGIN = 1e-4   # fp32 sums of <= 16 log-probabilities, |score| < 200, differ from fp64 by far less


def run_topk(gpu, lg, K):
    B, L, V = lg.shape
    t = dev(lg, gpu)
    idx = torch.empty(B, L, K, dtype=torch.int32, device=gpu)
    val = torch.empty(B, L, K, dtype=torch.float32, device=gpu)
    lse = torch.empty(B, L, dtype=torch.float32, device=gpu)
    ws = torch.empty(ddt.ddt_draft_topk_workspace(B, L, V, K), dtype=torch.uint8, device=gpu)
    ddt.ddt_draft_topk(t, K, idx, val, lse, ws)
    return idx, val, lse


def run_tree(gpu, idx, val, lse, N, roots):
    B = idx.shape[0]
    i32 = dict(dtype=torch.int32, device=gpu)
    parent, tok = torch.full((B, N), -7, **i32), torch.full((B, N), -7, **i32)
    score = torch.empty(B, N, dtype=torch.float32, device=gpu)
    n = torch.empty(B, **i32)
    ddt.ddt_tree_build(idx, val, lse, N, dev(np.asarray(roots, np.int32), gpu), parent, tok, score, n)
    torch.cuda.synchronize()
    return host(parent), host(tok), host(score), host(n)


def check_topk(lg, K, idx, val, lse):
    for b in range(lg.shape[0]):
        ri, rv, rl = oracle.draft_topk(lg[b], K)
        np.testing.assert_array_equal(host(idx)[b], ri)
        np.testing.assert_array_equal(host(val)[b].astype(np.float64), rv)
        got = host(lse)[b].astype(np.float64)
        fin = np.isfinite(rl)
        np.testing.assert_array_equal(np.isfinite(got), fin)
        assert np.abs(got[fin] - rl[fin]).max(initial=0) < 1e-5


def check_tree(ri, rv, rl, N, root, p, t, s, n):
    """GPU tree (p, t, s, n) for one sequence against the oracle's."""
    lp = oracle.log_probs(rv, rl)
    rp, rt, rs, rd, rk = oracle.build_tree(ri, lp, N, root)
    assert n == len(rp)
    p, t, s = p[:n], t[:n], s[:n]
    assert p[0] == -1 and t[0] == root
    # node ranks of the GPU tree, from its parents and tokens
    L, K = ri.shape
    rank, depth = [()], [0]
    for i in range(1, n):
        assert 0 <= p[i] < i
        d = depth[p[i]]
        hits = [k for k in range(K) if ri[d, k] == t[i]]
        assert len(hits) == 1, "token is not a candidate of its position"
        rank.append(rank[p[i]] + (hits[0],))
        depth.append(d + 1)
    assert len(set(rank)) == n, "a candidate was taken twice"
    score64 = np.array([sum(lp[j, r[j]] for j in range(len(r))) for r in rank])
    assert np.abs(score64 - s).max() < MARGIN
    # the decisions: consecutive kept keys, and the last kept against the best left out
    ordered = [(-rs[i], rk[i]) for i in range(1, len(rk))]
    kept = set(rk)
    left = [(-(rs[rk.index(x)] + lp[len(x), k]), x + (k,)) for x in rk if len(x) < L
            for k in range(K) if np.isfinite(lp[len(x), k]) and x + (k,) not in kept]
    sc = [-o[0] for o in ordered] + ([-min(left)[0]] if left else [])
    gaps = [abs(a - b) for a, b in zip(sc, sc[1:]) if a != b]
    exact_ties_only = all(g > MARGIN for g in gaps)
    if exact_ties_only:
        assert p.tolist() == rp.tolist() and t.tolist() == rt.tolist()
    else:   # near ties: the same scores were kept, in an order valid within the margin
        np.testing.assert_allclose(np.sort(score64), np.sort(rs), atol=MARGIN)
    return exact_ties_only


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("V", [3001, 4096])
def test_topk_small_vocab_ragged_and_special_values(gpu, dt, V):
    banner(f"draft top-K V={V} {dt}")
    rng = np.random.default_rng(V)
    x = rng.standard_normal((2, 5, V)).astype(np.float32) * 2
    x[0, 0, [7, 900, V - 1]] = 6.0          # tie at the top, lower index first
    x[0, 1, :] = np.round(x[0, 1, :])       # many ties everywhere
    x[0, 2, 5] = np.nan                     # NaN never chosen, ignored by LSE
    x[0, 2, 6] = 50.0
    x[1, 3, :] = -np.inf                    # no candidate at all
    x[1, 4, :] = -np.inf
    x[1, 4, [2, 11]] = [1.0, 3.0]           # fewer finite logits than K
    lg = synth.store(x, dt)
    for K in (1, 3, 8):
        idx, val, lse = run_topk(gpu, lg, K)
        torch.cuda.synchronize()
        check_topk(lg, K, idx, val, lse)


def test_tree_uniform_logits_exact_ties(gpu):
    banner("draft tree: uniform logits, ties resolved by candidate ranks")
    lg = np.zeros((1, 3, 20), np.float32)
    idx, val, lse = run_topk(gpu, lg, 3)
    p, t, s, n = run_tree(gpu, idx, val, lse, 9, [4])
    assert n[0] == 9
    assert p[0].tolist() == [-1, 0, 0, 0, 1, 1, 1, 2, 2]
    assert t[0].tolist() == [4, 0, 1, 2, 0, 1, 2, 0, 1]


@pytest.mark.parametrize("K,N", [(1, 22), (2, 22), (8, 22), (8, 64), (3, 1)])
def test_tree_matches_oracle(gpu, K, N):
    banner(f"draft tree K={K} N={N}")
    B, L, V = 3, 16, 2000
    lg = np.stack([synth.draft_logits(20 + b, (K, N), L, V, "f32") for b in range(B)])
    idx, val, lse = run_topk(gpu, lg, K)
    roots = [11, 12, 13]
    p, t, s, n = run_tree(gpu, idx, val, lse, N, roots)
    for b in range(B):
        ri, rv, rl = oracle.draft_topk(lg[b], K)
        check_tree(ri, rv, rl, N, roots[b], p[b], t[b], s[b], int(n[b]))


def test_tree_stops_at_a_dead_position(gpu):
    banner("draft tree: position without finite logits")
    lg = synth.draft_logits(3, (9,), 6, 500, "f32")[None]
    lg[0, 2, :] = np.nan
    idx, val, lse = run_topk(gpu, lg, 2)
    p, t, s, n = run_tree(gpu, idx, val, lse, 50, [1])
    assert n[0] == 7 and max(oracle.depth(p[0][:7])) == 2


@pytest.mark.parametrize("B", [1, 8])
def test_full_vocab_workload_and_plan(gpu, B):
    """The measured workload: L=16 draft positions, 151,936-token bf16 logits,
    K=8, budget 22; the trees then go straight into the verify plan."""
    c = synth.DRAFT
    L, K, N, V = c["L"], c["K"], c["N"], synth.VOCAB
    banner(f"draft top-K + tree, full vocabulary, B={B}")
    lg = np.stack([synth.draft_logits(0, (40, b), L, V, "bf16") for b in range(B)])
    idx, val, lse = run_topk(gpu, lg, K)
    roots = list(range(100, 100 + B))
    p, t, s, n = run_tree(gpu, idx, val, lse, N, roots)
    check_topk(lg, K, idx, val, lse)
    exact = 0
    for b in range(B):
        ri, rv, rl = oracle.draft_topk(lg[b], K)
        exact += check_tree(ri, rv, rl, N, roots[b], p[b], t[b], s[b], int(n[b]))
    assert exact >= B - 1   # near ties are rare on these inputs
    assert (n == N).all()
    tb = ddt.TreeBatch(p.reshape(-1), [N * b for b in range(B + 1)], 4, gpu)
    ddt.ddt_tree_plan(tb, 16)
    torch.cuda.synchronize()
    assert not host(tb.status).any()
