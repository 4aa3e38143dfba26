"""Pins for the oracle's verify argmax and acceptance walk (CPU only)."""
import itertools

import numpy as np

import oracle
import synth


def test_argmax_first_occurrence_and_nan():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((6, 50)).astype(np.float32)
    X[0, [3, 17, 40]] = 9.0                 # tie -> 3
    X[1, :] = -np.inf                       # all -inf -> 0
    X[2, 0] = np.nan
    X[2, 5] = 7.0                           # NaN never wins -> 5
    X[3, :] = np.nan                        # all NaN -> 0
    X[4, [10, 11]] = [0.0, -0.0]
    X[4, :10] = -1
    X[4, 12:] = -1                          # +0 and -0 compare equal -> 10
    a = oracle.argmax_rows(X)
    assert list(a[:5]) == [3, 0, 5, 0, 10]
    assert a[5] == np.argmax(X[5])
    bf = synth.store(rng.standard_normal((40, 151936)), "bf16")
    np.testing.assert_array_equal(oracle.argmax_rows(bf), np.argmax(oracle.num.f64(bf), axis=1))


def test_bf16_rows_do_tie():
    # sanity for the tie rule: N(0,1) bf16 rows of full vocabulary often tie at the max
    bf = synth.store(np.random.default_rng(1).standard_normal((64, 151936)), "bf16")
    X = oracle.num.f64(bf)
    ties = sum(int((X[r] == X[r].max()).sum() > 1) for r in range(64))
    assert ties >= 1


def _brute_longest(par, tok, amax):
    n = len(par)
    best = [0]
    for i in range(n):
        p = oracle.root_path(par, i)
        if all(tok[p[t + 1]] == amax[p[t]] for t in range(len(p) - 1)) and len(p) > len(best):
            best = p
    return best


def test_walk_is_longest_matching_path_exhaustive():
    rng = np.random.default_rng(2)
    for n in range(1, 7):
        for ps in itertools.product(*[range(i) for i in range(1, n)]):
            par = np.array([-1, *ps])
            ch = [[c for c in range(n) if par[c] == u] for u in range(n)]
            for _ in range(3):
                amax = rng.integers(0, 3, n)
                tok = np.zeros(n, dtype=np.int64)
                for u in range(n):   # distinct sibling tokens
                    vals = rng.permutation(6)[:len(ch[u])]
                    for c, t in zip(ch[u], vals):
                        tok[c] = t
                paths, L, bonus = oracle.accept_walk(par, tok, amax)
                assert paths[0] == _brute_longest(par, tok, amax)
                assert L[0] == len(paths[0]) and bonus[0] == amax[paths[0][-1]]


def test_walk_extremes():
    n, V = 22, 1000
    par = synth.random_tree(synth.rng_for(0, 1), n, 8)
    lg, tok = synth.logits_and_draft(0, (1,), par, V, "bf16", p_match=0.0)
    paths, L, _ = oracle.accept_walk(par, tok, oracle.argmax_rows(lg))
    assert L[0] == 1 and paths[0] == [0]
    ch = synth.chain(n)
    lg, tok = synth.logits_and_draft(0, (2,), ch, V, "bf16", p_match=1.0)
    paths, L, bonus = oracle.accept_walk(ch, tok, oracle.argmax_rows(lg))
    assert L[0] == n and paths[0] == list(range(n))


def test_duplicate_sibling_tokens_take_lowest_child():
    par = np.array([-1, 0, 0, 0])
    tok = np.array([0, 5, 7, 7])
    amax = np.array([7, 1, 2, 3])
    paths, L, bonus = oracle.accept_walk(par, tok, amax)
    assert paths[0] == [0, 2] and bonus[0] == 2
