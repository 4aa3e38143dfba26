"""Pins for the oracle's sampler and stochastic tree acceptance (CPU only)."""
import numpy as np
from scipy.special import softmax

import oracle
from oracle import sample as S
import synth


def _grid(M=20000):
    return (np.arange(M) + 0.5) / M


def test_top_k_one_and_tiny_top_p_are_argmax():
    r = synth.rng_for(1, 2)
    for _ in range(20):
        row = r.standard_normal(500).astype(np.float32)
        am = int(np.argmax(row))
        for u in (0.0, 0.37, 0.999):
            assert S.sample_row(row, u, 1.0, 1, 0.95)[0] == am
            assert S.sample_row(row, u, 0.7, 20, 1e-9)[0] == am


def test_grid_histogram_is_softmax_over_kept_tokens():
    # no filtering (top_k = V, top_p = 1): the share of the u grid mapped to
    # token i is softmax(logits / T)_i (scipy), to within the grid step
    r = synth.rng_for(3, 4)
    V, T = 12, 0.7
    row = r.standard_normal(V)
    g = _grid()
    toks = [S.sample_row(row, u, T, V, 1.0)[0] for u in g]
    hist = np.bincount(toks, minlength=V) / len(g)
    np.testing.assert_allclose(hist, softmax(row / T), atol=2.0 / len(g))


def test_hand_worked_top_p_cut():
    # p = (0.5, 0.3, 0.2) at T = 1; top_p 0.79 keeps the first two (0.5 + 0.3
    # reaches it), renormalised to (0.625, 0.375); top_p 0.81 keeps all three
    row = np.log(np.array([0.5, 0.3, 0.2]))
    assert S.sample_row(row, 0.62, 1.0, 3, 0.79)[0] == 0
    assert S.sample_row(row, 0.63, 1.0, 3, 0.79)[0] == 1
    assert S.sample_row(row, 0.999, 1.0, 3, 0.79)[0] == 1
    assert S.sample_row(row, 0.999, 1.0, 3, 0.81)[0] == 2
    assert S.sample_row(row, 0.49, 1.0, 3, 0.49)[0] == 0  # 0.5 alone reaches 0.49
    order, p = S.filtered_dist(row, 1.0, 3, 0.79)
    assert list(order) == [0, 1]
    np.testing.assert_allclose(p / p.sum(), [0.625, 0.375])


def test_top_k_limits_the_support_and_ties_take_lower_index():
    r = synth.rng_for(5, 6)
    row = r.standard_normal(300)
    top = set(np.argsort(-row, kind="stable")[:7])
    seen = {S.sample_row(row, u, 1.3, 7, 1.0)[0] for u in _grid(4000)}
    assert seen == top
    flat = np.zeros(50)
    g = _grid(3000)
    toks = [S.sample_row(flat, u, 1.0, 3, 1.0)[0] for u in g]
    np.testing.assert_allclose(np.bincount(toks, minlength=3)[:3] / len(g), [1 / 3] * 3, atol=1e-3)
    assert max(toks) == 2


def test_nan_and_inf_never_sampled():
    row = np.array([np.nan, -np.inf, 0.5, np.nan, 0.1], dtype=np.float32)
    seen = {S.sample_row(row, u, 1.0, 5, 1.0)[0] for u in _grid(1000)}
    assert seen == {2, 4}
    assert S.sample_row(np.full(4, -np.inf), 0.5, 1.0, 4, 1.0)[0] == -1


def test_sampled_walk_follows_matching_children():
    # a chain whose drafts are the samples is accepted whole; a mismatch at
    # depth 3 stops there with that node's sample as the bonus
    n, V = 6, 40
    r = synth.rng_for(7, 8)
    lg = r.standard_normal((n, V)).astype(np.float32)
    u = r.random(n)
    y, _ = S.sample_tokens(lg, u, 1.0, 20, 0.95)
    par = synth.chain(n)
    tok = np.concatenate([[0], y[:-1]]).astype(np.int64)
    paths, L, bonus = oracle.accept_walk(par, tok, y)
    assert L[0] == n and bonus[0] == y[-1]
    tok2 = tok.copy()
    tok2[3] = (y[2] + 1) % V
    paths, L, bonus = oracle.accept_walk(par, tok2, y)
    assert L[0] == 3 and bonus[0] == y[2]


def test_margin_flags_boundaries():
    row = np.log(np.array([0.5, 0.5]))
    t, mg = S.sample_row(row, 0.5, 1.0, 2, 1.0)   # u * R lands on c_0 exactly
    assert mg < 1e-12
    t, mg = S.sample_row(row, 0.25, 1.0, 2, 1.0)
    assert t == 0 and mg > 0.1
