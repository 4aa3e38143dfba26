"""Seeded synthetic inputs for the DDTree tree-verify step.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It only draws random numbers and lays them out in the storage
formats the library takes; it holds none of the verify step's arithmetic
(no plan, conv, recurrence, attention, argmax or walk).

Storage conventions
-------------------
* fp32 arrays are ``np.float32``, fp16 arrays are ``np.float16``.
* bf16 arrays are ``np.uint16`` holding the raw bf16 bit patterns
  (round-to-nearest-even from fp32).  No other input uses ``uint16``, so the
  dtype identifies them.
* Every array is generated from ``np.random.Generator(PCG64(SeedSequence(
  [seed, config, layer, tensor_id, ...])))`` so that any single tensor can be
  regenerated on its own.

Workload shapes follow the pages' serving setup: a DDTree budget of 22 nodes
(lucebox-hub README, "02 · DFlash DDtree", "Implemented here": budget 22 is
the sweet spot; codehub lucebox-hub@main, "Server flags", "--ddtree-budget"
default 22), 32K and 128K committed contexts, and several concurrent
sequences over a paged KV cache (Luce-Org/lucebox README, "Inference Engine
Optimizations": paged attention for concurrent serving).
"""
from __future__ import annotations

import numpy as np

PAGE = 16  # tokens per KV page

# tensor ids used in the seed key
_T_Q, _T_K, _T_V, _T_A, _T_B, _T_S = 1, 2, 3, 4, 5, 6
_T_X, _T_PRE, _T_W = 7, 8, 9
_T_AQ, _T_KC, _T_VC, _T_KT, _T_VT, _T_PT = 10, 11, 12, 13, 14, 15
_T_LOG, _T_TOK, _T_TREE, _T_T = 16, 17, 18, 19
_T_DL, _T_DP, _T_U = 20, 21, 22
_T_KQ, _T_KS, _T_VQ, _T_VS = 23, 24, 25, 26


def rng_for(seed: int, *key: int) -> np.random.Generator:
    """PCG64 stream keyed by (seed, *key)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def store(x, dtype: str) -> np.ndarray:
    """Cast an fp32/fp64 array to a storage dtype: 'f32', 'f16' or 'bf16'."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float16)
    if dtype == "bf16":
        return to_bf16(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# trees (parent-pointer arrays, node 0 is the root, parent[i] < i)
# ----------------------------------------------------------------------------

def random_tree(rng: np.random.Generator, n: int, max_levels: int) -> np.ndarray:
    """parent[i] uniform over the earlier nodes that still have room below
    them, i.e. whose own level is below ``max_levels`` (levels count nodes on
    a root path, so a lone root has one level).  Equivalent to drawing
    parent[i] uniform in [0, i-1] and rejecting draws that break the cap."""
    assert n >= 1 and max_levels >= 1
    parent = np.full(n, -1, dtype=np.int32)
    level = np.zeros(n, dtype=np.int64)
    level[0] = 1
    for i in range(1, n):
        ok = np.nonzero(level[:i] < max_levels)[0]
        if len(ok) == 0:
            raise ValueError("level cap leaves no room for more nodes")
        p = int(ok[rng.integers(0, len(ok))])
        parent[i] = p
        level[i] = level[p] + 1
    return parent


def binary_tree(levels: int) -> np.ndarray:
    """Complete binary tree in breadth-first numbering: parent[i] = (i-1)//2."""
    n = (1 << levels) - 1
    return np.array([-1] + [(i - 1) // 2 for i in range(1, n)], dtype=np.int32)


def chain(n: int) -> np.ndarray:
    """A chain (the non-tree speculative case): parent[i] = i-1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def _children(parent: np.ndarray):
    ch = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        ch[int(parent[i])].append(i)
    return ch


# ----------------------------------------------------------------------------
# per-op inputs
# ----------------------------------------------------------------------------

def _l2n_rows(x: np.ndarray) -> np.ndarray:
    # input recipe: q and k arrive L2-normalised per head
    return x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)


def gdn_inputs(seed, key, n, Hk, Hv, dk, dv, dtype="bf16", B=1):
    """Gated delta-net tree inputs for ``n`` nodes (all sequences together)
    and ``B`` committed states.  q,k ~ N(0,1) L2-normalised per head;
    v ~ N(0,1); beta = sigmoid(N(0,1)); alpha = exp(-softplus(N(0,1)));
    S_c ~ N(0,1) fp32."""
    q = _l2n_rows(rng_for(seed, *key, _T_Q).standard_normal((n, Hk, dk), dtype=np.float32))
    k = _l2n_rows(rng_for(seed, *key, _T_K).standard_normal((n, Hk, dk), dtype=np.float32))
    v = rng_for(seed, *key, _T_V).standard_normal((n, Hv, dv), dtype=np.float32)
    za = rng_for(seed, *key, _T_A).standard_normal((n, Hv)).astype(np.float64)
    zb = rng_for(seed, *key, _T_B).standard_normal((n, Hv)).astype(np.float64)
    alpha = np.exp(-np.logaddexp(0.0, za)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    S = rng_for(seed, *key, _T_S).standard_normal((B, Hv, dv, dk), dtype=np.float32)
    return dict(q=store(q, dtype), k=store(k, dtype), v=store(v, dtype),
                alpha=store(alpha, dtype), beta=store(beta, dtype), S_c=S)


def conv_inputs(seed, key, n, C, W, dtype="bf16", B=1):
    """Tree conv inputs: x [n][C], committed prefix [B][W-1][C] (oldest
    first), depthwise weights w [C][W]; all N(0,1)."""
    x = rng_for(seed, *key, _T_X).standard_normal((n, C), dtype=np.float32)
    pre = rng_for(seed, *key, _T_PRE).standard_normal((B, W - 1, C), dtype=np.float32)
    w = rng_for(seed, *key, _T_W).standard_normal((C, W), dtype=np.float32)
    return dict(x=store(x, dtype), prefix=store(pre, dtype), w=store(w, dtype))


def fused_inputs(seed, key, n, Hk, Hv, dk, dv, W, dtype="bf16", B=1):
    """Inputs of the fused conv -> delta-net layer: conv x / prefix / w over
    C = 2*Hk*dk + Hv*dv channels as conv_inputs draws them (stored in
    ``dtype``), fp32 gates and the committed state as gdn_inputs draws them."""
    C = 2 * Hk * dk + Hv * dv
    d = conv_inputs(seed, key, n, C, W, dtype, B)
    g = gdn_inputs(seed, key, n, Hk, Hv, dk, dv, "f32", B)
    d.update(alpha=g["alpha"], beta=g["beta"], S_c=g["S_c"])
    return d


def uniforms(seed, key, n):
    """One uniform in [0, 1) per tree node: the random draws of stochastic
    acceptance, passed to both sides as inputs."""
    return rng_for(seed, *key, _T_U).random(n).astype(np.float32)


def page_layout(seed, key, T, n_nodes, page=PAGE, shuffle=True):
    """Page table for sequences with committed lengths ``T`` and room for
    ``n_nodes`` more tokens each (the commit appends up to that many).

    Returns (page_table [B][max_pages] int32, n_pages).  Pages are a seeded
    permutation of the pool when ``shuffle``; otherwise consecutive."""
    T = np.asarray(T, dtype=np.int64)
    n_nodes = np.asarray(n_nodes, dtype=np.int64)
    need = (T + n_nodes + page - 1) // page
    total = int(need.sum())
    perm = rng_for(seed, *key, _T_PT).permutation(total) if shuffle else np.arange(total)
    mp = int(need.max())
    pt = np.zeros((len(T), mp), dtype=np.int32)
    o = 0
    for b in range(len(T)):
        pt[b, :need[b]] = perm[o:o + need[b]]
        o += int(need[b])
    return pt, total


def kv_pool(seed, key, n_pages, Hkv, D, dtype="f16", page=PAGE):
    """Paged KV pool, N(0,1).  K pages are [n_pages][Hkv][page][D]; V pages are
    [n_pages][Hkv][D][page] (each page stores V with the head dimension
    outermost so that a page's 16 values of one channel are contiguous)."""
    K = rng_for(seed, *key, _T_KC).standard_normal((n_pages, Hkv, page, D), dtype=np.float32)
    V = rng_for(seed, *key, _T_VC).standard_normal((n_pages, Hkv, D, page), dtype=np.float32)
    return store(K, dtype), store(V, dtype)


def kv_pool_q8(seed, key, n_pages, Hkv, D, page=PAGE, ksc=(0.015, 0.035), vsc=(0.015, 0.035), log2=False):
    """Paged 8-bit KV pool (the layouts of ``kv_pool``, int8) and one fp16 scale
    per token and KV head: Kq [n_pages][Hkv][page][D], Vq [n_pages][Hkv][D][page],
    Ksc and Vsc [n_pages][Hkv][page].  Codes are N(0, 40) rounded and clipped to
    +-127; scales are uniform in ``ksc`` / ``vsc`` (default [0.015, 0.035], so
    code * scale is about N(0, 1)), or with ``log2`` 2**u for u uniform in the
    given range of exponents."""
    def codes(tag, shape):
        x = np.rint(rng_for(seed, *key, tag).normal(0.0, 40.0, shape))
        return np.clip(x, -127, 127).astype(np.int8)

    def scales(tag, rng_):
        u = rng_for(seed, *key, tag).uniform(rng_[0], rng_[1], (n_pages, Hkv, page))
        return (np.exp2(u) if log2 else u).astype(np.float16)
    return dict(Kq=codes(_T_KQ, (n_pages, Hkv, page, D)), Ksc=scales(_T_KS, ksc),
                Vq=codes(_T_VQ, (n_pages, Hkv, D, page)), Vsc=scales(_T_VS, vsc))


def attn_inputs(seed, key, n, Hq, Hkv, D, dtype="f16"):
    """Tree-node queries and draft K/V, N(0,1): q [n][Hq][D], Kt/Vt [n][Hkv][D]."""
    q = rng_for(seed, *key, _T_AQ).standard_normal((n, Hq, D), dtype=np.float32)
    Kt = rng_for(seed, *key, _T_KT).standard_normal((n, Hkv, D), dtype=np.float32)
    Vt = rng_for(seed, *key, _T_VT).standard_normal((n, Hkv, D), dtype=np.float32)
    return dict(q=store(q, dtype), Kt=store(Kt, dtype), Vt=store(Vt, dtype))


def logits_and_draft(seed, key, parent, V, dtype="bf16", p_match=0.8, plant=True):
    """Target logits [n][V] ~ N(0,1) and draft tokens [n] for one tree.

    With ``plant`` every row gets one entry raised to 8.0 at a seeded token
    (far above any N(0,1) draw, so that token is the row's maximum by
    construction), and for each internal node one uniformly chosen child
    carries that token with probability ``p_match``.  All other children get
    distinct tokens that differ from the planted one.  This fixes the
    expected acceptance without computing anything from the logits.
    Without ``plant`` the logits are pure N(0,1) (in bf16 many rows then
    hold ties at their maximum) and sibling tokens are distinct uniform
    draws."""
    parent = np.asarray(parent)
    n = len(parent)
    lg = rng_for(seed, *key, _T_LOG).standard_normal((n, V), dtype=np.float32)
    r = rng_for(seed, *key, _T_TOK)
    target = r.integers(0, V, n)
    if plant:
        lg[np.arange(n), target] = 8.0
    tok = np.zeros(n, dtype=np.int32)
    tok[0] = r.integers(0, V)
    for u, ch in enumerate(_children(parent)):
        if not ch:
            continue
        used = {int(target[u])} if plant else set()
        hit = -1
        if plant and r.random() < p_match:
            hit = ch[int(r.integers(0, len(ch)))]
            tok[hit] = target[u]
        for c in ch:
            if c == hit:
                continue
            while True:
                t = int(r.integers(0, V))
                if t not in used:
                    break
            used.add(t)
            tok[c] = t
    return store(lg, dtype), tok


def draft_logits(seed, key, L, V, dtype="bf16"):
    """Draft logits [L][V] for one block of L draft positions: N(0,1) with,
    per position, 1 to 4 planted contenders raised by 4 to 9 (a confident
    drafter has a few likely tokens per position; how many and how far ahead
    is drawn at random), at distinct seeded tokens."""
    lg = rng_for(seed, *key, _T_DL).standard_normal((L, V), dtype=np.float32)
    r = rng_for(seed, *key, _T_DP)
    for i in range(L):
        m = int(r.integers(1, 5))
        toks = r.choice(V, size=m, replace=False)
        lg[i, toks] += r.uniform(4.0, 9.0, size=m).astype(np.float32)
    return store(lg, dtype)


DRAFT = dict(name="draft_tree_b8_l16_k8_n22", B=8, L=16, K=8, N=22)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

VOCAB = 151936

TINY = dict(name="tiny", Hk=2, Hv=2, dk=16, dv=16, C=64, W=4, Hq=2, Hkv=1, D=16, T=64,
            parent=[-1, 0, 0, 1, 1, 2, 2], dtype_gdn="f32", dtype_attn="f32")
LAYER_GDN = dict(name="gdn_conv_n22", N=22, levels=8, Hk=16, Hv=32, dk=128, dv=128, C=8192, W=4)
LAYER_ATTN = dict(name="attn_t32k_n22", N=22, levels=8, Hq=24, Hkv=4, D=256, T=32768)
STACK = dict(name="stack_48gdn_16attn_t128k_n22", N=22, levels=8, n_gdn=48, n_attn=16,
             T=131072, Hk=16, Hv=32, dk=128, dv=128, C=8192, W=4, Hq=24, Hkv=4, D=256)
BATCHED = dict(name="batched_8seq_paged", B=8, budgets=(8, 16, 22, 32, 64), levels=10,
               T_lo=2048, T_hi=65536, n_gdn=8, n_attn=4,
               Hk=16, Hv=32, dk=128, dv=128, C=8192, W=4, Hq=24, Hkv=4, D=256)


def batched_shape(seed):
    """Per-sequence budgets and contexts of the batched workload."""
    r = rng_for(seed, 4, _T_T)
    budgets = r.choice(np.array(BATCHED["budgets"]), size=BATCHED["B"])
    T = r.integers(BATCHED["T_lo"], BATCHED["T_hi"] + 1, size=BATCHED["B"])
    return budgets.astype(np.int64), T.astype(np.int64)


def batched_trees(seed):
    budgets, T = batched_shape(seed)
    trees = [random_tree(rng_for(seed, 4, _T_TREE, b), int(budgets[b]), BATCHED["levels"])
             for b in range(len(budgets))]
    return trees, T


def concat_trees(trees):
    """Concatenate per-sequence parent arrays; returns (parent, tree_off)."""
    off = np.zeros(len(trees) + 1, dtype=np.int32)
    for b, t in enumerate(trees):
        off[b + 1] = off[b] + len(t)
    return np.concatenate([np.asarray(t, dtype=np.int32) for t in trees]), off
