"""Tree-masked attention over a (paged) KV cache (oracle; test infrastructure).

Each tree node attends to every committed cache token of its sequence plus
the draft tokens on its own root path (itself included); this is what
verifying the whole tree in one pass means when each node must see exactly
the sequence ``context ++ root path`` (lucebox-hub README, "02 · DFlash
DDtree", "Algorithms used").  Attention is full, no window
(codehub lucebox-hub@main, "Server flags", --fa-window default 0), and the
cache may be paged (Luce-Org/lucebox README, "Inference Engine
Optimizations", paged attention).

Readings: q head h uses KV head h // (Hq // Hkv); scale = 1/sqrt(D); no
softcap, sink or window; draft K/V of the tree live in their own buffer
(Kt, Vt) and only enter the cache at commit.

Cache storage (shared input format): K pages [P][Hkv][PAGE][D]; V pages
[P][Hkv][D][PAGE]; token t of sequence b lives in page page_table[b][t // PAGE]
at slot t % PAGE (page_table None: one sequence, page t // PAGE).
"""
import numpy as np

from .num import f64
from .tree import root_path


def gather_cache(Kp, Vp, page_table, b, g, T):
    """Committed keys and values [T][D] of sequence b, KV head g, fp64."""
    PAGE = Kp.shape[2]
    t = np.arange(T)
    pages = (t // PAGE) if page_table is None else np.asarray(page_table)[b][t // PAGE]
    slot = t % PAGE
    K = f64(Kp[pages, g, slot, :])
    V = f64(Vp[pages, g, :, slot])
    return K, V


def dequant_q8(Kq, Ksc, Vq, Vsc):
    """The fp16 cache an 8-bit cache stands for: each code times its token's
    scale, the exact product rounded once to fp16 (the int8 code and the fp16
    scale multiply exactly in fp32, 8 + 11 significant bits).  Kq [P][Hkv][16][D],
    Vq [P][Hkv][D][16] int8; Ksc, Vsc [P][Hkv][16] fp16 (one per token).  Returns
    the (K, V) pages in ``tree_attn``'s fp16 layouts.  The pages keep the cache
    quantised to fit long contexts (lucebox-hub README, "Implemented here":
    the TQ3_0 and Q4_0 KV caches); the 8-bit layout and the rounding are a
    reading, stated here."""
    K = (np.asarray(Kq, np.float32) * np.asarray(Ksc, np.float32)[..., :, None]).astype(np.float16)
    V = (np.asarray(Vq, np.float32) * np.asarray(Vsc, np.float32)[..., None, :]).astype(np.float16)
    return K, V


def tree_attn(parent, q, Kp, Vp, T, Kt, Vt, page_table=None, tree_off=None, scale=None,
              rows=None):
    """o[i][h] = softmax(scale * keys q_ih) values, keys/values =
    cache[0:T_b] ++ draft K/V of i's root path.

    q [n][Hq][D]; Kt,Vt [n][Hkv][D]; T [B].  ``rows`` optionally restricts the
    computation to a list of (node, q_head) pairs (others left 0).
    Returns fp64 [n][Hq][D]."""
    parent = np.asarray(parent)
    Q, KT, VT = f64(q), f64(Kt), f64(Vt)
    n, Hq, D = Q.shape
    Hkv = KT.shape[1]
    grp = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if tree_off is None:
        tree_off = [0, n]
    T = np.atleast_1d(np.asarray(T))
    want = None if rows is None else set((int(a), int(b)) for a, b in rows)
    out = np.zeros((n, Hq, D))
    for b in range(len(tree_off) - 1):
        o, e = int(tree_off[b]), int(tree_off[b + 1])
        par = parent[o:e]
        for g in range(Hkv):
            sel = [(i, h) for i in range(o, e) for h in range(g * grp, (g + 1) * grp)
                   if want is None or (i, h) in want]
            if not sel:
                continue
            Kc, Vc = gather_cache(Kp, Vp, page_table, b, g, int(T[b]))
            Qm = np.stack([Q[i, h] for i, h in sel])          # [R][D]
            Sc = scale * (Qm @ Kc.T)                            # [R][T] cache scores
            for r, (i, h) in enumerate(sel):
                path = [o + j for j in root_path(par, i - o)]
                St = scale * (KT[path, g] @ Q[i, h])            # draft-path scores
                m = max(Sc[r].max(initial=-np.inf), St.max())
                pc = np.exp(Sc[r] - m)
                pt = np.exp(St - m)
                num = pc @ Vc + pt @ VT[path, g]
                out[i, h] = num / (pc.sum() + pt.sum())
    return out
