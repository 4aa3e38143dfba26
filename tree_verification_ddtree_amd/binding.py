"""ctypes binding of libddtree.so: argument marshalling only.

Every function keeps the name of the C entry point it wraps (include/ddtree.h)
and passes torch tensors as raw device pointers plus the current HIP stream.
Nothing here computes any part of the verify step; if the library is
missing, loading fails loudly.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libddtree.so")

DDT_F32, DDT_F16, DDT_BF16 = 0, 1, 2
DDT_COMMIT_REPLAY, DDT_COMMIT_SELECT, DDT_COMMIT_UPDATE = 0, 1, 2
DDT_ST_TREE, DDT_ST_LEVELS, DDT_ST_TOKEN, DDT_ST_ARGMAX, DDT_ST_CTX, DDT_ST_COMMIT = 1, 2, 4, 8, 16, 32
DDT_PAGE = 16
DDT_MAX_NODES = 64

_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class Plan(ctypes.Structure):
    _fields_ = [("B", _i32), ("n_total", _i32), ("n_max", _i32), ("W", _i32),
                ("tree_off", _vp), ("parent", _vp), ("depth", _vp), ("anc", _vp),
                ("win", _vp), ("status", _vp)]


class GdnLayer(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("beta", _vp),
                ("S_c", _vp), ("node_states", _vp), ("node_u", _vp), ("x", _vp), ("prefix", _vp)]


class AttnLayer(ctypes.Structure):
    _fields_ = [("Kt", _vp), ("Vt", _vp), ("Kc", _vp), ("Vc", _vp)]


class DDTError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {code} ({status_str(code)})")
        self.code = code


_SIGS = {
    "ddt_version": ([], _i32),
    "ddt_status_str": ([_i32], ctypes.c_char_p),
    "ddt_source_hash": ([], ctypes.c_char_p),
    "ddt_tree_plan_host": ([ctypes.POINTER(Plan), _i32], _i32),
    "ddt_tree_plan": ([ctypes.POINTER(Plan), _i32, _vp], _i32),
    "ddt_tree_conv": ([ctypes.POINTER(Plan), _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp], _i32),
    "ddt_tree_gdn": ([ctypes.POINTER(Plan), _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                      _f32, _i32, _vp, _vp, _vp, _vp], _i32),
    "ddt_tree_conv_gdn_lds": ([_i32, _i32], _sz),
    "ddt_tree_conv_gdn": ([ctypes.POINTER(Plan), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                           _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "ddt_accept_sample_workspace": ([ctypes.POINTER(Plan), _i32, _i32], _sz),
    "ddt_accept_sample": ([ctypes.POINTER(Plan), _vp, _i32, _i32, _vp, _vp, _f32, _i32, _f32, _vp, _vp, _vp,
                           _vp, _vp, _sz, _vp], _i32),
    "ddt_tree_attn_workspace": ([ctypes.POINTER(Plan), _i32, _i32, _i32, _i32, _i32], _sz),
    "ddt_tree_attn_q8": ([ctypes.POINTER(Plan), _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp,
                          _i32, _i32, _i32, _f32, _i32, _vp, _vp, _sz, _vp], _i32),
    "ddt_tree_attn": ([ctypes.POINTER(Plan), _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32,
                       _i32, _i32, _f32, _i32, _i32, _vp, _vp, _sz, _vp], _i32),
    "ddt_accept_walk_workspace": ([ctypes.POINTER(Plan), _i32], _sz),
    "ddt_accept_walk": ([ctypes.POINTER(Plan), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                         _vp], _i32),
    "ddt_accept_walk_noalloc": ([ctypes.POINTER(Plan), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "ddt_accept_walk_host": ([ctypes.POINTER(Plan), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
    "ddt_commit_state": ([ctypes.POINTER(Plan), _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp], _i32),
    "ddt_draft_topk_workspace": ([_i32, _i32, _i32, _i32], _sz),
    "ddt_draft_topk": ([_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "ddt_tree_build": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
}

_LIB = None


def lib():
    """The loaded libddtree.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python -m tree_verification_ddtree_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def status_str(code):
    return lib().ddt_status_str(int(code)).decode()


def _check(code, what):
    if code != 0:
        raise DDTError(code, what)


def _ptr(t):
    """Device (or host) address of a tensor / ndarray, None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t):
    import torch
    return {torch.float32: DDT_F32, torch.float16: DDT_F16, torch.bfloat16: DDT_BF16}[t.dtype]


def plan_struct(B, n_total, n_max, W, tree_off, parent, depth, anc, win, status):
    """Fill a Plan from tensors / arrays (device for ddt_tree_plan, host for
    ddt_tree_plan_host)."""
    return Plan(B, n_total, n_max, W, *[_ptr(x) for x in (tree_off, parent, depth, anc, win, status)])


class TreeBatch:
    """Device buffers of one step's plan: parent/tree_off inputs and every
    output array of ddt_tree_plan, sized per include/ddtree.h."""

    def __init__(self, parent, tree_off, W, device, n_max=None):
        import torch
        parent = np.asarray(parent, dtype=np.int32)
        tree_off = np.asarray(tree_off, dtype=np.int32)
        self.B = len(tree_off) - 1
        self.n_total = int(tree_off[-1])
        sizes = np.diff(tree_off)
        self.n_max = int(n_max if n_max is not None else max(1, int(sizes.max())))
        self.W = int(W)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.parent = torch.tensor(parent, **i32)
        self.tree_off = torch.tensor(tree_off, **i32)
        n = max(self.n_total, 1)
        self.depth = torch.zeros(n, **i32)
        self.anc = torch.zeros(n, dtype=torch.int64, device=dev)
        self.win = torch.zeros(n * max(self.W - 1, 1), **i32)
        self.status = torch.zeros(self.B, **i32)
        self.struct = plan_struct(self.B, self.n_total, self.n_max, self.W, self.tree_off,
                                  self.parent, self.depth, self.anc, self.win, self.status)
        # host copies of the tree for the host walk (its status words are its own)
        self.parent_host, self.tree_off_host = parent.copy(), tree_off.copy()
        self.status_host = np.zeros(self.B, np.int32)
        self.struct_host = plan_struct(self.B, self.n_total, self.n_max, self.W, self.tree_off_host,
                                       self.parent_host, None, None, None, self.status_host)


def _plan(p):
    return ctypes.byref(p.struct if isinstance(p, TreeBatch) else p)


# ------------------------------------------------------------------ entry points
def ddt_version():
    return lib().ddt_version()


def ddt_source_hash():
    return lib().ddt_source_hash().decode()


def ddt_tree_plan_host(plan_struct_host, max_levels):
    """Returns the status code (no raise): host-side validation is the point."""
    return lib().ddt_tree_plan_host(ctypes.byref(plan_struct_host), int(max_levels))


def ddt_tree_plan(plan, max_levels, stream=None):
    _check(lib().ddt_tree_plan(_plan(plan), int(max_levels), _stream(stream)), "ddt_tree_plan")


def ddt_tree_conv(plan, x, prefix, w, act, y, stream=None):
    _check(lib().ddt_tree_conv(_plan(plan), _ptr(x), _ptr(prefix), _ptr(w), int(x.shape[-1]),
                               int(act), dtype_code(x), _ptr(y), _stream(stream)), "ddt_tree_conv")


def ddt_tree_gdn(plan, q, k, v, alpha, beta, S_c, scale, out, node_states=None, node_u=None,
                 stream=None):
    Hk, dk = int(q.shape[1]), int(q.shape[2])
    Hv, dv = int(v.shape[1]), int(v.shape[2])
    _check(lib().ddt_tree_gdn(_plan(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                              _ptr(S_c), Hk, Hv, dk, dv, float(scale), dtype_code(q), _ptr(out),
                              _ptr(node_states), _ptr(node_u), _stream(stream)), "ddt_tree_gdn")


def ddt_tree_conv_gdn_lds(n_max, dk):
    return int(lib().ddt_tree_conv_gdn_lds(int(n_max), int(dk)))


def ddt_tree_conv_gdn(plan, x, prefix, w, alpha, beta, S_c, Hk, dk, scale, out, q_out=None, k_out=None,
                      v_out=None, node_states=None, node_u=None, stream=None):
    """Fused layer: x [n][2*Hk*dk + Hv*dv] (bf16 or fp32), gates fp32 [n][Hv],
    S_c [B][Hv][dv][dk]; out [n][Hv][dv]; optional q_out/k_out [n][Hk][dk],
    v_out [n][Hv][dv], node_states, node_u."""
    Hv, dv = int(out.shape[1]), int(out.shape[2])
    _check(lib().ddt_tree_conv_gdn(_plan(plan), _ptr(x), _ptr(prefix), _ptr(w), dtype_code(x), _ptr(alpha),
                                   _ptr(beta), _ptr(S_c), int(Hk), Hv, int(dk), dv, float(scale), _ptr(out),
                                   _ptr(q_out), _ptr(k_out), _ptr(v_out), _ptr(node_states), _ptr(node_u),
                                   _stream(stream)), "ddt_tree_conv_gdn")


def ddt_accept_sample_workspace(plan, V, top_k):
    return int(lib().ddt_accept_sample_workspace(_plan(plan), int(V), int(top_k)))


def ddt_accept_sample(plan, logits, draft_tok, uniforms, temperature, top_k, top_p, sample, path, L, bonus,
                      ws, stream=None):
    """Stochastic acceptance: logits [n][V] (bf16 or fp32), uniforms [n] fp32."""
    _check(lib().ddt_accept_sample(_plan(plan), _ptr(logits), dtype_code(logits), int(logits.shape[-1]),
                                   _ptr(draft_tok), _ptr(uniforms), float(temperature), int(top_k),
                                   float(top_p), _ptr(sample), _ptr(path), _ptr(L), _ptr(bonus), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "ddt_accept_sample")


def ddt_tree_attn_workspace(plan, Hq, Hkv, D, T_max, n_splits=0):
    return lib().ddt_tree_attn_workspace(_plan(plan), int(Hq), int(Hkv), int(D), int(T_max),
                                         int(n_splits))


def ddt_tree_attn(plan, q, Kc, Vc, page_table, T, T_max, Kt, Vt, out, ws, scale=None,
                  n_splits=0, stream=None):
    Hq, D = int(q.shape[1]), int(q.shape[2])
    Hkv = int(Kt.shape[1])
    max_pages = int(page_table.shape[1]) if page_table is not None else 0
    scale = float(scale if scale is not None else 1.0 / np.sqrt(D))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ddt_tree_attn(_plan(plan), _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(page_table),
                               max_pages, _ptr(T), int(T_max), _ptr(Kt), _ptr(Vt), Hq, Hkv, D,
                               scale, dtype_code(q), int(n_splits), _ptr(out), _ptr(ws), wsb,
                               _stream(stream)), "ddt_tree_attn")


def ddt_tree_attn_q8(plan, q, Kq, Ksc, Vq, Vsc, page_table, T, T_max, Kt, Vt, out, ws, scale=None,
                     n_splits=0, stream=None):
    """8-bit cache: Kq [P][Hkv][16][D], Vq [P][Hkv][D][16] int8; Ksc, Vsc [P][Hkv][16] fp16."""
    import torch
    if Kq.dtype != torch.int8 or Vq.dtype != torch.int8:
        raise TypeError("ddt_tree_attn_q8: Kq and Vq must be int8")
    if any(t.dtype != torch.float16 for t in (q, Ksc, Vsc, Kt, Vt)) or out.dtype != torch.float32:
        raise TypeError("ddt_tree_attn_q8: q, Ksc, Vsc, Kt, Vt must be float16 and out float32")
    Hq, D = int(q.shape[1]), int(q.shape[2])
    Hkv = int(Kt.shape[1])
    max_pages = int(page_table.shape[1]) if page_table is not None else 0
    scale = float(scale if scale is not None else 1.0 / np.sqrt(D))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ddt_tree_attn_q8(_plan(plan), _ptr(q), _ptr(Kq), _ptr(Ksc), _ptr(Vq), _ptr(Vsc),
                                  _ptr(page_table), max_pages, _ptr(T), int(T_max), _ptr(Kt), _ptr(Vt),
                                  Hq, Hkv, D, scale, int(n_splits), _ptr(out), _ptr(ws), wsb,
                                  _stream(stream)), "ddt_tree_attn_q8")


def ddt_accept_walk_workspace(plan, V):
    return lib().ddt_accept_walk_workspace(_plan(plan), int(V))


def ddt_accept_walk(plan, logits, draft_tok, argmax, path, L, bonus, ws, stream=None):
    V = int(logits.shape[-1])
    wsb = ws.numel() * ws.element_size()
    _check(lib().ddt_accept_walk(_plan(plan), _ptr(logits), dtype_code(logits), V,
                                 _ptr(draft_tok), _ptr(argmax), _ptr(path), _ptr(L), _ptr(bonus),
                                 _ptr(ws), wsb, _stream(stream)), "ddt_accept_walk")


def ddt_accept_walk_noalloc(plan, logits, draft_tok, argmax, path, L, bonus, stream=None):
    """ddt_accept_walk with the library's static scratch instead of a workspace."""
    _check(lib().ddt_accept_walk_noalloc(_plan(plan), _ptr(logits), dtype_code(logits), int(logits.shape[-1]),
                                         _ptr(draft_tok), _ptr(argmax), _ptr(path), _ptr(L), _ptr(bonus),
                                         _stream(stream)), "ddt_accept_walk_noalloc")


def ddt_accept_walk_host(plan_struct_host, logits, draft_tok, argmax, path, L, bonus):
    """The host walk on numpy arrays: logits float32, or uint16 holding bf16
    bits, [n_total][V]; outputs int32 arrays sized as for ddt_accept_walk."""
    arrs = [np.ascontiguousarray(a) for a in (logits, draft_tok)]
    for a in (argmax, path, L, bonus):
        if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
            raise TypeError("ddt_accept_walk_host: outputs must be C-contiguous int32 arrays")
    code = {np.dtype(np.float32): DDT_F32, np.dtype(np.uint16): DDT_BF16}.get(arrs[0].dtype)
    if code is None or arrs[1].dtype != np.int32:
        raise TypeError("ddt_accept_walk_host: logits float32 or uint16 (bf16 bits), draft_tok int32")
    _check(lib().ddt_accept_walk_host(ctypes.byref(plan_struct_host), _ptr(arrs[0]), code, int(arrs[0].shape[-1]),
                                      _ptr(arrs[1]), _ptr(argmax), _ptr(path), _ptr(L), _ptr(bonus)),
           "ddt_accept_walk_host")


def accept_walk_with_fallback(tb, logits, draft_tok, argmax, path, L, bonus, ws, stream=None):
    """The validate-then-fall-back walk: the device walk, then (after the
    stream is synchronised) its status words; if the device check of the
    argmax failed for any sequence (DDT_ST_ARGMAX), the step's logits and
    draft tokens are copied to the host, the host walk recomputes every
    output and the results are written back to the device arrays.  Returns
    (status [B] as left by the device walk, whether the host walk ran)."""
    import torch
    ddt_accept_walk(tb, logits, draft_tok, argmax, path, L, bonus, ws, stream)
    (stream or torch.cuda.current_stream()).synchronize()
    st = tb.status.cpu().numpy()
    if not (st & DDT_ST_ARGMAX).any():
        return st, False
    lg = logits.cpu()
    lg = lg.view(torch.int16).numpy().view(np.uint16) if lg.dtype == torch.bfloat16 else lg.numpy()
    out = [np.empty(tuple(t.shape), np.int32) for t in (argmax, path, L, bonus)]
    tb.status_host[:] = 0
    ddt_accept_walk_host(tb.struct_host, lg, draft_tok.cpu().numpy(), *out)
    for t, a in zip((argmax, path, L, bonus), out):
        t.copy_(torch.from_numpy(a))
    return st, True


def layer_table(structs, device):
    """Copy an array of GdnLayer / AttnLayer structs to device memory (uint8 tensor)."""
    import torch
    if not structs:
        return None
    arr = (type(structs[0]) * len(structs))(*structs)
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device)


def ddt_commit_state(plan, path, L, mode, gdn_table, n_gdn, Hk, Hv, dk, dv, gdn_dtype, C,
                     conv_dtype, attn_table, n_attn, Hkv, D, kv_dtype, page_table, T,
                     stream=None, cache_pages=None):
    """cache_pages: pages of a contiguous cache (page_table None), which
    bounds the appends; with a page table its width is the bound."""
    max_pages = int(page_table.shape[1]) if page_table is not None else int(cache_pages or 0)
    _check(lib().ddt_commit_state(_plan(plan), _ptr(path), _ptr(L), int(mode), _ptr(gdn_table),
                                  int(n_gdn), int(Hk), int(Hv), int(dk), int(dv), int(gdn_dtype),
                                  int(C), int(conv_dtype), _ptr(attn_table), int(n_attn),
                                  int(Hkv), int(D), int(kv_dtype), _ptr(page_table), max_pages,
                                  _ptr(T), _stream(stream)), "ddt_commit_state")


def ddt_draft_topk_workspace(B, L, V, K):
    return int(lib().ddt_draft_topk_workspace(int(B), int(L), int(V), int(K)))


def ddt_draft_topk(logits, K, topk_idx, topk_logit, lse, ws, stream=None):
    """logits [B][L][V] (bf16 or fp32 device tensor)."""
    B, L, V = (int(x) for x in logits.shape)
    wsb = ws.numel() * ws.element_size()
    _check(lib().ddt_draft_topk(_ptr(logits), B, L, V, dtype_code(logits), int(K), _ptr(topk_idx),
                                _ptr(topk_logit), _ptr(lse), _ptr(ws), wsb, _stream(stream)), "ddt_draft_topk")


def ddt_tree_build(topk_idx, topk_logit, lse, N, root_token, parent, tok, score, n_nodes, stream=None):
    """topk_* [B][L][K], lse [B][L]; outputs [B][N] and n_nodes [B]."""
    B, L, K = (int(x) for x in topk_idx.shape)
    _check(lib().ddt_tree_build(_ptr(topk_idx), _ptr(topk_logit), _ptr(lse), B, L, K, int(N),
                                _ptr(root_token), _ptr(parent), _ptr(tok), _ptr(score), _ptr(n_nodes),
                                _stream(stream)), "ddt_tree_build")
