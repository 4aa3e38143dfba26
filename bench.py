"""Benchmark of the DDTree tree-verify step on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  plan -> 16 x [3 x (tree conv + tree gated delta-net), tree attention]
       -> verify argmax + greedy walk -> commit of the accepted path (the
          delta-net states rebuilt from the u the tree kernel saved)
on the hybrid stack of 48 gated delta-net layers and 16 attention layers at
131,072 committed tokens and a 22-node draft tree (the pages' budget 22:
lucebox-hub README, "02 · DFlash DDtree", "Implemented here"; 128K context:
same section, first list).

    python bench.py [--steps K] [--warmup W] [--settle S] [--no-graph] [--no-cpu-baseline]

Prints ONE JSON line.  ``value`` is verify steps per second with every input
already resident in HBM; the step is captured once in a HIP graph and
replayed.  Before the timed steps, untimed replays keep the GPU busy for
``--settle`` seconds (its clock ramps over a few hundred ms of load).  ``roofline`` is for the dominant kernel (tree attention: context
split kernel + split combine, timed per call with HIP events on the launch
stream); ``cpu_baseline`` is the CPU oracle timed on a bounded sample of the
same step.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix peak
METRIC = "tree-verify steps/sec (budget 22) + achieved HBM GB/s vs peak, 1 GPU"


def _dev(a, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


SETTLE_BATCH = 10  # settle-phase steps between restores of the committed length


def headroom(warmup=5, steps=20, kernel_reps=5):
    """Steps the context must have room for: each step commits up to N tokens
    (warmup, timed steps, two eager passes of kernel_reps steps, graph capture,
    one batch of the settle phase)."""
    return warmup + steps + 2 * kernel_reps + 8 + SETTLE_BATCH


class Stack:
    """Device-resident inputs, outputs and descriptors of one verify step."""

    def __init__(self, device, seed=0, cfg=None, headroom_steps=256):
        import torch
        import tree_verification_ddtree_amd as ddt
        self.ddt = ddt
        c = dict(synth.STACK if cfg is None else cfg)
        self.c = c
        self.device = device
        N, T = c["N"], c["T"]
        self.parent = synth.random_tree(synth.rng_for(seed, 3, 18), N, c["levels"])
        self.tb = ddt.TreeBatch(self.parent, [0, N], c["W"], device)
        self.T0 = T
        # room for the accepted tokens of every step the benchmark runs
        self.T_max = T + headroom_steps * N
        npages = (self.T_max + N + 15) // 16
        self.npages = npages
        g = torch.Generator(device=device)
        n_gdn, n_attn = c["n_gdn"], c["n_attn"]
        self.gdn, self.conv, self.gdn_out, self.conv_out, self.gdn_u = [], [], [], [], []
        for l in range(n_gdn):
            gi = synth.gdn_inputs(seed, (3, l), N, c["Hk"], c["Hv"], c["dk"], c["dv"], "bf16")
            self.gdn.append({k: _dev(v, device) for k, v in gi.items()})
            ci = synth.conv_inputs(seed, (3, 1000 + l), N, c["C"], c["W"], "bf16")
            self.conv.append({k: _dev(v, device) for k, v in ci.items()})
            self.gdn_out.append(torch.empty(N, c["Hv"], c["dv"], dtype=torch.float32, device=device))
            self.gdn_u.append(torch.empty(N, c["Hv"], c["dv"], dtype=torch.float32, device=device))
            self.conv_out.append(torch.empty(N, c["C"], dtype=torch.float32, device=device))
        self.attn, self.kv, self.attn_out = [], [], []
        for l in range(n_attn):
            ai = synth.attn_inputs(seed, (3, 2000 + l), N, c["Hq"], c["Hkv"], c["D"], "f16")
            self.attn.append({k: _dev(v, device) for k, v in ai.items()})
            g.manual_seed(int(seed) * 1000003 + 3 * 10007 + l)
            K = torch.randn((npages, c["Hkv"], 16, c["D"]), generator=g, device=device,
                            dtype=torch.float16)
            V = torch.randn((npages, c["Hkv"], c["D"], 16), generator=g, device=device,
                            dtype=torch.float16)
            self.kv.append((K, V))
            self.attn_out.append(torch.empty(N, c["Hq"], c["D"], dtype=torch.float32, device=device))
        self.T = torch.tensor([T], dtype=torch.int32, device=device)
        self.attn_ws = torch.empty(
            ddt.ddt_tree_attn_workspace(self.tb, c["Hq"], c["Hkv"], c["D"], self.T_max),
            dtype=torch.uint8, device=device)
        V = synth.VOCAB
        lg, tok = synth.logits_and_draft(seed, (3, 3000), self.parent, V, "bf16", p_match=0.8)
        self.logits, self.tok = _dev(lg, device), _dev(tok, device)
        self.walk_ws = torch.empty(ddt.ddt_accept_walk_workspace(self.tb, V), dtype=torch.uint8,
                                   device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.amax = torch.empty(N, **i32)
        self.path = torch.empty(1, self.tb.n_max, **i32)
        self.L = torch.empty(1, **i32)
        self.bonus = torch.empty(1, **i32)
        gl = [ddt.GdnLayer(q=a["q"].data_ptr(), k=a["k"].data_ptr(), v=a["v"].data_ptr(),
                           alpha=a["alpha"].data_ptr(), beta=a["beta"].data_ptr(),
                           S_c=a["S_c"].data_ptr(), node_u=u.data_ptr(), x=x["x"].data_ptr(),
                           prefix=x["prefix"].data_ptr())
              for a, x, u in zip(self.gdn, self.conv, self.gdn_u)]
        al = [ddt.AttnLayer(a["Kt"].data_ptr(), a["Vt"].data_ptr(), K.data_ptr(), Vv.data_ptr())
              for a, (K, Vv) in zip(self.attn, self.kv)]
        self.gdn_table, self.attn_table = ddt.layer_table(gl, device), ddt.layer_table(al, device)
        self.timer = None  # {op: [(start, end) events]} while timing eager steps

    def _timed(self, name, fn):
        """Run one call; with the timer on, bracket it with HIP events on the
        current stream (every call of this benchmark uses it)."""
        if self.timer is None or name not in self.timer:
            return fn()
        import torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.timer[name].append((a, b))

    def setup_fused(self):
        """Buffers of the fused variant of the step, where each conv + delta-net
        pair is one ddt_tree_conv_gdn call on the conv's x (its channels are
        the layer's q | k | v): fp32 gates, the normalised keys handed to the
        commit, and the commit's layer table (fused layers commit as fp32)."""
        import torch
        ddt, c, N = self.ddt, self.c, self.c["N"]
        f32 = dict(dtype=torch.float32, device=self.device)
        self.fz, gl = [], []
        for g, x, u in zip(self.gdn, self.conv, self.gdn_u):
            f = dict(alpha=g["alpha"].float(), beta=g["beta"].float(),
                     q=torch.zeros(N, c["Hk"], c["dk"], **f32), k=torch.zeros(N, c["Hk"], c["dk"], **f32),
                     v=torch.zeros(N, c["Hv"], c["dv"], **f32))
            self.fz.append(f)
            gl.append(ddt.GdnLayer(q=f["q"].data_ptr(), k=f["k"].data_ptr(), v=f["v"].data_ptr(),
                                   alpha=f["alpha"].data_ptr(), beta=f["beta"].data_ptr(),
                                   S_c=g["S_c"].data_ptr(), node_u=u.data_ptr(), x=x["x"].data_ptr(),
                                   prefix=x["prefix"].data_ptr()))
        self.fused_table = ddt.layer_table(gl, self.device)

    def fused_call(self, l, stream=None):
        c, g, x, f = self.c, self.gdn[l], self.conv[l], self.fz[l]
        self.ddt.ddt_tree_conv_gdn(self.tb, x["x"], x["prefix"], x["w"], f["alpha"], f["beta"], g["S_c"],
                                   c["Hk"], c["dk"], 1.0, self.gdn_out[l], k_out=f["k"],
                                   node_u=self.gdn_u[l], stream=stream)

    def step(self, stream=None, fused=False):
        ddt, c = self.ddt, self.c
        self._timed("plan", lambda: ddt.ddt_tree_plan(self.tb, c["levels"], stream))
        gi = 0
        for a in range(c["n_attn"]):
            for _ in range(c["n_gdn"] // c["n_attn"]):
                x, g, l = self.conv[gi], self.gdn[gi], gi
                if fused:
                    self._timed("fused", lambda: self.fused_call(l, stream))
                    gi += 1
                    continue
                self._timed("conv", lambda: ddt.ddt_tree_conv(self.tb, x["x"], x["prefix"], x["w"], 0,
                                                             self.conv_out[l], stream))
                self._timed("gdn", lambda: ddt.ddt_tree_gdn(
                    self.tb, g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S_c"], 1.0,
                    self.gdn_out[l], None, self.gdn_u[l], stream))
                gi += 1
            at, (K, V) = self.attn[a], self.kv[a]
            self._timed("attn", lambda: ddt.ddt_tree_attn(
                self.tb, at["q"], K, V, None, self.T, self.T_max, at["Kt"], at["Vt"], self.attn_out[a],
                self.attn_ws, stream=stream))
        self._timed("walk", lambda: ddt.ddt_accept_walk(self.tb, self.logits, self.tok, self.amax,
                                                        self.path, self.L, self.bonus, self.walk_ws,
                                                        stream))
        self._timed("commit", lambda: ddt.ddt_commit_state(
            self.tb, self.path, self.L, ddt.DDT_COMMIT_UPDATE, self.fused_table if fused else self.gdn_table,
            c["n_gdn"], c["Hk"], c["Hv"], c["dk"], c["dv"], ddt.DDT_F32 if fused else ddt.DDT_BF16, c["C"],
            ddt.DDT_BF16, self.attn_table, c["n_attn"], c["Hkv"], c["D"], ddt.DDT_F16, None, self.T, stream,
            cache_pages=self.npages))

    def op_batches(self):
        """Idempotent calls of the short ops for batch timing: every layer's
        conv, every layer's delta-net, and the plan and walk (20 each)."""
        ddt, c = self.ddt, self.c
        conv = [lambda x=x, y=y: ddt.ddt_tree_conv(self.tb, x["x"], x["prefix"], x["w"], 0, y)
                for x, y in zip(self.conv, self.conv_out)]
        gdn = [lambda g=g, o=o, u=u: ddt.ddt_tree_gdn(self.tb, g["q"], g["k"], g["v"], g["alpha"],
                                                      g["beta"], g["S_c"], 1.0, o, None, u)
               for g, o, u in zip(self.gdn, self.gdn_out, self.gdn_u)]
        plan = [lambda: ddt.ddt_tree_plan(self.tb, c["levels"])] * 20
        walk = [lambda: ddt.ddt_accept_walk(self.tb, self.logits, self.tok, self.amax, self.path,
                                            self.L, self.bonus, self.walk_ws)] * 20
        return {"plan": plan, "conv": conv, "gdn": gdn, "walk": walk}

    # ---------------------------------------------------------------- bytes
    def attn_bytes(self, T):
        c = self.c
        N = c["N"]
        kv = T * c["Hkv"] * c["D"] * 2 * 2
        return kv + N * c["Hq"] * c["D"] * 2 + N * c["Hkv"] * c["D"] * 2 * 2 + N * c["Hq"] * c["D"] * 4

    def op_bytes(self, T, L):
        """Algorithmic HBM bytes of one call of each op: every input read
        once, every output written once (the commit: the new state, prefix
        and K/V it writes; the delta-net call: the committed state it reads)."""
        c = self.c
        N, W1 = c["N"], c["W"] - 1
        state = c["Hv"] * c["dv"] * c["dk"] * 4
        return {
            "plan": N * 4 + N * (4 + 8 + 4 * max(W1, 1) + 4 + 4),
            "conv": N * c["C"] * 2 + W1 * c["C"] * 2 + c["C"] * c["W"] * 2 + N * c["C"] * 4,
            "gdn": (state + N * c["Hk"] * c["dk"] * 2 * 2 + N * c["Hv"] * c["dv"] * 2
                    + N * c["Hv"] * 2 * 2 + N * c["Hv"] * c["dv"] * 4),
            "attn": self.attn_bytes(T),
            "walk": N * synth.VOCAB * 2 + N * 4 + N * 4 + N * 4 + 8,
            "commit": (c["n_gdn"] * (state + W1 * c["C"] * 2)
                       + L * c["Hkv"] * c["D"] * 2 * 2 * c["n_attn"]),
        }

    def step_bytes(self, T, L):
        """Algorithmic HBM bytes of one step (the sum over its calls)."""
        c = self.c
        b = self.op_bytes(T, L)
        per = {"plan": 1, "conv": c["n_gdn"], "gdn": c["n_gdn"], "attn": c["n_attn"], "walk": 1, "commit": 1}
        return sum(per[k] * v for k, v in b.items())


def draft_bench(device, B, reps=5, calls=20, settle=0.3, cpu_s=0.0):
    """Ahead of the verify step: draft top-K / log-sum-exp and the DDTree
    build on L=16 draft positions of the full vocabulary (bf16 logits), K=8,
    budget 22.  Timed as graph-replayed back-to-back batches (each call is a
    few microseconds), the two entry points on their own and together, each
    after `settle` seconds of untimed replays (the clock ramps under load)."""
    import torch
    import tree_verification_ddtree_amd as ddt
    c = synth.DRAFT
    L, K, N, V = c["L"], c["K"], c["N"], synth.VOCAB
    lg = _dev(np.stack([synth.draft_logits(0, (40, b), L, V, "bf16") for b in range(B)]), device)
    i32 = dict(dtype=torch.int32, device=device)
    idx, lse = torch.empty(B, L, K, **i32), torch.empty(B, L, dtype=torch.float32, device=device)
    val = torch.empty(B, L, K, dtype=torch.float32, device=device)
    ws = torch.empty(ddt.ddt_draft_topk_workspace(B, L, V, K), dtype=torch.uint8, device=device)
    roots = torch.arange(B, **i32)
    parent, tok, n = torch.empty(B, N, **i32), torch.empty(B, N, **i32), torch.empty(B, **i32)
    score = torch.empty(B, N, dtype=torch.float32, device=device)
    topk = lambda: ddt.ddt_draft_topk(lg, K, idx, val, lse, ws)  # noqa: E731
    tree = lambda: ddt.ddt_tree_build(idx, val, lse, N, roots, parent, tok, score, n)  # noqa: E731
    res = {}
    for name, fns in (("topk", [topk]), ("tree", [tree]), ("both", [topk, tree])):
        for f in fns:
            f()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                for f in fns:
                    f()
        g.replay()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle
        while time.perf_counter() < t_end:
            for _ in range(10):
                g.replay()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / (reps * calls)
        del g
    nbytes = B * L * V * 2 + B * L * (K * 8 + 4)
    gbps = nbytes / (res["topk"] * 1e-6) / 1e9
    out = {"workload": f"draft_tree_b{B}_l{L}_k{K}_n{N}", "B": B, "L": L, "V": V, "K": K, "N": N,
           "us_topk": res["topk"], "us_tree": res["tree"], "us_per_call": res["both"],
           "trees_per_s": B / (res["both"] * 1e-6),
           "topk_bytes": nbytes, "topk_GBps": gbps, "topk_frac_hbm_peak": gbps / HBM_PEAK_GBPS,
           "timed": "graph-replayed back-to-back batch", "bound": "hbm (top-K); latency (tree)",
           "cpu_baseline": None}
    if cpu_s > 0:
        # the oracle on sequence 0 of the same logits, repeated for about cpu_s seconds
        import oracle
        x = lg[0].float().cpu().numpy()
        n, t0 = 0, time.perf_counter()
        while True:
            ti, tv, tl = oracle.draft_topk(x, K)
            oracle.build_tree(ti, oracle.log_probs(tv, tl), N, 0)
            n += 1
            if time.perf_counter() - t0 >= cpu_s:
                break
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / el, "unit": "trees/s", "cores": 1, "kind": "oracle",
                               "sample": f"numpy fp64 oracle, {n} tree(s) from one sequence's "
                                         f"[{L}][{V}] bf16 logits"}
    return out


def fused_stack_bench(st, T_set, steps, settle, reps=5):
    """The same 128K step with each conv + delta-net pair replaced by one
    fused ddt_tree_conv_gdn call (48 launches fewer), timed like the step:
    eager warmup, one captured graph, settle replays with the committed
    length put back, then `steps` timed replays from the configured
    context.  The fused call alone is timed as a graph-replayed batch of
    the 48 layers."""
    import torch
    st.setup_fused()
    st.T.copy_(T_set)
    for _ in range(2):
        st.step(fused=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step(fused=True)
    t_end = time.perf_counter() + settle
    while time.perf_counter() < t_end:
        st.T.copy_(T_set)
        for _ in range(SETTLE_BATCH):
            g.replay()
        torch.cuda.synchronize()
    st.T.copy_(T_set)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    status = st.tb.status.cpu().numpy()
    if status.any():
        raise RuntimeError(f"device status {status}")
    del g
    calls = [lambda l=l: st.fused_call(l) for l in range(st.c["n_gdn"])]
    for fn in calls:
        fn()
    gb = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gb):
        for fn in calls:
            fn()
    gb.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gb.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * len(calls))
    del gb
    st.T.copy_(T_set)
    return {"workload": st.c["name"] + "_fused_conv_gdn", "ms_per_step": ms, "steps_per_s": 1000.0 / ms,
            "fused_us_per_layer": us, "layers": st.c["n_gdn"],
            "timed": "graph-replayed step after a settle phase; the fused call as a graph-replayed batch"}


def q8_attn_bench(st, reps=5, settle=0.4, pools=4):
    """One attention layer of the step over an 8-bit cache of the same shape
    (codes and per-token scales drawn on the device), against the same call
    over the step's fp16 caches, both as graphs of back-to-back calls that
    cycle through `pools` caches (more bytes than the last-level cache holds),
    replayed after a settle phase."""
    import torch
    ddt, c, dev = st.ddt, st.c, st.device
    Hkv, D = c["Hkv"], c["D"]
    npages = st.kv[0][0].shape[0]
    g = torch.Generator(device=dev)
    g.manual_seed(8)
    q8 = []
    for _ in range(pools):
        Kq = torch.randint(-127, 128, (npages, Hkv, synth.PAGE, D), generator=g, device=dev, dtype=torch.int8)
        Vq = torch.randint(-127, 128, (npages, Hkv, D, synth.PAGE), generator=g, device=dev, dtype=torch.int8)
        Ks = (torch.rand((npages, Hkv, synth.PAGE), generator=g, device=dev) * 0.01 + 0.005).half()
        Vs = (torch.rand((npages, Hkv, synth.PAGE), generator=g, device=dev) * 0.01 + 0.005).half()
        q8.append((Kq, Ks, Vq, Vs))
    at, out = st.attn[0], st.attn_out[0]

    def timed(call):
        call(0)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(4 * pools):
                call(i)
        gr.replay()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle
        while time.perf_counter() < t_end:
            gr.replay()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * 4 * pools)

    def call_q8(i):
        Kq, Ks, Vq, Vs = q8[i % pools]
        ddt.ddt_tree_attn_q8(st.tb, at["q"], Kq, Ks, Vq, Vs, None, st.T, st.T_max, at["Kt"], at["Vt"], out,
                             st.attn_ws)

    def call_f16(i):
        K, V = st.kv[i % min(pools, len(st.kv))]
        ddt.ddt_tree_attn(st.tb, at["q"], K, V, None, st.T, st.T_max, at["Kt"], at["Vt"], out, st.attn_ws)
    us_q8, us_f16 = timed(call_q8), timed(call_f16)
    T = int(st.T.item())
    nbytes = st.attn_bytes(T) - T * Hkv * D * 2 * 2 + T * Hkv * (D * 2 + 2 * 2)
    del q8
    return {"workload": "tree_attn_t128k_n22_q8 (one layer, 8-bit K/V codes, one fp16 scale per token)",
            "us_per_call": us_q8, "fp16_us_per_call": us_f16, "speedup_vs_fp16": us_f16 / us_q8,
            "bytes_per_call": nbytes, "GBps": nbytes / (us_q8 * 1e-6) / 1e9,
            "frac_hbm_peak": nbytes / (us_q8 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "timed": "graph of back-to-back calls over 4 caches, after a settle phase"}


def sample_bench(st, reps=5, calls=20, settle=0.3, cpu_s=0.0):
    """Stochastic acceptance on the step's own verify logits and tree (22 x
    151,936 bf16), the model card's sampling (temperature 1.0, top_k 20,
    top_p 0.95), timed like the short ops: a graph of back-to-back calls,
    replayed after a settle phase.  Reported beside the greedy walk."""
    import torch
    ddt, c, dev = st.ddt, st.c, st.device
    N, V = c["N"], synth.VOCAB
    T, k, p = 1.0, 20, 0.95
    i32 = dict(dtype=torch.int32, device=dev)
    u = _dev(synth.uniforms(0, (3, 4000), N), dev)
    sample, path = torch.empty(N, **i32), torch.empty(1, st.tb.n_max, **i32)
    L, bonus = torch.empty(1, **i32), torch.empty(1, **i32)
    ws = torch.empty(ddt.ddt_accept_sample_workspace(st.tb, V, k), dtype=torch.uint8, device=dev)
    call = lambda: ddt.ddt_accept_sample(st.tb, st.logits, st.tok, u, T, k, p, sample, path, L, bonus, ws)  # noqa: E731
    call()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            call()
    g.replay()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle
    while time.perf_counter() < t_end:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * calls)
    del g
    nbytes = N * V * 2
    out = {"workload": "stack_t128k_n22 verify logits, temperature 1.0 top_k 20 top_p 0.95",
           "us_per_call": us, "logits_bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
           "frac_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
           "mean_accepted_L": float(L.float().mean().item()),
           "timed": "graph-replayed back-to-back batch", "cpu_baseline": None}
    if cpu_s > 0:
        import oracle
        lg = st.logits.float().cpu().numpy()
        tok, uu = st.tok.cpu().numpy().astype(np.int64), u.cpu().numpy()
        n, t0 = 0, time.perf_counter()
        while True:
            y, _ = oracle.sample_tokens(lg, uu, T, k, p)
            oracle.accept_walk(st.parent, tok, y)
            n += 1
            if time.perf_counter() - t0 >= cpu_s:
                break
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
                               "sample": f"numpy fp64 oracle, {n} full sampled acceptance(s) of the step"}
    return out


def _traffic(kernel_src_sha):
    """HBM traffic of the attention call from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "tree_attn_t128k_n22_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_src_sha:
        return None
    return d.get("bytes_per_call")


def cpu_baseline(st, seed, gdn_s=6.0, attn_s=8.0):
    """The CPU oracle on a bounded sample of the same step, scaled to a
    whole step.  Gated delta-net + conv layers are run one after another
    until ``gdn_s`` seconds have passed, attention one (layer, KV head) at a
    time until ``attn_s`` seconds have passed, then the full verify walk
    once; per-layer and per-head means are scaled to the 48 + 16 x 4 of one
    step.  Inputs are copied from the device before the clock starts."""
    import torch
    import oracle
    c = st.c
    N = c["N"]
    nthreads = len(os.sched_getaffinity(0))
    torch.set_num_threads(nthreads)
    par = st.parent
    host = lambda t: t.detach().cpu()
    u16 = lambda t: host(t).view(torch.int16).numpy().view(np.uint16)
    T = st.T0
    npg = (T + 15) // 16
    G = c["Hq"] // c["Hkv"]

    def gdn_in(l):
        g = {k: (u16(v) if v.dtype == torch.bfloat16 else host(v).numpy()) for k, v in st.gdn[l].items()}
        x = {k: u16(v) for k, v in st.conv[l].items()}
        return g, x

    def attn_in(l, h):
        K, V = st.kv[l]
        a = {k: host(v).numpy() for k, v in st.attn[l].items()}
        return (a["q"][:, h * G:(h + 1) * G], host(K[:npg, h:h + 1]).numpy(),
                host(V[:npg, h:h + 1]).numpy(), a["Kt"][:, h:h + 1], a["Vt"][:, h:h + 1])

    t_gdn, n_gdn = 0.0, 0
    while n_gdn < c["n_gdn"] and t_gdn < gdn_s:
        g0, x0 = gdn_in(n_gdn)
        t0 = time.perf_counter()
        oracle.tree_conv(par, x0["x"], x0["prefix"], x0["w"])
        oracle.tree_gdn(par, g0["q"], g0["k"], g0["v"], g0["alpha"], g0["beta"], g0["S_c"])
        t_gdn += time.perf_counter() - t0
        n_gdn += 1
    t_attn, n_heads = 0.0, 0
    while n_heads < c["n_attn"] * c["Hkv"] and t_attn < attn_s:
        q1, Kh, Vh, kt1, vt1 = attn_in(n_heads // c["Hkv"], n_heads % c["Hkv"])
        t0 = time.perf_counter()
        oracle.tree_attn(par, q1, Kh, Vh, [T], kt1, vt1)
        t_attn += time.perf_counter() - t0
        n_heads += 1
    lg, tok = u16(st.logits), host(st.tok).numpy()
    t0 = time.perf_counter()
    am = oracle.argmax_rows(lg)
    oracle.accept_walk(par, tok, am)
    t_walk = time.perf_counter() - t0
    step_s = (c["n_gdn"] * t_gdn / n_gdn + c["n_attn"] * c["Hkv"] * t_attn / n_heads + t_walk)
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": nthreads, "kind": "oracle",
            "sample": (f"numpy fp64 oracle: {n_gdn} of {c['n_gdn']} gated delta-net+conv layers, "
                       f"{n_heads} of {c['n_attn'] * c['Hkv']} (attention layer, KV head) pairs "
                       f"({G} q-heads x {N} nodes each) at T={T}, full argmax+walk over "
                       f"{N}x{synth.VOCAB}; means scaled to one step; sample took "
                       f"{t_gdn + t_attn + t_walk:.1f} s of CPU time"),
            "seconds_per_step": step_s}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the measurements of the widenings beside the step (draft tree build)")
    ap.add_argument("--kernel-reps", type=int, default=5, help="eager steps timed per attention call")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed sustained steps before timing (the GPU clock ramps "
                         "over a few hundred ms of load)")
    ap.add_argument("--draft", type=int, default=0, metavar="B",
                    help="only time the draft top-K and tree build for B sequences and print that line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference kernel "
                         "that scales the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the verify step of one batch runs on a single MI355X; "
              "runs over several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    import tree_verification_ddtree_amd as ddt
    ddt.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 3}), flush=True)
        return
    if args.draft > 0:
        print(json.dumps(draft_bench(dev, args.draft, settle=args.settle,
                                     cpu_s=0.0 if args.no_cpu_baseline else 3.0)), flush=True)
        return
    print(f"[bench] building the 128K stack (seed {args.seed})", file=sys.stderr, flush=True)
    st = Stack(dev, seed=args.seed, headroom_steps=headroom(args.warmup, args.steps, args.kernel_reps))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    status = st.tb.status.cpu().numpy()
    if status.any():
        raise RuntimeError(f"device status {status}")
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                st.step()
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001 - report and time eagerly instead
            print(f"[bench] graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph, use_graph = None, False
    # The GPU clock ramps up over a few hundred ms of sustained load and falls
    # back while the host builds the inputs, so untimed steps keep the GPU
    # busy for --settle seconds first.  The committed length is put back
    # after every batch, so the timed steps run at the configured context.
    T_set = st.T.clone()
    t_set = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_set < args.settle:
        for _ in range(SETTLE_BATCH):
            if graph is not None:
                graph.replay()
            else:
                st.step()
        st.T.copy_(T_set)
        torch.cuda.synchronize()
        n_settle += SETTLE_BATCH
    status = st.tb.status.cpu().numpy()
    if status.any():
        raise RuntimeError(f"device status {status}")
    T_start = int(st.T.item())
    print(f"[bench] settled for {n_settle} steps; timing {args.steps} steps (graph={use_graph})",
          file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            st.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    T_end = int(st.T.item())
    L_mean = (T_end - T_start) / args.steps
    status = st.tb.status.cpu().numpy()
    if status.any():
        raise RuntimeError(f"device status {status}")

    # Per-op call times, with HIP events on the launch stream.  Attention (the
    # dominant kernel) and the commit are timed call by call inside eager
    # steps, one op per pass; the short ops (plan, conv, delta-net, walk) are
    # timed as graph-replayed back-to-back batches under one event pair,
    # because an event pair around a single few-microsecond call adds a gap
    # of its own.
    timer = {}
    for op in ("attn", "commit"):
        st.timer = {op: []}
        for _ in range(args.kernel_reps):
            st.step()
            torch.cuda.synchronize()
        timer[op] = [a.elapsed_time(b) for a, b in st.timer[op]]
    st.timer = None
    for op, calls in st.op_batches().items():
        # the batch is captured in a HIP graph so that host launch cost does
        # not enter the measurement (as for the timed step itself)
        for fn in calls:  # one untimed eager round first
            fn()
        gb = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gb):
            for fn in calls:
                fn()
        gb.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.kernel_reps):
            gb.replay()
        b.record()
        torch.cuda.synchronize()
        timer[op] = [a.elapsed_time(b) / (args.kernel_reps * len(calls))]
        del gb
    T_mid = (T_start + T_end) / 2
    L_step = max(L_mean, 1.0)
    ob = st.op_bytes(T_mid, L_step)
    per_step = {"plan": 1, "conv": st.c["n_gdn"], "gdn": st.c["n_gdn"], "attn": st.c["n_attn"],
                "walk": 1, "commit": 1}
    kernels = {}
    for op in ("plan", "conv", "gdn", "attn", "walk", "commit"):
        us = float(np.mean(timer[op])) * 1e3
        gbps = ob[op] / (us * 1e-6) / 1e9
        kernels[op] = {"us_per_call": us, "calls_per_step": per_step[op], "bytes_per_call": ob[op],
                       "GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                       "timed": "per call in eager steps" if op in ("attn", "commit")
                       else "graph-replayed back-to-back batch"}
    attn_ms = kernels["attn"]["us_per_call"] * 1e-3
    attn_bytes = ob["attn"]
    # the attention tiles' matrix work: Q K^T and P V over the cache, 2 flops
    # per multiply-add, every real query row (q-heads x nodes), fp16 dense peak
    attn_flops = 2.0 * 2.0 * st.c["Hq"] * st.c["N"] * T_mid * st.c["D"]
    kernels["attn"]["mfma"] = {
        "flops_per_call": attn_flops, "TFLOPs": attn_flops / (attn_ms * 1e-3) / 1e12,
        "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": attn_flops / (attn_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    src = open(os.path.join(ROOT, "tree_verification_ddtree_amd", "csrc", "attn.hip"), "rb").read()
    traffic = _traffic(hashlib.sha256(src).hexdigest())
    step_bytes = st.step_bytes(T_mid, L_mean)
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": synth.STACK["name"],
            "budget": st.c["N"], "context": st.T0, "gdn_layers": st.c["n_gdn"],
            "attn_layers": st.c["n_attn"], "kv_heads": st.c["Hkv"], "q_heads": st.c["Hq"],
            "head_dim": st.c["D"], "gdn_heads": [st.c["Hk"], st.c["Hv"]], "state": [st.c["dv"], st.c["dk"]],
            "conv_channels": st.c["C"], "vocab": synth.VOCAB, "graph": use_graph,
            "inputs": "fp16 KV cache and attention, bf16 delta-net/conv/logits, fp32 state and accumulation",
            "mean_accepted_L": L_mean,
        },
        "achieved_GBps_step": step_bytes / (ms * 1e-3) / 1e9,
        "roofline_frac_step": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "wall_s_timed": wall,
        "roofline": {
            "kernel": "ddt_tree_attn (attn_mfma_kernel + attn_combine_kernel)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "bytes_per_call": attn_bytes, "ms_per_call": attn_ms,
        },
        "kernels": kernels,
        "cpu_baseline": None,
        "library_source_sha256": ddt.ddt_source_hash(),
    }
    if not args.no_next:
        # widening ahead of the step (reported beside it, not part of `value`)
        print("[bench] draft top-K + tree build", file=sys.stderr, flush=True)
        cs = 0.0 if args.no_cpu_baseline else 3.0
        print("[bench] fused conv -> delta-net step", file=sys.stderr, flush=True)
        fz = fused_stack_bench(st, T_set, args.steps, args.settle)
        fz["vs_unfused_step"] = ms / fz["ms_per_step"]
        fz["unfused_conv_plus_gdn_us"] = kernels["conv"]["us_per_call"] + kernels["gdn"]["us_per_call"]
        out["next"] = {"fused_stack": fz}
        print("[bench] 8-bit KV attention", file=sys.stderr, flush=True)
        out["next"]["q8_attention"] = q8_attn_bench(st)
        print("[bench] sampled acceptance", file=sys.stderr, flush=True)
        sb = sample_bench(st, cpu_s=cs)
        sb["greedy_walk_us"] = kernels["walk"]["us_per_call"]
        out["next"]["sampled_walk"] = sb
        print("[bench] draft top-K + tree build", file=sys.stderr, flush=True)
        out["next"]["draft_tree"] = [draft_bench(dev, 1, cpu_s=cs), draft_bench(dev, 8)]
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(st, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
