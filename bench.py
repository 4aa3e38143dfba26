"""Benchmark of the DDTree tree-verify step on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  plan -> the stack's layers in order [tree conv + tree gated delta-net (G),
  tree attention (A)] -> verify argmax + greedy walk -> commit of the
  accepted path (the delta-net states rebuilt from the u the tree kernel
  saved)

The headline is the hybrid stack (G, G, G, A) x 16 -- 48 gated delta-net
layers and 16 attention layers -- at 131,072 committed tokens and a 22-node
draft tree (the pages' budget 22: lucebox-hub README, "02 · DFlash DDtree",
"Implemented here"; 128K context: same section, first list).  Beside it the
same measurement runs on the other four workloads: a tiny step, one
delta-net + conv layer, one attention layer at 32K, and eight concurrent
sequences over a paged cache (Luce-Org/lucebox README, "Inference Engine
Optimizations").

    python bench.py [--steps K] [--warmup W] [--settle S] [--no-graph]
                    [--no-cpu-baseline] [--no-next] [--configs all|none|a,b]

Prints ONE JSON line.  ``value`` is verify steps per second of the stack
with every input already resident in HBM: the step is captured once in a HIP
graph, W steps are replayed untimed, then K steps are timed under one event
pair (whole-job throughput).  A second pass times K more steps one by one
for the median, p10 and p90.  Before timing, untimed replays keep the GPU
busy for ``--settle`` seconds (its clock ramps over a few hundred ms of
load).  ``roofline`` is for the dominant kernel (tree attention: context
split kernel + split combine, timed per call with HIP events on the launch
stream); ``roofline_step`` is the whole step against the same peak;
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the step.
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
SETTLE_BATCH = 10  # settle-phase steps between restores of the committed length
MIN_EACH_STEPS = 100  # one-by-one timed steps of a workload line, at least
ELEM = {"f32": 4, "f16": 2, "bf16": 2}
CONFIGS = ("tiny", "layer_gdn", "layer_attn", "batched")


def _dev(a, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def headroom(warmup=5, steps=100, kernel_reps=5):
    """Steps of context growth a workload must have room for: the committed
    length is put back to its configured value before every timed phase, and
    the longest phase is the larger of the timed steps (at least the 100 a
    workload line times one by one), the warmup, the per-call passes and a
    settle batch (plus a few for the graph capture)."""
    return max(warmup, steps, MIN_EACH_STEPS, kernel_reps, SETTLE_BATCH) + 8


class Workload:
    """Device-resident inputs, outputs and descriptors of one verify step.

    ``pattern`` lists the stack's layers in order ('G': tree conv + tree
    gated delta-net, 'A': tree attention); ``trees`` and ``T`` give each
    sequence's draft tree and committed length.  With ``copies`` > 1 every
    layer input and the logits exist that many times and step(c) uses copy
    c, so that a graph cycling through them moves more bytes than the
    last-level cache holds.  Layer inputs are drawn on the host by ``synth``
    (copy 0) and copied on the device for the other copies; fp16 attention
    caches are N(0,1) drawn on the device (the same distribution; it saves
    set-up time)."""

    def __init__(self, device, cfg, trees, T, pattern, paged=False, copies=1, seed=0, key=3,
                 room_steps=64):
        import torch
        import tree_verification_ddtree_amd as ddt
        self.ddt, self.device, self.c = ddt, device, dict(cfg)
        c = self.c
        self.name = c["name"]
        self.pattern = list(pattern)
        self.trees = [np.asarray(t, dtype=np.int32) for t in trees]
        par, off = synth.concat_trees(self.trees)
        self.parent = self.trees[0] if len(self.trees) == 1 else par
        self.off, self.B, self.n = off, len(self.trees), len(par)
        self.sizes = [len(t) for t in self.trees]
        self.tb = ddt.TreeBatch(par, off, c["W"], device)
        self.T0 = np.asarray(T, dtype=np.int64)
        self.gdt = c.get("dtype_gdn", "bf16")
        self.adt = c.get("dtype_attn", "f16")
        self.ldt = c.get("dtype_logits", "bf16")
        self.ncopies = copies
        n, B = self.n, self.B
        self.n_gdn, self.n_attn = self.pattern.count("G"), self.pattern.count("A")
        room = room_steps * max(self.sizes)  # tokens the commits may add before T is put back
        self.T_max = int(self.T0.max()) + room
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.pt, self.max_pages, npages = None, 0, 0
        if self.n_attn:
            if paged:
                pt, npages = synth.page_layout(seed, (key, 7), self.T0, [room] * B)
                self.pt, self.max_pages = _dev(pt, device), int(pt.shape[1])
            else:
                assert B == 1, "a contiguous cache holds one sequence"
                npages = (self.T_max + 15) // 16
                self.max_pages = npages
        self.npages = npages
        g = torch.Generator(device=device)
        V = synth.VOCAB
        self.copy = []
        for ci in range(copies):
            cp = dict(gdn=[], conv=[], gdn_out=[], gdn_u=[], conv_out=[], attn=[], kv=[], attn_out=[])
            base = self.copy[0] if ci else None
            for l in range(self.n_gdn):
                if base is None:
                    gi = synth.gdn_inputs(seed, (key, l), n, c["Hk"], c["Hv"], c["dk"], c["dv"], self.gdt, B=B)
                    xi = synth.conv_inputs(seed, (key, 1000 + l), n, c["C"], c["W"], self.gdt, B=B)
                    cp["gdn"].append({k: _dev(v, device) for k, v in gi.items()})
                    cp["conv"].append({k: _dev(v, device) for k, v in xi.items()})
                else:
                    cp["gdn"].append({k: v.clone() for k, v in base["gdn"][l].items()})
                    cp["conv"].append({k: v.clone() for k, v in base["conv"][l].items()})
                cp["gdn_out"].append(torch.empty(n, c["Hv"], c["dv"], **f32))
                cp["gdn_u"].append(torch.empty(n, c["Hv"], c["dv"], **f32))
                cp["conv_out"].append(torch.empty(n, c["C"], **f32))
            for l in range(self.n_attn):
                if base is None:
                    ai = synth.attn_inputs(seed, (key, 2000 + l), n, c["Hq"], c["Hkv"], c["D"], self.adt)
                    cp["attn"].append({k: _dev(v, device) for k, v in ai.items()})
                else:
                    cp["attn"].append({k: v.clone() for k, v in base["attn"][l].items()})
                if self.adt == "f16":
                    g.manual_seed(int(seed) * 1000003 + key * 10007 + l + 7919 * ci)
                    K = torch.randn((npages, c["Hkv"], 16, c["D"]), generator=g, device=device,
                                    dtype=torch.float16)
                    Vv = torch.randn((npages, c["Hkv"], c["D"], 16), generator=g, device=device,
                                     dtype=torch.float16)
                else:
                    Kh, Vh = synth.kv_pool(seed, (key, 4000 + l), npages, c["Hkv"], c["D"], self.adt)
                    K, Vv = _dev(Kh, device), _dev(Vh, device)
                cp["kv"].append((K, Vv))
                cp["attn_out"].append(torch.empty(n, c["Hq"], c["D"], **f32))
            if base is None:
                if B == 1:
                    lg, tok = synth.logits_and_draft(seed, (key, 3000), self.parent, V, self.ldt, p_match=0.8)
                else:
                    parts = [synth.logits_and_draft(seed, (key, 3000, b), t, V, self.ldt, p_match=0.8)
                             for b, t in enumerate(self.trees)]
                    lg = np.concatenate([p[0] for p in parts])
                    tok = np.concatenate([p[1] for p in parts]).astype(np.int32)
                cp["logits"], cp["tok"] = _dev(lg, device), _dev(tok, device)
            else:
                cp["logits"], cp["tok"] = base["logits"].clone(), base["tok"]
            gl = [ddt.GdnLayer(q=a["q"].data_ptr(), k=a["k"].data_ptr(), v=a["v"].data_ptr(),
                               alpha=a["alpha"].data_ptr(), beta=a["beta"].data_ptr(),
                               S_c=a["S_c"].data_ptr(), node_u=u.data_ptr(), x=x["x"].data_ptr(),
                               prefix=x["prefix"].data_ptr())
                  for a, x, u in zip(cp["gdn"], cp["conv"], cp["gdn_u"])]
            al = [ddt.AttnLayer(a["Kt"].data_ptr(), a["Vt"].data_ptr(), K.data_ptr(), Vv.data_ptr())
                  for a, (K, Vv) in zip(cp["attn"], cp["kv"])]
            cp["gdn_table"] = ddt.layer_table(gl, device)
            cp["attn_table"] = ddt.layer_table(al, device)
            self.copy.append(cp)
        # copy 0 under the names of a single-copy step
        for k in ("gdn", "conv", "gdn_out", "gdn_u", "conv_out", "attn", "kv", "attn_out", "logits", "tok"):
            setattr(self, k, self.copy[0][k])
        self.T = torch.tensor(self.T0.astype(np.int32), device=device)
        self._T0d = torch.tensor(self.T0.astype(np.int32), device=device)
        self.attn_ws = None
        if self.n_attn:
            nb = ddt.ddt_tree_attn_workspace(self.tb, c["Hq"], c["Hkv"], c["D"], self.T_max)
            self.attn_ws = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None
        self.walk_ws = torch.empty(ddt.ddt_accept_walk_workspace(self.tb, V), dtype=torch.uint8, device=device)
        self.amax = torch.empty(n, **i32)
        self.path = torch.empty(B, self.tb.n_max, **i32)
        self.L = torch.empty(B, **i32)
        self.bonus = torch.empty(B, **i32)
        self.timer = None  # {op: [(start, end) events]} while timing eager steps
        self.fused_step = False  # steps run each conv + delta-net pair as one fused call (setup_fused)

    # ------------------------------------------------------------------ step
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

    def reset_T(self):
        """Put the committed lengths back to their configured values."""
        self.T.copy_(self._T0d)

    def setup_fused(self):
        """Buffers of the fused variant of the step, where each conv + delta-net
        pair is one ddt_tree_conv_gdn call on the conv's x (its channels are
        the layer's q | k | v): fp32 gates, the normalised keys handed to the
        commit, and the commit's layer table (fused layers commit as fp32)."""
        import torch
        ddt, c, n = self.ddt, self.c, self.n
        f32 = dict(dtype=torch.float32, device=self.device)
        self.fz, gl = [], []
        for g, x, u in zip(self.gdn, self.conv, self.gdn_u):
            f = dict(alpha=g["alpha"].float(), beta=g["beta"].float(),
                     q=torch.zeros(n, c["Hk"], c["dk"], **f32), k=torch.zeros(n, c["Hk"], c["dk"], **f32),
                     v=torch.zeros(n, c["Hv"], c["dv"], **f32))
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

    def step(self, ci=0, stream=None, fused=None):
        """One verify step on copy ci of the inputs (fused: each conv +
        delta-net pair as one fused layer call; copy 0 only; None: the
        workload's own choice, fused_step)."""
        if fused is None:
            fused = self.fused_step
        ddt, c, cp = self.ddt, self.c, self.copy[ci]
        gdt = {"bf16": ddt.DDT_BF16, "f32": ddt.DDT_F32}[self.gdt]
        self._timed("plan", lambda: ddt.ddt_tree_plan(self.tb, c["levels"], stream))
        gi = ai = 0
        for kind in self.pattern:
            if kind == "G":
                x, g, l = cp["conv"][gi], cp["gdn"][gi], gi
                gi += 1
                if fused:
                    self._timed("fused", lambda: self.fused_call(l, stream))
                    continue
                self._timed("conv", lambda: ddt.ddt_tree_conv(self.tb, x["x"], x["prefix"], x["w"], 0,
                                                             cp["conv_out"][l], stream))
                self._timed("gdn", lambda: ddt.ddt_tree_gdn(
                    self.tb, g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S_c"], 1.0,
                    cp["gdn_out"][l], None, cp["gdn_u"][l], stream))
            else:
                at, (K, V), a = cp["attn"][ai], cp["kv"][ai], ai
                ai += 1
                self._timed("attn", lambda: ddt.ddt_tree_attn(
                    self.tb, at["q"], K, V, self.pt, self.T, self.T_max, at["Kt"], at["Vt"],
                    cp["attn_out"][a], self.attn_ws, stream=stream))
        self._timed("walk", lambda: ddt.ddt_accept_walk(self.tb, cp["logits"], cp["tok"], self.amax,
                                                        self.path, self.L, self.bonus, self.walk_ws,
                                                        stream))
        table = self.fused_table if fused else cp["gdn_table"]
        kvdt = {"f16": ddt.DDT_F16, "f32": ddt.DDT_F32}[self.adt]
        self._timed("commit", lambda: ddt.ddt_commit_state(
            self.tb, self.path, self.L, ddt.DDT_COMMIT_UPDATE, table if self.n_gdn else None,
            self.n_gdn, c["Hk"], c["Hv"], c["dk"], c["dv"], ddt.DDT_F32 if fused else gdt, c["C"], gdt,
            cp["attn_table"] if self.n_attn else None, self.n_attn, c.get("Hkv", 1), c.get("D", 8), kvdt, self.pt,
            self.T if self.n_attn else None, stream,
            cache_pages=self.max_pages if (self.n_attn and self.pt is None) else None))

    def op_batches(self):
        """Idempotent calls of the ops for batch timing: every layer's conv,
        every layer's delta-net, every attention layer's call (each on its own
        cache, as in the step), and the plan and walk (20 each)."""
        ddt, c, cp = self.ddt, self.c, self.copy[0]
        conv = [lambda x=x, y=y: ddt.ddt_tree_conv(self.tb, x["x"], x["prefix"], x["w"], 0, y)
                for x, y in zip(self.conv, self.conv_out)]
        gdn = [lambda g=g, o=o, u=u: ddt.ddt_tree_gdn(self.tb, g["q"], g["k"], g["v"], g["alpha"],
                                                      g["beta"], g["S_c"], 1.0, o, None, u)
               for g, o, u in zip(self.gdn, self.gdn_out, self.gdn_u)]
        plan = [lambda: ddt.ddt_tree_plan(self.tb, c["levels"])] * 20
        walk = [lambda: ddt.ddt_accept_walk(self.tb, self.logits, self.tok, self.amax, self.path,
                                            self.L, self.bonus, self.walk_ws)] * 20
        attn = [lambda at=at, kv=kv, o=o: ddt.ddt_tree_attn(self.tb, at["q"], kv[0], kv[1], self.pt, self.T,
                                                            self.T_max, at["Kt"], at["Vt"], o, self.attn_ws)
                for at, kv, o in zip(cp.get("attn", []), cp.get("kv", []), cp.get("attn_out", []))]
        out = {"plan": plan, "conv": conv, "gdn": gdn, "walk": walk, "attn": attn}
        if hasattr(self, "fz"):
            out["fused"] = [lambda l=l: self.fused_call(l) for l in range(self.n_gdn)]
        return out

    # ---------------------------------------------------------------- bytes
    def _e(self, which):
        return ELEM[{"g": self.gdt, "a": self.adt, "l": self.ldt}[which]]

    def op_bytes(self, T, L):
        """Algorithmic HBM bytes of one call of each op, summed over the
        batch's sequences (T, L: per-sequence committed and accepted
        lengths): every input read once, every output written once.  The
        delta-net call reads the committed state and the commit writes the
        new one; the commit also writes the conv prefixes and the accepted
        K/V."""
        c, n, B = self.c, self.n, self.B
        T = np.atleast_1d(np.asarray(T, dtype=np.float64))
        L = np.atleast_1d(np.asarray(L, dtype=np.float64))
        eg, ea, el = self._e("g"), self._e("a"), self._e("l")
        W1 = c["W"] - 1
        out = {"plan": n * 4 + (B + 1) * 4 + n * (4 + 8 + 4 * max(W1, 1)) + B * 4,
               "conv": 0, "gdn": 0, "fused": 0, "attn": 0,
               "walk": n * synth.VOCAB * el + n * 4 + n * 4 + B * (self.tb.n_max * 4 + 8), "commit": 0}
        if self.n_gdn:
            state = c["Hv"] * c["dv"] * c["dk"] * 4
            out["conv"] = n * c["C"] * eg + B * W1 * c["C"] * eg + c["C"] * c["W"] * eg + n * c["C"] * 4
            out["gdn"] = (B * state + n * c["Hk"] * c["dk"] * eg * 2 + n * c["Hv"] * c["dv"] * eg
                          + n * c["Hv"] * eg * 2 + n * c["Hv"] * c["dv"] * 4)
            out["commit"] += self.n_gdn * B * (state + W1 * c["C"] * eg)
            # the fused layer: x, prefix and taps in, gates (fp32) and state in, o out
            out["fused"] = (n * c["C"] * eg + B * W1 * c["C"] * eg + c["C"] * c["W"] * eg + B * state
                            + n * c["Hv"] * 4 * 2 + n * c["Hv"] * c["dv"] * 4)
        if self.n_attn:
            out["attn"] = (float(T.sum()) * c["Hkv"] * c["D"] * ea * 2 + n * c["Hq"] * c["D"] * ea
                           + n * c["Hkv"] * c["D"] * ea * 2 + n * c["Hq"] * c["D"] * 4)
            out["commit"] += float(L.sum()) * c["Hkv"] * c["D"] * ea * 2 * self.n_attn
        return out

    def attn_bytes(self, T):
        return self.op_bytes([T], [0])["attn"]

    def kernel_bytes(self, L):
        """Bytes the kernels move beyond the algorithmic ones, by design: the
        delta-net call also writes every node's u (for the commit), and the
        commit's state rebuild reads the committed state and the u, keys and
        gates of the accepted path."""
        c, n, B = self.c, self.n, self.B
        if not self.n_gdn:
            return {"gdn": 0, "fused": 0, "commit": 0}
        Ls = float(np.atleast_1d(np.asarray(L, dtype=np.float64)).sum())
        eg = self._e("g")
        ek = 4 if self.fused_step else eg  # the keys the commit reads: the fused layer hands out fp32
        state = c["Hv"] * c["dv"] * c["dk"] * 4
        return {"gdn": n * c["Hv"] * c["dv"] * 4,
                "fused": n * c["Hv"] * c["dv"] * 4 + n * c["Hk"] * c["dk"] * 4,
                "commit": self.n_gdn * (B * state + Ls * (c["Hv"] * c["dv"] * 4 + c["Hk"] * c["dk"] * ek
                                                         + c["Hv"] * eg))}

    def calls(self):
        g, f = (0, self.n_gdn) if self.fused_step else (self.n_gdn, 0)
        return {"plan": 1, "conv": g, "gdn": g, "fused": f, "attn": self.n_attn, "walk": 1, "commit": 1}

    def step_bytes(self, T, L):
        """Algorithmic HBM bytes of one step (the sum over its calls)."""
        b, k = self.op_bytes(T, L), self.calls()
        return sum(k[o] * v for o, v in b.items())

    def attn_flops(self, T):
        """Matrix flops of one attention layer over the cache: Q K^T and P V,
        2 flops per multiply-add, every (node, q-head) row of each sequence."""
        c = self.c
        return sum(4.0 * c["Hq"] * s * float(t) * c["D"]
                   for s, t in zip(self.sizes, np.atleast_1d(np.asarray(T, dtype=np.float64))))

    def bound_ms(self, T, L):
        """Time of one step at the chip's peaks: each attention layer of each
        sequence takes the longer of its bytes at 8 TB/s and its matrix flops
        at the dense fp16 peak; everything else its bytes at 8 TB/s."""
        c = self.c
        T = np.atleast_1d(np.asarray(T, dtype=np.float64))
        other = self.step_bytes(T, L) - self.n_attn * self.op_bytes(T, L)["attn"]
        ms = other / (HBM_PEAK_GBPS * 1e6)
        if not self.n_attn:
            return ms
        ea = self._e("a")
        for s, t in zip(self.sizes, T):
            by = t * c["Hkv"] * c["D"] * ea * 2 + s * c["Hq"] * c["D"] * (ea + 4) + s * c["Hkv"] * c["D"] * ea * 2
            fl = 4.0 * c["Hq"] * s * t * c["D"]
            ms += self.n_attn * max(by / (HBM_PEAK_GBPS * 1e6), fl / (MFMA_F16_PEAK_TFLOPS * 1e9))
        return ms


def Stack(device, seed=0, cfg=None, headroom_steps=256):
    """The 128K hybrid stack: (G, G, G, A) x 16 over one 22-node tree."""
    c = dict(synth.STACK if cfg is None else cfg)
    tree = synth.random_tree(synth.rng_for(seed, 3, 18), c["N"], c["levels"])
    per = c["n_gdn"] // c["n_attn"]
    return Workload(device, c, [tree], [c["T"]], (["G"] * per + ["A"]) * c["n_attn"], seed=seed, key=3,
                    room_steps=headroom_steps)


def build_config(name, device, seed, room_steps):
    """One of the other four workloads, sized as synth states them."""
    if name == "tiny":
        c = dict(synth.TINY, levels=8, dtype_gdn="f32", dtype_attn="f32", dtype_logits="f32")
        return Workload(device, c, [np.array(c["parent"], np.int32)], [c["T"]], ["G", "A"], seed=seed, key=10,
                        room_steps=room_steps)
    if name == "layer_gdn":
        c = dict(synth.LAYER_GDN)
        tree = synth.random_tree(synth.rng_for(seed, 1, 18), c["N"], c["levels"])
        # 256 copies, each 2 MB of state + 0.4 MB of layer inputs + 6.7 MB of
        # logits, against a 256 MB last-level cache
        return Workload(device, c, [tree], [0], ["G"], copies=256, seed=seed, key=11, room_steps=room_steps)
    if name == "layer_attn":
        c = dict(synth.LAYER_ATTN, W=4, C=0, Hk=1, Hv=1, dk=16, dv=16)  # no delta-net layer
        tree = synth.random_tree(synth.rng_for(seed, 2, 18), c["N"], c["levels"])
        # four caches of 134 MB each against a 256 MB last-level cache
        return Workload(device, c, [tree], [c["T"]], ["A"], copies=4, seed=seed, key=12,
                        room_steps=4 * room_steps)
    if name == "batched":
        c = dict(synth.BATCHED)
        trees, T = synth.batched_trees(seed)
        per = c["n_gdn"] // c["n_attn"]
        return Workload(device, c, trees, T, (["G"] * per + ["A"]) * c["n_attn"], paged=True, seed=seed,
                        key=13, room_steps=room_steps)
    raise ValueError(name)


# ------------------------------------------------------------------ timing
def capture(wl, fused=None):
    """One HIP graph of one step per copy (after one eager round)."""
    import torch
    for ci in range(wl.ncopies):
        wl.step(ci, fused=fused)
    torch.cuda.synchronize()
    check_status(wl)
    wl.reset_T()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for ci in range(wl.ncopies):
            wl.step(ci, fused=fused)
    torch.cuda.synchronize()
    return g


def run_steps(wl, graph, k, fused=None):
    for _ in range(k):
        if graph is not None:
            graph.replay()
        else:
            for ci in range(wl.ncopies):
                wl.step(ci, fused=fused)


def settle(wl, graph, seconds, fused=None):
    """Untimed replays for `seconds` (the clock ramps under load), with the
    committed length put back after every batch; returns the steps run."""
    import torch
    t_end, n = time.perf_counter() + seconds, 0
    while True:
        run_steps(wl, graph, SETTLE_BATCH, fused)
        wl.reset_T()
        torch.cuda.synchronize()
        n += SETTLE_BATCH * wl.ncopies
        if time.perf_counter() >= t_end:
            return n


def check_status(wl):
    st = wl.tb.status.cpu().numpy()
    if st.any():
        raise RuntimeError(f"{wl.name}: device status {st}")


def time_total(wl, graph, k, fused=None):
    """k replays under one event pair, from the configured context: ms per
    step, the per-sequence mean accepted length, and the host wall time."""
    import torch
    wl.reset_T()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run_steps(wl, graph, k, fused)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_status(wl)
    steps = k * wl.ncopies
    if wl.n_attn:
        L = (wl.T.cpu().numpy().astype(np.int64) - wl.T0) / steps
    else:
        L = wl.L.cpu().numpy().astype(np.float64)
    return e0.elapsed_time(e1) / steps, L, wall


def time_each(wl, graph, k, fused=None):
    """k replays, each under its own event pair: per-step times (a replay of
    a graph of several copies counts as that many steps)."""
    import torch
    wl.reset_T()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    for a, b in ev:
        a.record()
        run_steps(wl, graph, 1, fused)
        b.record()
    torch.cuda.synchronize()
    check_status(wl)
    return np.array([a.elapsed_time(b) / wl.ncopies for a, b in ev])


def dist(ms):
    return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90)), "mean": float(np.mean(ms))}


def copy_bandwidth(device, nbytes=1 << 30, reps=20):
    """Achieved rate of a plain device-to-device copy (torch copy_, which
    runs the runtime's copy kernel): (bytes read + written) / time."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return gbps


def measure_config(wl, steps, warmup, settle_s, copy_gbps, use_graph=True):
    """Per-step time (median, p10, p90 of one-by-one timed steps), bytes,
    achieved rate and the chip bound of one workload."""
    graph = capture(wl) if use_graph else None
    run_steps(wl, graph, max(1, warmup // wl.ncopies))
    n_settle = settle(wl, graph, settle_s)
    k = max(10, steps // wl.ncopies) if wl.ncopies > 1 else max(steps, MIN_EACH_STEPS)
    ms_mean, L, _ = time_total(wl, graph, k)
    each = time_each(wl, graph, k)
    d = dist(each)
    T_mid = wl.T0 + np.asarray(L) * (k * wl.ncopies) / 2 if wl.n_attn else wl.T0
    nbytes = wl.step_bytes(T_mid, L)
    bound = wl.bound_ms(T_mid, L)
    gbps = nbytes / (d["median"] * 1e-3) / 1e9
    del graph
    return {"workload": wl.name, "sequences": wl.B, "nodes": wl.sizes, "context": [int(t) for t in wl.T0],
            "layers": f"{wl.n_gdn} G + {wl.n_attn} A", "copies_cycled": wl.ncopies,
            "steps_per_s": 1000.0 / d["median"], "ms_per_step": d, "ms_per_step_one_event_pair": ms_mean,
            "timed_steps": int(len(each) * wl.ncopies), "settle_steps": n_settle,
            "algorithmic_bytes_per_step": nbytes, "GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
            "frac_copy": gbps / copy_gbps, "bound_ms": bound, "frac_of_bound": bound / d["median"],
            "mean_accepted_L": [float(x) for x in np.atleast_1d(L)]}


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


def unfused_stack_bench(st, steps, settle_s):
    """The same 128K step with each linear-attention layer as two launches,
    ddt_tree_conv then ddt_tree_gdn (on the layer's own bf16 q, k, v), timed
    like the headline step: eager round, one captured graph, settle replays
    with the committed length put back, then `steps` timed replays from the
    configured context."""
    graph = capture(st, fused=False)
    settle(st, graph, settle_s, fused=False)
    ms, _, _ = time_total(st, graph, steps, fused=False)
    each = time_each(st, graph, steps, fused=False)
    del graph
    st.reset_T()
    d = dist(each)
    return {"workload": st.name + "_unfused_conv_then_gdn", "ms_per_step": ms, "ms_per_step_each": d,
            "steps_per_s": 1000.0 / ms, "layers": st.n_gdn,
            "timed": "graph-replayed step after a settle phase"}


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
    st.reset_T()
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
    whole step.  First the full verify walk; then gated delta-net + conv
    layers one after another, each with its commit of the accepted path
    (state replay and conv prefix), until ``gdn_s`` seconds have passed;
    then attention one (layer, KV head) at a time until ``attn_s`` seconds
    have passed; per-layer and per-head means are scaled to the 48 + 16 x 4
    of one step.  Inputs are copied from the device before the clock
    starts."""
    import torch
    import oracle
    c = st.c
    N = c["N"]
    nthreads = len(os.sched_getaffinity(0))
    torch.set_num_threads(nthreads)
    par = st.parent
    host = lambda t: t.detach().cpu()  # noqa: E731
    u16 = lambda t: host(t).view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    T = int(st.T0[0])
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

    lg, tok = u16(st.logits), host(st.tok).numpy()
    t0 = time.perf_counter()
    am = oracle.argmax_rows(lg)
    paths, _, _ = oracle.accept_walk(par, tok, am)
    t_walk = time.perf_counter() - t0
    path = list(paths[0])
    t_gdn, n_gdn = 0.0, 0
    while n_gdn < c["n_gdn"] and t_gdn < gdn_s:
        g0, x0 = gdn_in(n_gdn)
        t0 = time.perf_counter()
        oracle.tree_conv(par, x0["x"], x0["prefix"], x0["w"])
        oracle.tree_gdn(par, g0["q"], g0["k"], g0["v"], g0["alpha"], g0["beta"], g0["S_c"])
        oracle.commit_gdn_state(g0["S_c"], g0["q"], g0["k"], g0["v"], g0["alpha"], g0["beta"], path, 0)
        oracle.commit_conv_prefix(x0["prefix"], x0["x"], path, 0)
        t_gdn += time.perf_counter() - t0
        n_gdn += 1
    t_attn, n_heads = 0.0, 0
    while n_heads < c["n_attn"] * c["Hkv"] and t_attn < attn_s:
        q1, Kh, Vh, kt1, vt1 = attn_in(n_heads // c["Hkv"], n_heads % c["Hkv"])
        t0 = time.perf_counter()
        oracle.tree_attn(par, q1, Kh, Vh, [T], kt1, vt1)
        t_attn += time.perf_counter() - t0
        n_heads += 1
    step_s = (c["n_gdn"] * t_gdn / n_gdn + c["n_attn"] * c["Hkv"] * t_attn / n_heads + t_walk)
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": nthreads, "kind": "oracle",
            "sample": (f"numpy fp64 oracle: full argmax+walk over {N}x{synth.VOCAB}; {n_gdn} of "
                       f"{c['n_gdn']} gated delta-net+conv layers with their commit (state replay of the "
                       f"accepted path, conv prefix); {n_heads} of {c['n_attn'] * c['Hkv']} (attention "
                       f"layer, KV head) pairs ({G} q-heads x {N} nodes each) at T={T}; means scaled to "
                       f"one step (the K/V append of the accepted tokens is not timed); sample took "
                       f"{t_gdn + t_attn + t_walk:.1f} s of CPU time"),
            "seconds_per_step": step_s}


def kernel_timings(st, reps, settle_s=0.3):
    """Per-call times of the step's ops, with HIP events on the launch stream.
    The commit is timed call by call inside eager steps; the others (plan,
    conv, delta-net, attention, walk) as graph-replayed back-to-back batches
    under one event pair (all 16 attention layers, each on its own cache,
    as the step runs them), so that a call's time is its kernels' time on
    the stream and not the gaps an event pair or an eager launch adds; each
    batch is replayed untimed for settle_s seconds first."""
    import torch
    timer = {}
    for op in ("commit",):
        st.reset_T()
        st.timer = {op: []}
        for _ in range(reps):
            st.step()
            torch.cuda.synchronize()
        timer[op] = [a.elapsed_time(b) for a, b in st.timer[op]]
    st.timer = None
    st.reset_T()
    for op, calls in st.op_batches().items():
        for fn in calls:  # one untimed eager round first
            fn()
        gb = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gb):
            for fn in calls:
                fn()
        gb.replay()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle_s  # the clock falls while the host captures
        while time.perf_counter() < t_end:
            gb.replay()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gb.replay()
        b.record()
        torch.cuda.synchronize()
        timer[op] = [a.elapsed_time(b) / (reps * len(calls))]
        del gb
    return timer


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the measurements of the widenings beside the step")
    ap.add_argument("--configs", default="all",
                    help="the other workloads measured beside the stack: all, none, or a comma list of "
                         + ", ".join(CONFIGS))
    ap.add_argument("--kernel-reps", type=int, default=5, help="eager steps timed per attention call")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed sustained steps before timing (the GPU clock ramps "
                         "over a few hundred ms of load)")
    ap.add_argument("--draft", type=int, default=0, metavar="B",
                    help="only time the draft top-K and tree build for B sequences and print that line")
    ap.add_argument("--workload", default=None, metavar="NAME",
                    help="measure only this workload (one of the --configs names) and print its line; "
                         "for profiling one workload alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference kernel "
                         "that scales the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the verify step of one batch runs on a single MI355X; "
              "runs over several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)
    configs = [] if args.configs == "none" else (list(CONFIGS) if args.configs == "all"
                                                 else [x for x in args.configs.split(",") if x])
    for name in configs:
        if name not in CONFIGS:
            print(f"unknown workload {name}; choose from {', '.join(CONFIGS)}", file=sys.stderr)
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
    if args.workload:
        if args.workload not in CONFIGS:
            print(f"unknown workload {args.workload}; choose from {', '.join(CONFIGS)}", file=sys.stderr)
            sys.exit(2)
        copy_gbps = copy_bandwidth(dev)
        print(f"[bench] workload {args.workload} alone", file=sys.stderr, flush=True)
        wl = build_config(args.workload, dev, args.seed, headroom(args.warmup, args.steps, args.kernel_reps))
        res = measure_config(wl, args.steps, args.warmup, args.settle, copy_gbps, not args.no_graph)
        print(json.dumps({"workload": args.workload, **res}), flush=True)
        return
    room = headroom(args.warmup, args.steps, args.kernel_reps)
    copy_gbps = copy_bandwidth(dev)
    print(f"[bench] device copy {copy_gbps:.0f} GB/s; building the 128K stack (seed {args.seed})",
          file=sys.stderr, flush=True)
    st = Stack(dev, seed=args.seed, headroom_steps=room)
    # each linear-attention layer runs as one fused conv -> delta-net call
    # (ddt_tree_conv_gdn), the faster of the two paths; the unfused step
    # (ddt_tree_conv, then ddt_tree_gdn) is timed beside it under `next`
    st.setup_fused()
    st.fused_step = True
    torch.cuda.synchronize()
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    check_status(st)
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        try:
            graph = capture(st)
        except Exception as e:  # noqa: BLE001 - report and time eagerly instead
            print(f"[bench] graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph, use_graph = None, False
    # The GPU clock ramps up over a few hundred ms of sustained load and falls
    # back while the host builds the inputs, so untimed steps keep the GPU
    # busy for --settle seconds first.  The committed length is put back
    # before every timed phase, so every timed step runs at the configured
    # context (plus the few tokens its own phase has committed).
    n_settle = settle(st, graph, args.settle)
    print(f"[bench] settled for {n_settle} steps; timing {args.steps} steps (graph={use_graph})",
          file=sys.stderr, flush=True)
    ms, L_mean, wall = time_total(st, graph, args.steps)
    each = time_each(st, graph, args.steps)
    d = dist(each)
    L_step = float(np.mean(L_mean))
    T_mid = st.T0 + L_step * args.steps / 2
    timer = kernel_timings(st, args.kernel_reps)
    ob = st.op_bytes(T_mid, [max(L_step, 1.0)])
    kb = st.kernel_bytes([max(L_step, 1.0)])
    per_step = st.calls()
    kernels = {}
    for op in ("plan", "fused", "conv", "gdn", "attn", "walk", "commit"):
        us = float(np.mean(timer[op])) * 1e3
        gbps = ob[op] / (us * 1e-6) / 1e9
        kernels[op] = {"us_per_call": us, "calls_per_step": per_step[op], "bytes_per_call": ob[op],
                       "GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                       "timed": "per call in eager steps" if op == "commit"
                       else "graph-replayed back-to-back batch"}
        if per_step[op] == 0:
            kernels[op]["note"] = "the unfused path's kernel, not in the headline step"
        if op in kb:
            kernels[op]["kernel_bytes_per_call"] = ob[op] + kb[op]
            kernels[op]["kernel_GBps"] = (ob[op] + kb[op]) / (us * 1e-6) / 1e9
    attn_ms = kernels["attn"]["us_per_call"] * 1e-3
    attn_bytes = ob["attn"]
    attn_flops = st.attn_flops(T_mid)
    kernels["attn"]["mfma"] = {
        "flops_per_call": attn_flops, "TFLOPs": attn_flops / (attn_ms * 1e-3) / 1e12,
        "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": attn_flops / (attn_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    src = open(os.path.join(ROOT, "tree_verification_ddtree_amd", "csrc", "attn.hip"), "rb").read()
    traffic = _traffic(hashlib.sha256(src).hexdigest())
    step_bytes = st.step_bytes(T_mid, [L_step])
    step_gbps = step_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms,
        "ms_per_step_each": d,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": synth.STACK["name"],
            "budget": st.c["N"], "context": int(st.T0[0]), "gdn_layers": st.n_gdn,
            "attn_layers": st.n_attn, "kv_heads": st.c["Hkv"], "q_heads": st.c["Hq"],
            "head_dim": st.c["D"], "gdn_heads": [st.c["Hk"], st.c["Hv"]], "state": [st.c["dv"], st.c["dk"]],
            "conv_channels": st.c["C"], "vocab": synth.VOCAB, "graph": use_graph,
            "linear_attention_layer": "fused conv -> SiLU -> q|k|v -> L2 norm -> delta-net (ddt_tree_conv_gdn)",
            "inputs": "fp16 KV cache and attention, bf16 conv input/logits, fp32 gates, state and accumulation",
            "mean_accepted_L": L_step,
        },
        "achieved_GBps_step": step_gbps,
        "roofline_frac_step": step_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "copy_GBps": copy_gbps,
        "wall_s_timed": wall,
        "roofline": {
            "kernel": "ddt_tree_attn (attn_mfma_kernel + attn_combine_kernel)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "bytes_per_call": attn_bytes, "ms_per_call": attn_ms,
        },
        "roofline_step": {
            "what": "the whole verify step (all kernels, one graph replay per step)",
            "bound": "hbm", "achieved": step_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": step_gbps / HBM_PEAK_GBPS, "frac_copy": step_gbps / copy_gbps,
            "bytes_per_step": step_bytes, "ms_per_step": ms, "bound_ms": st.bound_ms(T_mid, [L_step]),
        },
        "kernels": kernels,
        "cpu_baseline": None,
        "library_source_sha256": ddt.ddt_source_hash(),
    }
    if not args.no_next:
        # widenings beside the step (not part of `value`)
        cs = 0.0 if args.no_cpu_baseline else 3.0
        print("[bench] unfused conv, delta-net step", file=sys.stderr, flush=True)
        uf = unfused_stack_bench(st, args.steps, args.settle)
        uf["fused_step_speedup"] = uf["ms_per_step"] / ms
        uf["conv_plus_gdn_us"] = kernels["conv"]["us_per_call"] + kernels["gdn"]["us_per_call"]
        uf["fused_us"] = kernels["fused"]["us_per_call"]
        out["next"] = {"unfused_stack": uf}
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
    # the stack's own line first, then the other workloads (their caches replace the stack's)
    out["configs"] = {"stack": {"workload": st.name, "steps_per_s": 1000.0 / d["median"], "ms_per_step": d,
                                "algorithmic_bytes_per_step": step_bytes,
                                "GBps": step_bytes / (d["median"] * 1e-3) / 1e9,
                                "frac_hbm_peak": step_bytes / (d["median"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                "frac_copy": step_bytes / (d["median"] * 1e-3) / 1e9 / copy_gbps,
                                "bound_ms": st.bound_ms(T_mid, [L_step]),
                                "frac_of_bound": st.bound_ms(T_mid, [L_step]) / d["median"]}}
    del graph, st
    torch.cuda.empty_cache()
    for name in configs:
        print(f"[bench] workload {name}", file=sys.stderr, flush=True)
        wl = build_config(name, dev, args.seed, room)
        out["configs"][name] = measure_config(wl, args.steps, args.warmup, args.settle, copy_gbps, use_graph)
        del wl
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
