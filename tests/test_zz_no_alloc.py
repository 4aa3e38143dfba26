"""The allocation-free walk (ddt_accept_walk_noalloc) against the walk with a
caller workspace (ddt_accept_walk), through the C ABI: two calls in a row,
the second on a smaller input, each equal to the workspace call bit for bit."""
import numpy as np
import pytest
import torch

import synth
import tree_verification_ddtree_amd as ddt
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def _case(gpu, seed, sizes, V, dtype):
    trees = [synth.random_tree(synth.rng_for(seed, 70, b), s, 10) for b, s in enumerate(sizes)]
    par, off = synth.concat_trees(trees)
    tb = ddt.TreeBatch(par, off, 4, gpu)
    ddt.ddt_tree_plan(tb, 10)
    lg, tok = [], []
    for b, t in enumerate(trees):
        l_, t_ = synth.logits_and_draft(seed, (71, b), t, V, dtype, p_match=0.85)
        lg.append(l_)
        tok.append(t_)
    return tb, dev(np.concatenate(lg)), dev(np.concatenate(tok).astype(np.int32))


def _outs(gpu, tb):
    i32 = dict(dtype=torch.int32, device=gpu)
    return (torch.full((tb.n_total,), -7, **i32), torch.full((tb.B, tb.n_max), -7, **i32),
            torch.full((tb.B,), -7, **i32), torch.full((tb.B,), -7, **i32))


def test_noalloc_walk_equals_workspace_walk_twice(gpu):
    cases = [(0, [64, 22, 64, 7, 33, 64, 1, 64], synth.VOCAB, "bf16"),   # 319 nodes, full vocabulary
             (1, [22, 5], 5003, "f32")]                                   # then a smaller, ragged one
    for seed, sizes, V, dt in cases:
        banner(f"no-alloc walk: seed={seed} sizes={sizes} V={V} {dt}")
        tb, lg, tok = _case(gpu, seed, sizes, V, dt)
        ws = torch.empty(ddt.ddt_accept_walk_workspace(tb, V), dtype=torch.uint8, device=gpu)
        ref = _outs(gpu, tb)
        ddt.ddt_accept_walk(tb, lg, tok, *ref, ws)
        got = _outs(gpu, tb)
        ddt.ddt_accept_walk_noalloc(tb, lg, tok, *got)
        torch.cuda.synchronize()
        assert not tb.status.cpu().numpy().any()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        assert int(ref[2].max()) > 1   # some drafts were accepted
