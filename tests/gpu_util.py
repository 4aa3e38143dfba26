"""Helpers for the GPU parity tests: moving synth arrays to the device and
the tolerance metric.  Imports no oracle arithmetic."""
import os

import numpy as np
import torch

TOL = 2e-3  # max relative error for floating-point outputs and states


def dev(a, device="cuda:0"):
    """numpy -> torch device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    return t.detach().cpu().numpy()


def rel_err(got, ref, axes):
    """max over slices of max|got-ref| / max|ref|; a slice keeps the leading
    axes listed in ``axes`` fixed (e.g. (0, 1) = per node and head)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    red = tuple(i for i in range(ref.ndim) if i not in axes)
    num = np.abs(got - ref).max(axis=red) if red else np.abs(got - ref)
    den = np.abs(ref).max(axis=red) if red else np.abs(ref)
    den = np.where(den == 0, 1.0, den)
    r = float((num / den).max())
    log = os.environ.get("DDT_REL_LOG")
    if log:  # record observed errors: one line per comparison
        with open(log, "a") as f:
            f.write(f"{os.environ.get('PYTEST_CURRENT_TEST', '?').split(' ')[0]} {r:.3e}\n")
    return r


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
