"""Shared helpers for the GPU parity tests: moving seeded inputs to the device, running the
library's three calls, and the error measures used against the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

# Tolerances on max|gpu - ref| / max|ref| (per tensor), fixed before any kernel was written:
# bf16 inputs with fp32 accumulation: 2e-2; the fp32 path: 1e-4.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_np(t):
    return t.detach().to("cpu").double().numpy()


def rel_err(gpu, ref):
    gpu = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), "non-finite values in GPU output"
    scale = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (scale if scale > 0 else 1.0))


def per_head_rel_err(gpu, ref, head_axis_from_end):
    """Worst normwise relative error over (batch, head) slices; head axis given from the end."""
    gpu = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = np.moveaxis(gpu, gpu.ndim - head_axis_from_end, 1)
    r = np.moveaxis(ref, ref.ndim - head_axis_from_end, 1)
    worst = 0.0
    for bi in range(r.shape[0]):
        for hi in range(r.shape[1]):
            s = np.abs(r[bi, hi]).max()
            worst = max(worst, float(np.abs(g[bi, hi] - r[bi, hi]).max() / (s if s > 0 else 1.0)))
    return worst


def per_step_rel_err(gpu, ref, axis, floor=1e-2):
    """Worst over the steps along `axis` of max|gpu_t - ref_t| / max|ref_t|, where a step whose
    reference is below `floor` times the largest one is measured against that floor instead (a
    step whose output is near zero, e.g. where Cbar_t . Bbar_t nearly cancels, has no relative
    scale of its own: its absolute error is the usual one)."""
    g = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all()
    g, r = np.moveaxis(g, axis, 0), np.moveaxis(r, axis, 0)
    big = np.abs(r).max()
    worst = 0.0
    for t in range(r.shape[0]):
        s = max(np.abs(r[t]).max(), floor * big, 1e-300)
        worst = max(worst, float(np.abs(g[t] - r[t]).max() / s))
    return worst


def angle_err(gpu_phi, ref_phi):
    d = to_np(gpu_phi) - np.asarray(ref_phi, dtype=np.float64)
    d = (d + math.pi) % (2 * math.pi) - math.pi
    return float(np.abs(d).max())


def to_dev(inp: dict, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
