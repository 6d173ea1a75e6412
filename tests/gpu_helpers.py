"""Shared helpers of the GPU parity tests: build a quantized matrix with the
oracle on the CPU, upload it, and compare results to the bar of the tests."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from nested_int_matmul_amd import inputs

REL_L2_TOL = 1e-3   # rel-L2 bound on matmul outputs
MAX_ABS_TOL = 2e-2  # max-abs bound on matmul outputs


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=6)
def quantized(workload, n, k, group, layer=0, matrix=0, outlier_frac=0.0):
    """Seeded weights -> oracle codes/alpha/zero (numpy) + device copies.
    Cached: callers must not modify the returned arrays or tensors."""
    w = inputs.gaussian_weights(workload, n, k, layer, matrix, outlier_frac=outlier_frac)
    q, a, z = oracle.quantize_minmax(w, group)
    d = dev()
    return {
        "w": w, "q": q, "alpha": a, "zero": z, "N": n, "K": k, "group": group,
        "q_d": torch.from_numpy(q).to(d),
        "alpha_d": torch.from_numpy(a).to(d),
        "zero_d": torch.from_numpy(z).to(d),
    }


def x_device(x_bits: np.ndarray):
    return torch.from_numpy(x_bits.view(np.int16)).to(dev())


def compare(y_gpu, y_ref, what=""):
    """rel-L2 and max-abs of a GPU result against the float64 oracle."""
    y = y_gpu.detach().double().cpu().numpy() if hasattr(y_gpu, "cpu") else np.asarray(y_gpu)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = y - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mab = float(np.max(np.abs(err))) if err.size else 0.0
    note(f"  parity {what}: rel-L2 {rel:.3e} max-abs {mab:.3e}")
    assert rel <= REL_L2_TOL, f"{what}: rel-L2 {rel} > {REL_L2_TOL}"
    assert mab <= MAX_ABS_TOL, f"{what}: max-abs {mab} > {MAX_ABS_TOL}"
    return rel, mab
