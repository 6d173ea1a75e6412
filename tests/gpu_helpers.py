"""Shared helpers of the GPU parity tests: build a quantized matrix with the
oracle on the CPU, upload it, and compare results to the bar of the tests."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from nested_int_matmul_amd import inputs

# The stated bar on matmul outputs (rel-L2 and max-abs against the float64
# oracle).
REL_L2_TOL = 1e-3
MAX_ABS_TOL = 2e-2
# Regression bounds on top of the bar, from the fp32 arithmetic of the
# kernels: every product is an exact integer contraction accumulated in fp32,
# so its error is a few fp32 roundings of its partial sums (see term_scale).
# The bounds sit above every measured error (per element at most 2e-6 of
# the term scale); a wrong code is caught by ELEM_REG when one level,
# alpha * 2^(8-r) * |x_k|, exceeds it relative to the term scale (about
# 2.6e-5 at r = 8 and K = 14336, more at lower r or shorter K), and at every
# r by the one-hot read-back test, which checks each weight alone.
REL_L2_REG = 1e-4
ELEM_REG = 1e-5


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
    return upload(q, a, z, group, w=w)


def upload(q, a, z, group, w=None):
    d = dev()
    n, k = q.shape
    return {
        "w": w, "q": q, "alpha": a, "zero": z, "N": n, "K": k, "group": group,
        "q_d": torch.from_numpy(q).to(d),
        "alpha_d": torch.from_numpy(a).to(d),
        "zero_d": torch.from_numpy(z).to(d),
    }


def x_device(x_bits: np.ndarray):
    return torch.from_numpy(x_bits.view(np.int16)).to(dev())


def term_scale(x_bits, q, alpha, zero, group, r):
    """Per output element, the size of the fp32 numbers the kernels sum:
    sqrt(sum_k (x[m,k] * alpha[n,g] * (|S - z| + 256))^2), S the slice and z
    the zero point on the int8 scale.  The kernels contract x with an exact
    integer operand u (u = 2^r + t for r < 8, t at r = 8) and form
    alpha * (2^(8-r) * u - (z + 256)) on the int8 scale, so each term they
    accumulate is at most of that size; their rounding error is relative to
    it (and a constant vector, alpha = 1, carries a correspondingly larger
    absolute error than its small dequantized value)."""
    x = oracle.float_from_bf16_bits(x_bits)
    q = np.asarray(q)
    n, k = q.shape
    g = k // group
    s = oracle.slice_value(q, r).astype(np.float64).reshape(n, g, group)
    a = np.asarray(alpha, dtype=np.float64).reshape(n, g, 1)
    z = np.asarray(zero, dtype=np.float64).reshape(n, g, 1)
    w = (a * (np.abs(s - z) + 256.0)).reshape(n, k)
    return np.sqrt((x * x) @ (w * w).T)


def compare(y_gpu, y_ref, what="", scale=None, reg=REL_L2_REG):
    """rel-L2 and max-abs of a GPU result against the float64 oracle (the
    stated bar), a tighter rel-L2 regression bound `reg`, and, when the
    terms' scale is given, a per-element bound relative to it (so that one
    wrong output element cannot hide in a large matrix).  End-to-end stacks
    pass reg=REL_L2_TOL: there a bf16 rounding of an intermediate may land on
    the other side of a rounding boundary than in float64, a legitimate
    difference far above the per-product bound."""
    y = y_gpu.detach().double().cpu().numpy() if hasattr(y_gpu, "cpu") else np.asarray(y_gpu)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = y - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mab = float(np.max(np.abs(err))) if err.size else 0.0
    msg = f"  parity {what}: rel-L2 {rel:.3e} max-abs {mab:.3e}"
    elem = None
    if scale is not None:
        s = np.asarray(scale, dtype=np.float64)
        assert s.shape == ref.shape
        elem = float(np.max(np.abs(err) / np.maximum(s, 1e-30))) if err.size else 0.0
        msg += f" max err/scale {elem:.3e}"
    note(msg)
    assert rel <= REL_L2_TOL, f"{what}: rel-L2 {rel} > {REL_L2_TOL}"
    assert mab <= MAX_ABS_TOL, f"{what}: max-abs {mab} > {MAX_ABS_TOL}"
    assert rel <= reg, f"{what}: rel-L2 {rel} > regression bound {reg}"
    if elem is not None:
        assert elem <= ELEM_REG, f"{what}: max err/scale {elem} > {ELEM_REG}"
    return rel, mab


def compare_linear(y_gpu, x_bits, q, alpha, zero, group, r, what=""):
    """compare() against oracle.linear on the same inputs, with the
    per-element bound."""
    ref = oracle.linear(x_bits, q, alpha, zero, group, r)
    return compare(y_gpu, ref, what, scale=term_scale(x_bits, q, alpha, zero, group, r))


GUARD = 4096  # guard elements after an output


def guarded_f32(M, N):
    """An fp32 [M, N] output view followed by GUARD guard elements holding a
    sentinel; check() asserts the guard is untouched after a call."""
    buf = torch.empty(M * N + GUARD, dtype=torch.float32, device=dev())
    sentinel = torch.tensor([-1.2345678e30], dtype=torch.float32)
    buf[M * N:] = sentinel.to(dev())
    out = buf[:M * N].view(M, N)

    def check(what=""):
        g = buf[M * N:].cpu()
        assert torch.equal(g, sentinel.expand(GUARD)), f"{what}: write past the output"

    return out, check
