"""GPU parity of the bit-plane storage (one stored copy serving every r).

The planes written by the GPU are compared bit for bit with the oracle's
layout; products read from planes are compared with the float64 oracle's
product at the same r, clamped (Eq. 6) or unclamped (the errata Eq. 8,
Extra-Precision), to rel-L2 1e-3 and max-abs 2e-2.
"""

import numpy as np
import pytest
import torch

import nested_int_matmul_amd as mq
import oracle
from nested_int_matmul_amd import inputs

from gpu_helpers import compare, dev, note, quantized, x_device

pytestmark = pytest.mark.gpu


def _sample_rows(n, count, seed=0):
    rg = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1], rg.choice(n, size=min(count, n), replace=False)]))
    return rows


def _with_edge_rows(m):
    """Codes of a quantized matrix with rows at the clamp edge: all 255 (every
    h all ones and c = 1 for r < 8), all 0, and codes around each threshold."""
    q = m["q"].copy()
    q[5] = 255
    q[6] = 0
    q[7, ::2] = 255 - (np.arange(q.shape[1] // 2) % 16)
    return q


def _ref(xb, q, a, z, g, r, extra):
    if extra:
        return oracle.linear_extra_precision(xb, q, a, z, g, r)
    return oracle.linear(xb, q, a, z, g, r)


@pytest.mark.parametrize("shape", [(17, 1024), (64, 512), (3, 2560)])
def test_pack_bitplanes_bit_exact(shape):
    n, k = shape
    note(f"pack bitplanes {shape}")
    rg = np.random.default_rng(n + k)
    q = rg.integers(0, 256, size=(n, k), dtype=np.uint8)
    q[0] = np.tile(np.arange(256, dtype=np.uint8), k // 256)   # every code
    q[-1] = 255
    got = mq.pack_bitplanes(torch.from_numpy(q).to(dev()))
    torch.cuda.synchronize()
    assert tuple(got.shape) == (8, n, k // 8)
    assert np.array_equal(got.cpu().numpy(), oracle.pack_bitplanes(q))


def test_pack_bitplanes_gemma_down_full_size():
    note("pack bitplanes gemma down full size (sampled rows)")
    m = quantized("gemma9b_mlp", 3584, 14336, 14336, matrix=2, outlier_frac=1e-3)
    got = mq.pack_bitplanes(m["q_d"])
    torch.cuda.synchronize()
    rows = _sample_rows(3584, 24, seed=3)
    want = oracle.pack_bitplanes(m["q"][rows])
    assert np.array_equal(got[:, rows, :].cpu().numpy(), want)


@pytest.mark.parametrize("extra", [False, True])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("r", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_bitplanes_ragged(r, M, group, extra):
    """N = 40 (a ragged last row block), K = 1536 (three superblocks), rows at
    the clamp edge."""
    n, k = 40, 1536
    g = k if group == "K" else 128
    note(f"gemv bitplanes r={r} M={M} g={g} extra={extra}")
    m = quantized("gemma9b_mlp", n, k, g, matrix=7, outlier_frac=1e-2)
    q = _with_edge_rows(m)
    planes = mq.pack_bitplanes(torch.from_numpy(q).to(dev()))
    xb = inputs.activations_bf16("gemma9b_mlp", M, k, matrix=7)
    y = mq.gemv_bitplanes(planes, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb),
                          extra=extra)
    torch.cuda.synchronize()
    compare(y, _ref(xb, q, m["alpha"], m["zero"], g, r, extra),
            f"bitplanes r{r} M{M} g{g} extra{int(extra)}")


@pytest.mark.parametrize("case", [(8, 33, 6144, 128), (1, 17, 65536, "K"), (2, 300, 8192, "K")])
@pytest.mark.parametrize("r", [2, 4, 8])
def test_gemv_bitplanes_chunks_and_max_k(case, r):
    """Several staged activation chunks (M = 8 stages 2048 codes at a time),
    K at the library maximum, and a wider N."""
    M, n, k, group = case
    g = k if group == "K" else 128
    note(f"gemv bitplanes chunks r={r} M={M} N={n} K={k} g={g}")
    m = quantized("tiny_linear", n, k, g, matrix=31)
    planes = mq.pack_bitplanes(m["q_d"])
    xb = inputs.activations_bf16("tiny_linear", M, k, matrix=31)
    for extra in (False, True):
        y = mq.gemv_bitplanes(planes, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb),
                              extra=extra)
        torch.cuda.synchronize()
        compare(y, _ref(xb, m["q"], m["alpha"], m["zero"], g, r, extra),
                f"bitplanes chunks r{r} M{M} K{k} extra{int(extra)}")


@pytest.mark.parametrize("name", ["up", "down"])
@pytest.mark.parametrize("r", [2, 4, 8])
def test_gemv_bitplanes_gemma_full_size(name, r):
    """One stored copy of a Gemma-2-9B MLP matrix served at r = 2, 4, 8 (and
    unclamped at r = 2), checked on sampled rows."""
    n, k = inputs.GEMMA9B_MLP[name]
    idx = {"up": 0, "gate": 1, "down": 2}[name]
    note(f"gemv bitplanes gemma {name} r={r}")
    m = quantized("gemma9b_mlp", n, k, k, matrix=idx, outlier_frac=1e-3)
    planes = mq.pack_bitplanes(m["q_d"])
    xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=idx)
    rows = _sample_rows(n, 200, seed=idx)
    for extra in ((False, True) if r == 2 else (False,)):
        y = mq.gemv_bitplanes(planes, r, m["alpha_d"], m["zero_d"], k, n, k, x_device(xb),
                              extra=extra)
        torch.cuda.synchronize()
        ref = _ref(xb, m["q"][rows], m["alpha"][rows], m["zero"][rows], k, r, extra)
        compare(y[:, rows], ref, f"bitplanes gemma {name} r{r} extra{int(extra)}")


def test_gemv_bitplanes_agrees_with_packed_planes():
    """The same product from the bit-planes and from the per-r packed plane."""
    n, k = 512, 3584
    m = quantized("gemma9b_mlp", n, k, 128, matrix=8)
    planes = mq.pack_bitplanes(m["q_d"])
    xb = inputs.activations_bf16("gemma9b_mlp", 4, k, matrix=8)
    for r in (2, 4, 8):
        note(f"bitplanes vs packed r={r}")
        yb = mq.gemv_bitplanes(planes, r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb))
        yp = mq.gemv(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb))
        torch.cuda.synchronize()
        compare(yb, yp.double().cpu().numpy(), f"bitplanes vs packed r{r}")


def test_gemv_bitplanes_error_enqueues_nothing():
    n, k = 16, 512
    m = quantized("tiny_linear", n, k, k)
    planes = mq.pack_bitplanes(m["q_d"])
    xb = x_device(inputs.activations_bf16("tiny_linear", 1, k))
    y = torch.full((1, n), 7.0, device=dev())
    with pytest.raises(mq.MQError):
        mq.gemv_bitplanes(planes, 9, m["alpha_d"], m["zero_d"], k, n, k, xb, out=y)
    with pytest.raises(mq.MQError):
        mq.gemv_bitplanes(planes, 4, m["alpha_d"], m["zero_d"], 64, n, k, xb, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
