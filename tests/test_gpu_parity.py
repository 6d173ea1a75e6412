"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Integer work (codes, slices, packed planes) must match bit for bit; products
must be within rel-L2 1e-3 and max-abs 2e-2 of the oracle.  Full-size
workloads are checked on sampled output rows the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import nested_int_matmul_amd as mq
import oracle
from nested_int_matmul_amd import inputs

from gpu_helpers import (compare, compare_linear, dev, guarded_f32, note, quantized, term_scale,
                         upload, x_device)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- quantize / pack

@pytest.mark.parametrize("shape,group,outliers", [
    ((256, 512), 512, 0.0),         # tiny linear, per-channel
    ((300, 3584), 3584, 1e-3),      # Gemma up-proj rows with outliers, ragged N
    ((64, 4096), 128, 0.0),         # group 128
])
def test_quantize_bit_exact(shape, group, outliers):
    n, k = shape
    note(f"quantize {shape} group {group}")
    w = inputs.gaussian_weights("tiny_linear", n, k, outlier_frac=outliers)
    w[3, :] = 0.125                     # a constant vector (alpha = 1 case)
    w[5, :] = 0.0
    w[5, 1::2] = 1e-38                  # range too small for a normal fp32 alpha
    w[6, :] = 0.0
    w[6, 7::64] = np.float32(255 * 2.0 ** -126)   # alpha exactly 2^-126: normal
    q, a, z = oracle.quantize_minmax(w, group)
    codes, alpha, zero = mq.quantize(torch.from_numpy(w).to(dev()), group)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), q)
    assert np.array_equal(alpha.cpu().numpy().view(np.uint32), a.view(np.uint32))
    assert np.array_equal(zero.cpu().numpy().view(np.uint32), z.view(np.uint32))


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
def test_pack_all_codes_bit_exact(r):
    note(f"pack all codes r={r}")
    q = np.tile(np.arange(256, dtype=np.uint8), (7, 4))          # [7, 1024], every code
    q[3] = np.random.default_rng(r).integers(0, 256, 1024, dtype=np.uint8)
    got = mq.pack(torch.from_numpy(q).to(dev()), r)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.pack_codes(q, r))
    # unpacking the GPU plane on the host gives back the oracle's indices
    t = oracle.unpack_indices(got.cpu().numpy(), r, 1024)
    assert np.array_equal(t, oracle.slice_index(q, r))


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
def test_pack_gemma_down_full_size(r):
    note(f"pack gemma down full r={r}")
    m = quantized("gemma9b_mlp", 3584, 14336, 14336, matrix=2, outlier_frac=1e-3)
    got = mq.pack(m["q_d"], r)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.pack_codes(m["q"], r))


# ---------------------------------------------------------------- GEMV (M <= 8)

@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_tiny_linear(r, M):
    note(f"gemv tiny r={r} M={M}")
    m = quantized("tiny_linear", 256, 512, 512)
    xb = inputs.activations_bf16("tiny_linear", M, 512)
    plane = mq.pack(m["q_d"], r)
    y = mq.gemv(plane, r, m["alpha_d"], m["zero_d"], 512, 256, 512, x_device(xb))
    torch.cuda.synchronize()
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], 512, r, f"tiny r{r} M{M}")


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_gemv_ragged(r, group, M):
    # N not a multiple of 16, K not a multiple of 256, several chunks at M = 8
    n, k = 301, (1152 if group == 128 else 576)
    g = k if group == "K" else 128
    note(f"gemv ragged r={r} group={g} M={M}")
    m = quantized("tiny_linear", n, k, g, matrix=7)
    xb = inputs.activations_bf16("tiny_linear", M, k, matrix=7)
    plane = mq.pack(m["q_d"], r)
    y, check = guarded_f32(M, n)
    mq.gemv(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"ragged r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"ragged r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [4, 2])
def test_gemv_long_k_chunked(r):
    # K = 16384 at M = 8 needs four activation chunks in LDS
    n, k, M = 48, 16384, 8
    note(f"gemv chunked r={r}")
    for g in (k, 128):
        m = quantized("tiny_linear", n, k, g, matrix=9)
        xb = inputs.activations_bf16("tiny_linear", M, k, matrix=9, heavy_channels=8)
        plane = mq.pack(m["q_d"], r)
        y = mq.gemv(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
        torch.cuda.synchronize()
        compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"chunked r{r} g{g}")


def _sample_rows(n, count=384, seed=0):
    rg = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, n - 1], rg.choice(n, count, replace=False)]))
    return rows


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
def test_gemv_gemma_mlp_full_size(r):
    """Decode GEMV at the Gemma-2-9B MLP shapes, in one grouped launch as the
    benchmark runs it; sampled rows against the oracle."""
    note(f"gemma mlp grouped r={r}")
    mats, probs, xs = [], [], []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        m = dict(quantized("gemma9b_mlp", n, k, k, matrix=i, outlier_frac=1e-3))
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        m["plane"] = mq.pack(m["q_d"], r)
        m["y"] = torch.empty((1, n), dtype=torch.float32, device=dev())
        m["xb"] = xb
        mats.append(m)
        probs.append({"packed": m["plane"], "alpha": m["alpha_d"], "zero": m["zero_d"],
                      "x": x_device(xb), "y": m["y"], "N": n, "K": k, "group": k})
    mq.gemv_grouped(probs, r, 1)
    torch.cuda.synchronize()
    for i, m in enumerate(mats):
        rows = _sample_rows(m["N"], seed=i)
        compare_linear(m["y"][:, rows], m["xb"], m["q"][rows], m["alpha"][rows], m["zero"][rows], m["K"], r, f"gemma mat{i} r{r}")


def test_gemv_mixed_precisions_one_launch():
    """mq_gemv_mixed: the three Gemma MLP matrices at r = 8, 4 and 2 (nine
    products) in one launch, as the benchmark runs them; sampled rows of
    every product against the oracle at its own r."""
    note("gemma mlp mixed r=8,4,2 one launch")
    mats, probs, rs = [], [], []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        m = dict(quantized("gemma9b_mlp", n, k, k, matrix=i, outlier_frac=1e-3))
        m["xb"] = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        mats.append(m)
    outs = []
    for r in (8, 4, 2):
        for i, m in enumerate(mats):
            y = torch.empty((1, m["N"]), dtype=torch.float32, device=dev())
            probs.append({"packed": mq.pack(m["q_d"], r), "alpha": m["alpha_d"],
                          "zero": m["zero_d"], "x": x_device(m["xb"]), "y": y, "N": m["N"],
                          "K": m["K"], "group": m["K"]})
            rs.append(r)
            outs.append((i, r, y))
    mq.gemv_grouped(probs, rs, 1)
    torch.cuda.synchronize()
    for i, r, y in outs:
        m = mats[i]
        rows = _sample_rows(m["N"], 128, seed=10 * i + r)
        compare_linear(y[:, rows], m["xb"], m["q"][rows], m["alpha"][rows], m["zero"][rows], m["K"], r, f"mixed mat{i} r{r}")


@pytest.mark.parametrize("M", [1, 5])
def test_gemv_mixed_granularities(M):
    """Per-channel and group-128 problems at different r in one call."""
    note(f"gemv mixed granularities M={M}")
    cases = [(200, 768, "K", 2), (136, 1024, 128, 8), (72, 512, 128, 4), (300, 640, "K", 4),
             (96, 1024, 128, 6), (160, 576, "K", 3), (64, 1280, 128, 3), (40, 448, "K", 6)]
    probs, rs, refs = [], [], []
    for j, (n, k, g, r) in enumerate(cases):
        gg = k if g == "K" else 128
        m = quantized("tiny_linear", n, k, gg, matrix=20 + j)
        xb = inputs.activations_bf16("tiny_linear", M, k, matrix=20 + j)
        y = torch.empty((M, n), dtype=torch.float32, device=dev())
        probs.append({"packed": mq.pack(m["q_d"], r), "alpha": m["alpha_d"], "zero": m["zero_d"],
                      "x": x_device(xb), "y": y, "N": n, "K": k, "group": gg})
        rs.append(r)
        refs.append((y, (xb, m["q"], m["alpha"], m["zero"], gg, r), f"case{j} r{r}"))
    mq.gemv_grouped(probs, rs, M)
    torch.cuda.synchronize()
    for y, args, what in refs:
        compare_linear(y, *args, what)


@pytest.mark.parametrize("r", [6, 3])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [65, 130, 256, 300])
def test_gemm_split_precision_large_batch(r, group, M):
    """M > 64 at r = 3 and 6 on the prefill kernel: partial 256-row tiles,
    ragged N, 24 K iterations."""
    n, k = 300, 1536
    g = k if group == "K" else 128
    note(f"gemm split precision large r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=7)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=7, heavy_channels=8)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    torch.cuda.synchronize()
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [6, 3])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [9, 16, 33, 64])
def test_gemm_split_precision_small_batch(r, group, M):
    """9 <= M <= 64 at r = 3 and 6 (high and low planes) on the small-batch
    kernel: ragged N, two K slices and a ragged last slice at K = 1536."""
    n, k = 300, 1536
    g = k if group == "K" else 128
    note(f"gemm split precision r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=6)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=6, heavy_channels=8)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    torch.cuda.synchronize()
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [6, 3])
def test_gemm_split_precision_mistral_full_size(r):
    """Mistral 14336 x 4096 and 4096 x 14336 at M = 16, group 128, sampled rows."""
    for (n, k) in inputs.MISTRAL_SMALL_SHAPES:
        note(f"gemm split precision mistral r={r} {n}x{k}")
        m = quantized("mistral_small", n, k, 128, matrix=n // 4096)
        xb = inputs.activations_bf16("mistral_small", 16, k, heavy_channels=8)
        y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(r).choice(n, 150, replace=False)]))
        compare_linear(y[:, rows], xb, m["q"][rows], m["alpha"][rows], m["zero"][rows], 128, r,
                       f"gemm mistral r{r} {n}x{k}")


def test_gemv_deterministic():
    note("gemv determinism")
    m = quantized("tiny_linear", 512, 4096, 4096, matrix=3)
    xb = inputs.activations_bf16("tiny_linear", 2, 4096, matrix=3)
    plane = mq.pack(m["q_d"], 2)
    y1 = mq.gemv(plane, 2, m["alpha_d"], m["zero_d"], 4096, 512, 4096, x_device(xb))
    y2 = mq.gemv(plane, 2, m["alpha_d"], m["zero_d"], 4096, 512, 4096, x_device(xb))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("r", [2, 4, 8, 6])
def test_gemv_grouped_repeated_launches_identical(r):
    """Group-128 scales read per-group activation sums that other threads of
    the workgroup write to LDS.  40 launches, single and grouped, must be
    bit-identical to the first (the kernel's order is fixed), and the first
    must match the oracle.  Regression test for a missing barrier between
    those writes and the reads."""
    note(f"gemv grouped repeated r={r}")
    n, k = 520, 1536
    m = quantized("mistral_small", n, k, 128, matrix=9)
    xb = inputs.activations_bf16("mistral_small", 3, k, matrix=9, heavy_channels=8)
    x = x_device(xb)
    plane = mq.pack(m["q_d"], r)
    y0 = mq.gemv(plane, r, m["alpha_d"], m["zero_d"], 128, n, k, x)
    torch.cuda.synchronize()
    compare_linear(y0, xb, m["q"], m["alpha"], m["zero"], 128, r, f"grouped r{r}")
    lin = dict(packed=plane, alpha=m["alpha_d"], zero=m["zero_d"], N=n, K=k, group=128, x=x)
    for i in range(40):
        y = mq.gemv(plane, r, m["alpha_d"], m["zero_d"], 128, n, k, x)
        y2, y3 = torch.empty_like(y), torch.empty_like(y)
        mq.gemv_grouped([dict(lin, y=y2), dict(lin, y=y3)], r, 3)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"launch {i} differs"
        assert torch.equal(y2, y0) and torch.equal(y3, y0), f"grouped launch {i} differs"


def test_error_enqueues_nothing():
    note("error path")
    m = quantized("tiny_linear", 64, 512, 512)
    plane = mq.pack(m["q_d"], 4)
    xb = x_device(inputs.activations_bf16("tiny_linear", 1, 512))
    y = torch.full((1, 64), 7.0, device=dev())
    with pytest.raises(mq.MQError):
        mq.gemv(plane, 5, m["alpha_d"], m["zero_d"], 512, 64, 512, xb, out=y)
    with pytest.raises(mq.MQError):
        mq.gemv(plane, 4, m["alpha_d"], m["zero_d"], 100, 64, 512, xb, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------- Extra precision

@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
def test_overflow_lists_bit_exact(r):
    note(f"overflow lists r={r}")
    m = quantized("gemma9b_mlp", 300, 1536, 1536, matrix=4, outlier_frac=1e-2)
    q = m["q"].copy()
    q[7] = 255                      # a full row at the extra level
    q[8] = 0                        # an empty row
    q[9, ::3] = 255 - (np.arange(512) % 4)   # codes around the threshold
    row_ptr, col_idx = mq.overflow_lists(torch.from_numpy(q).to(dev()), r)
    torch.cuda.synchronize()
    want_ptr, want_idx = oracle.overflow_lists(q, r)
    assert row_ptr.cpu().numpy().tolist() == want_ptr.tolist()
    assert col_idx.cpu().numpy().view(np.uint16).tolist() == want_idx.tolist()


@pytest.mark.parametrize("r", [6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_extra_precision_product(r, group, M):
    """plane product at r + the sparse addition = the unclamped (errata Eq. 8)
    product of the oracle."""
    n, k = 260, 1024
    g = k if group == "K" else 128
    note(f"extra precision r={r} g={g} M={M}")
    m = quantized("gemma9b_mlp", n, k, g, matrix=6, outlier_frac=2e-2)
    assert np.any(oracle.slice_value_noclamp(m["q"], r) == 256)
    xb = inputs.activations_bf16("gemma9b_mlp", M, k, matrix=6)
    plane = mq.pack(m["q_d"], r)
    y = mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    row_ptr, col_idx = mq.overflow_lists(m["q_d"], r)
    mq.overflow_apply(row_ptr, col_idx, r, m["alpha_d"], g, n, k, x_device(xb), y)
    torch.cuda.synchronize()
    compare(y, oracle.linear_extra_precision(xb, m["q"], m["alpha"], m["zero"], g, r),
            f"extra r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [2, 4])
def test_extra_precision_grouped_gemma_mlp(r):
    """The three Gemma-2-9B MLP matrices (per-channel, 0.1% x10 outliers) at
    full size: plane products, then the three sparse additions in one
    launch (mq_overflow_apply_grouped); sampled rows against the unclamped
    oracle product."""
    note(f"extra precision grouped gemma mlp r={r}")
    mats, probs = [], []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        m = quantized("gemma9b_mlp", n, k, k, matrix=i, outlier_frac=1e-3)
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        y = mq.gemv(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], k, n, k, x_device(xb))
        row_ptr, col_idx = mq.overflow_lists(m["q_d"], r)
        probs.append(dict(row_ptr=row_ptr, col_idx=col_idx, alpha=m["alpha_d"], x=x_device(xb),
                          y=y, N=n, K=k, group=k))
        mats.append((m, xb, y))
    mq.overflow_apply_grouped(probs, r, 1)
    torch.cuda.synchronize()
    for i, (m, xb, y) in enumerate(mats):
        rows = _sample_rows(m["N"], 200, seed=40 + i)
        ref = oracle.linear_extra_precision(xb, m["q"][rows], m["alpha"][rows], m["zero"][rows],
                                            m["K"], r)
        compare(y[:, rows], ref, f"extra grouped mat{i} r{r}")


@pytest.mark.parametrize("group", ["K", 128])
def test_extra_precision_maximum_k(group):
    """K = 65536, the largest the library serves: column indices up to 65535
    fill the 16 bits of the lists; lists bit-exact and the product with the
    sparse addition against the unclamped oracle product, r = 2, M = 3."""
    n, k, r, M = 24, 65536, 2, 3
    g = k if group == "K" else 128
    note(f"extra precision max K g={g}")
    m = quantized("gemma9b_mlp", n, k, g, matrix=33, outlier_frac=2e-2)
    q = m["q"]
    assert q[:, -4096:].max() >= 256 - 32  # entries listed near the end of the rows
    row_ptr, col_idx = mq.overflow_lists(m["q_d"], r)
    torch.cuda.synchronize()
    want_ptr, want_idx = oracle.overflow_lists(q, r)
    assert row_ptr.cpu().numpy().tolist() == want_ptr.tolist()
    assert col_idx.cpu().numpy().view(np.uint16).tolist() == want_idx.tolist()
    assert want_idx.max() > 65000
    xb = inputs.activations_bf16("gemma9b_mlp", M, k, matrix=33)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    mq.overflow_apply(row_ptr, col_idx, r, m["alpha_d"], g, n, k, x_device(xb), y)
    torch.cuda.synchronize()
    compare(y, oracle.linear_extra_precision(xb, q, m["alpha"], m["zero"], g, r),
            f"extra max K g{g}")


def test_extra_precision_gemma_up_full_size():
    note("extra precision gemma up r=2 full size")
    n, k = inputs.GEMMA9B_MLP["up"]
    m = quantized("gemma9b_mlp", n, k, k, matrix=0, outlier_frac=1e-3)
    xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=0)
    plane = mq.pack(m["q_d"], 2)
    y = mq.gemv(plane, 2, m["alpha_d"], m["zero_d"], k, n, k, x_device(xb))
    row_ptr, col_idx = mq.overflow_lists(m["q_d"], 2)
    mq.overflow_apply(row_ptr, col_idx, 2, m["alpha_d"], k, n, k, x_device(xb), y)
    torch.cuda.synchronize()
    want_ptr, _ = oracle.overflow_lists(m["q"], 2)
    assert row_ptr.cpu().numpy().tolist() == want_ptr.tolist()
    rows = _sample_rows(n, 256, seed=5)
    ref = oracle.linear_extra_precision(xb, m["q"][rows], m["alpha"][rows], m["zero"][rows], k, 2)
    compare(y[:, rows], ref, "extra gemma up r2")


# ---------------------------------------------------------------- GEMM (M > 8)

@pytest.mark.parametrize("r", [8, 4, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [9, 16, 64, 130, 300])
def test_gemm_small(r, group, M):
    n, k = 200, (640 if group == "K" else 768)
    g = k if group == "K" else 128
    note(f"gemm small r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=5)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=5, heavy_channels=8)
    plane = mq.pack(m["q_d"], r)
    y, check = guarded_f32(M, n)
    mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm small r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [12, 24, 40])
def test_gemm_small_batch_every_instance(r, group, M):
    """The small-batch kernel at every precision, both scale granularities
    and each number of 16-row activation blocks (1, 2, 4), with a ragged
    last panel and three K slices whose last is short: 128 codes at group
    128 (at r = 2 a step spans two groups, the second past the slice) and 64
    codes per-channel (a partial step at r = 2, 3, 4 and 6).  N = 300 takes
    the 16-byte output stores, N = 302 the element stores."""
    n = 300 if group == 128 else 302
    k = 2176 if group == 128 else 2112
    g = k if group == "K" else 128
    note(f"gemm small-batch every instance r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=7)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=7, heavy_channels=8)
    plane = mq.pack(m["q_d"], r)
    y, check = guarded_f32(M, n)
    mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm small-batch r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm every instance r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [9, 16])
@pytest.mark.parametrize("k", [2048, 4096])
def test_gemm_small_batch_whole_k(r, group, M, k):
    """M <= 16 with many output rows (N >= 12288) and K <= 4096: one
    workgroup takes a 64-row panel over all of K, its two halves of K summed
    in LDS (no partial slices, no second launch).  N = 12300 leaves a ragged
    last panel; K = 4096 fills the staged activations' LDS."""
    if k == 4096 and not (r in (4, 2) and M == 16):
        pytest.skip("K = 4096 at r = 4 and 2, M = 16 only (the oracle's cost)")
    n = 12300
    g = k if group == "K" else 128
    note(f"gemm small-batch whole K r={r} g={g} M={M} K={k}")
    m = quantized("mistral_small", n, k, g, matrix=8)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=8, heavy_channels=8)
    plane = mq.pack(m["q_d"], r)
    assert mq.gemm_workspace_bytes(M, n, k, g) == 0  # no partial slices on this path
    y, check = guarded_f32(M, n)
    mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm whole K r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm whole K r{r} g{g} M{M} K{k}")


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [9, 16])
def test_gemm_small_batch_wide_panels_split_k(r, group, M):
    """M <= 16, K longer than one 4096-code slice: 64-row panels over three
    slices (4096, 4096, 512 codes), each slice's halves summed in LDS, the
    slices by reduce_slices; 65 panels (N = 4100, ragged) x 3 slices."""
    n, k = 4100, 8704
    g = k if group == "K" else 128
    note(f"gemm small-batch wide panels split K r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=9)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=9, heavy_channels=8)
    plane = mq.pack(m["q_d"], r)
    assert mq.gemm_workspace_bytes(M, n, k, g) == 3 * M * n * 4  # three partial slices
    y, check = guarded_f32(M, n)
    mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm wide split r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm wide split r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [8, 4, 2])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [65, 100, 127, 128, 255])
def test_gemm_mid_batch_split_k(r, group, M):
    """M > 64 with few output tiles and a long K: K (66 iterations of 64) is
    cut into 7 slices of 10, the last one short, summed in slice order;
    128-row tiles up to M = 128, 256-row tiles above."""
    n, k = 300, 4224
    g = k if group == "K" else 128
    assert mq.gemm_workspace_bytes(M, n, k, g) > 0
    note(f"gemm mid batch split-K r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=8)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=8, heavy_channels=8)
    y, check = guarded_f32(M, n)
    mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm mid r{r} g{g} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"gemm r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [4, 8, 3])
@pytest.mark.parametrize("M", [9, 33, 65, 131])
def test_gemm_split_k_unaligned_slices(r, M):
    """K splits whose partial slices are M * N = odd floats long (N = 301),
    so slice starts are not 16-byte aligned: the panel kernel (M = 9, 33)
    and the M >= 65 kernel with 128-row (65) and 256-row (131) tiles, group
    128, K = 4224."""
    n, k = 301, 4224
    assert mq.gemm_workspace_bytes(M, n, k, 128) > 0
    note(f"gemm split-K unaligned slices r={r} M={M}")
    m = quantized("mistral_small", n, k, 128, matrix=10)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=10, heavy_channels=8)
    y, check = guarded_f32(M, n)
    mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"gemm unaligned r{r} M{M}")
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], 128, r, f"gemm r{r} M{M}")


@pytest.mark.parametrize("r", [8, 6, 4])
def test_gemm_prefill_split_k_odd_iterations(r):
    """Per-channel K = 4160: 65 iterations of 64 on the prefill kernel, split
    into 7 slices of 10 (whole groups) whose last one has 5 and ends
    mid-pair; M = 256 rows (one tile row), N = 300 (two tiles, ragged)."""
    M, n, k = 256, 300, 4160
    assert mq.gemm_workspace_bytes(M, n, k, k) == 7 * M * n * 4
    note(f"gemm prefill split-K odd r={r}")
    m = quantized("mistral_small", n, k, k, matrix=9)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=9, heavy_channels=8)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], k, n, k, x_device(xb))
    torch.cuda.synchronize()
    compare_linear(y, xb, m["q"], m["alpha"], m["zero"], k, r, f"gemm odd r{r}")


@pytest.mark.parametrize("r", [4, 6])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [9, 40])
def test_gemm_small_batch_ragged_last_panel(r, group, M):
    """N = 14000, K = 4096 on the small-batch kernel: 55 panels of 256 rows
    (the last one 176 rows) x 4 K slices; sampled rows include the last 230."""
    n, k = 14000, 4096
    g = k if group == "K" else 128
    note(f"gemm small batch ragged last panel r={r} g={g} M={M}")
    m = quantized("mistral_small", n, k, g, matrix=11)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=11, heavy_channels=8)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([_sample_rows(n, 200, seed=M), np.arange(n - 230, n)]))
    compare_linear(y[:, rows], xb, m["q"][rows], m["alpha"][rows], m["zero"][rows], g, r, f"ragged panel r{r} g{g} M{M}")


@pytest.mark.parametrize("r", [4, 2])
@pytest.mark.parametrize("M", [16, 64, 96, 200])
@pytest.mark.parametrize("shape", inputs.MISTRAL_SMALL_SHAPES)
def test_gemm_mistral_small_full_size(r, M, shape):
    n, k = shape
    note(f"gemm mistral small r={r} M={M} {shape}")
    m = quantized("mistral_small", n, k, 128, matrix=shape[0] // 4096)
    xb = inputs.activations_bf16("mistral_small", M, k, heavy_channels=8)
    plane = mq.pack(m["q_d"], r)
    y = mq.gemm(plane, r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb))
    torch.cuda.synchronize()
    rows = _sample_rows(n, 256)
    compare_linear(y[:, rows], xb, m["q"][rows], m["alpha"][rows], m["zero"][rows], 128, r, f"mistral small r{r} M{M} {shape}")


@pytest.mark.parametrize("r", [4, 2, 8, 6, 3])
def test_gemm_prefill_full_size(r):
    M, k, n = inputs.PREFILL_SHAPE
    note(f"gemm prefill r={r}")
    m = quantized("prefill", n, k, 128)
    xb = inputs.activations_bf16("prefill", M, k)
    plane = mq.pack(m["q_d"], r)
    y = mq.gemm(plane, r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb))
    torch.cuda.synchronize()
    cols = _sample_rows(n, 128)
    compare_linear(y[:, cols], xb, m["q"][cols], m["alpha"][cols], m["zero"][cols], 128, r, f"prefill r{r}")


@pytest.mark.parametrize("r", [4, 2, 8, 6, 3])
@pytest.mark.parametrize("group", [128, "K"])
def test_gemm_prefill_second_round_ragged(r, group):
    """More 256 x 256 tiles than one round of CUs (2048 x 8676: 272 tiles,
    the last column of tiles ragged).  Every column from 8128 on (the tiles
    of the second round and the ragged end) and a sample before it, all
    2048 rows, against the oracle; guard elements after the output."""
    M, n, k = 2048, 8676, 256
    g = k if group == "K" else 128
    note(f"gemm prefill second round ragged r={r} g={g}")
    m = quantized("prefill", n, k, g, matrix=2)
    xb = inputs.activations_bf16("prefill", M, k, matrix=2)
    y, check = guarded_f32(M, n)
    mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"second round ragged r{r} g{g}")
    cols = np.unique(np.concatenate([_sample_rows(8128, 64, seed=r), np.arange(8128, n)]))
    compare_linear(y[:, cols], xb, m["q"][cols], m["alpha"][cols], m["zero"][cols], g, r,
                   f"second round ragged r{r} g{g}")


@pytest.mark.parametrize("r", [4, 2, 8, 6, 3])
@pytest.mark.parametrize("M,group", [(2048, 128), (512, 128), (512, "K")])
def test_gemm_prefill_down_projection_split_k(r, M, group):
    """The 4096-wide down projection (K = 14336) has 128 (M = 2048) or 32
    (M = 512) tiles of 256 x 256, so K is split over workgroups (2 or 8
    slices) and the slices are summed in order; sampled columns."""
    n, k = 4096, 14336
    g = k if group == "K" else 128
    assert mq.gemm_workspace_bytes(M, n, k, g) > 0
    note(f"gemm prefill down projection r={r} M={M} g={g}")
    m = quantized("prefill", n, k, g, matrix=1)
    xb = inputs.activations_bf16("prefill", M, k, matrix=1)
    y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
    torch.cuda.synchronize()
    cols = _sample_rows(n, 128, seed=r)
    compare_linear(y[:, cols], xb, m["q"][cols], m["alpha"][cols], m["zero"][cols], g, r, f"prefill down r{r} M{M} g{g}")


# ---------------------------------------------------------------- Mix'n'Match

def _small_stack(rs, H=256, Hkv=64, F=512, group_kind="K"):
    shapes = {"q": (H, H), "k": (Hkv, H), "v": (Hkv, H), "o": (H, H),
              "up": (F, H), "gate": (F, H), "down": (H, F)}
    host, devl = [], []
    for li, r in enumerate(rs):
        hl, dl = {"r": r}, {"r": r}
        for mi, name in enumerate(oracle.LAYER_LINEARS):
            n, k = shapes[name]
            if group_kind == "split":  # gate per group of 128, the rest per channel
                g = 128 if name == "gate" else k
            else:
                g = k if group_kind == "K" else 128
            m = quantized("mistral_stack", n, k, g, layer=li, matrix=mi)
            hl[name] = {"q": m["q"], "alpha": m["alpha"], "zero": m["zero"], "group": g}
            dl[name] = {"packed": mq.pack(m["q_d"], r), "alpha": m["alpha_d"],
                        "zero": m["zero_d"], "N": n, "K": k, "group": g}
        host.append(hl)
        devl.append(dl)
    return host, devl


def _bf16_bits_of_f32(t):
    return t.float().to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rs", [(8, 4, 2, 4, 8), (6, 3, 8)])
@pytest.mark.parametrize("group_kind", ["K", 128, "split"])
@pytest.mark.parametrize("M", [1, 2])
def test_mixnmatch_small_stack(group_kind, M, rs):
    rs = list(rs)
    note(f"mixnmatch small group={group_kind} M={M} r={rs}")
    host, devl = _small_stack(rs, group_kind=group_kind)
    arr = mq.make_layers(devl)
    H = 256
    xb = inputs.activations_bf16("mistral_stack", M, H)
    h0 = oracle.float_from_bf16_bits(xb)
    ws = torch.empty(mq.mixnmatch_workspace_bytes(arr, M), dtype=torch.uint8, device=dev())
    off = mq.mixnmatch_workspace_offsets(mq.make_layers(devl[0:1]), M)

    # teacher-forced: one layer at a time from the GPU's own residual stream
    h = torch.from_numpy(h0.astype(np.float32)).to(dev())
    for li in range(len(rs)):
        h_in = h.clone()
        one = mq.make_layers(devl[li:li + 1])
        mq.mixnmatch_forward_inplace(one, h, ws)
        torch.cuda.synchronize()
        L = host[li]
        a_bits = ws[off[0]:off[0] + M * H * 2].view(torch.int16).cpu().numpy().view(np.uint16)
        a_bits = a_bits.reshape(M, H)
        # the GPU's normalized input matches the definition on its own h
        hin = h_in.double().cpu().numpy()
        want_a = oracle.bf16_bits_from_float(oracle.rms_normalize(hin))
        mism = np.count_nonzero(a_bits != want_a)
        assert mism <= max(2, a_bits.size // 200), f"layer {li}: {mism} bf16 rounding differences"

        def fetch(i, n):
            return ws[off[i]:off[i] + M * n * 4].view(torch.float32).reshape(M, n)

        outs = {"q": fetch(1, H), "k": fetch(2, 64), "v": fetch(3, 64), "up": fetch(4, 512),
                "gate": fetch(5, 512)}
        for name, y in outs.items():
            p = L[name]
            compare_linear(y, a_bits, p["q"], p["alpha"], p["zero"], p["group"], L["r"], f"layer {li} {name}")
        qb = _bf16_bits_of_f32(outs["q"])
        ugb = _bf16_bits_of_f32(outs["up"] * outs["gate"])

        def fetch_bf16(i, n):
            t = ws[off[i]:off[i] + M * n * 2].view(torch.int16).cpu().numpy().view(np.uint16)
            return t.reshape(M, n)

        # the bf16 copies the first launch writes are the nearest-even
        # roundings of its own fp32 outputs (bit-exact)
        np.testing.assert_array_equal(fetch_bf16(8, H), qb, err_msg=f"layer {li} bf16(q)")
        if group_kind != "split":  # up and gate paired
            np.testing.assert_array_equal(fetch_bf16(9, 512), ugb,
                                          err_msg=f"layer {li} bf16(u*g)")
        o = fetch(6, H)
        d = fetch(7, H)
        compare_linear(o, qb, L["o"]["q"], L["o"]["alpha"], L["o"]["zero"],
                                 L["o"]["group"], L["r"], f"layer {li} o")
        compare_linear(d, ugb, L["down"]["q"], L["down"]["alpha"], L["down"]["zero"],
                                 L["down"]["group"], L["r"], f"layer {li} down")
        h_ref = hin + o.double().cpu().numpy() + d.double().cpu().numpy()
        compare(h, h_ref, f"layer {li} residual")

    # end to end: all layers in one call from the bf16 input, against the
    # float64 stack; the in-place form from h = x gives the same bits
    h_out, check = guarded_f32(M, H)
    mq.mixnmatch_forward(arr, x_device(xb), ws, out=h_out)
    torch.cuda.synchronize()
    check("stack h_out")
    compare(h_out, oracle.mixnmatch_forward(host, xb), "stack end-to-end", reg=1e-3)
    h = torch.from_numpy(h0.astype(np.float32)).to(dev())
    mq.mixnmatch_forward_inplace(arr, h, ws)
    torch.cuda.synchronize()
    assert torch.equal(h, h_out)


@pytest.mark.parametrize("M", [1, 2])
def test_mixnmatch_wide_rows(M):
    """H = 4160 (1040 four-float vectors per row): the norm's first 16
    threads hold two vectors and the rest one, its four-vector path partly
    filled.  The plain, the loading and the residual norm are each checked:
    a of a one-layer in-place call against the definition, then two layers
    end to end from the bf16 input against the float64 stack."""
    H, rs = 4160, [8, 2]
    note(f"mixnmatch wide rows H={H} M={M}")
    host, devl = _small_stack(rs, H=H, Hkv=64, F=128)
    arr = mq.make_layers(devl)
    xb = inputs.activations_bf16("mistral_stack", M, H)
    h0 = oracle.float_from_bf16_bits(xb)
    ws = torch.empty(mq.mixnmatch_workspace_bytes(arr, M), dtype=torch.uint8, device=dev())
    off = mq.mixnmatch_workspace_offsets(mq.make_layers(devl[0:1]), M)
    h = torch.from_numpy(h0.astype(np.float32)).to(dev())
    mq.mixnmatch_forward_inplace(mq.make_layers(devl[0:1]), h, ws)
    torch.cuda.synchronize()
    a_bits = ws[off[0]:off[0] + M * H * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    want_a = oracle.bf16_bits_from_float(oracle.rms_normalize(h0))
    mism = np.count_nonzero(a_bits.reshape(M, H) != want_a)
    assert mism <= max(2, M * H // 200), f"{mism} bf16 rounding differences in a"
    h_out, check = guarded_f32(M, H)
    mq.mixnmatch_forward(arr, x_device(xb), ws, out=h_out)
    torch.cuda.synchronize()
    check("wide stack h_out")
    compare(h_out, oracle.mixnmatch_forward(host, xb), "wide stack end-to-end", reg=1e-3)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("r", [8, 4, 2])
@pytest.mark.parametrize("group", ["K", 128])
def test_gemv_maximum_k(r, group):
    """K at the library's maximum (65536), ragged N, several activation chunks."""
    n, k = 17, 65536
    g = k if group == "K" else 128
    note(f"gemv max K r={r} g={g}")
    m = quantized("tiny_linear", n, k, g, matrix=30)
    for M in (1, 3):
        xb = inputs.activations_bf16("tiny_linear", M, k, matrix=30)
        y = mq.gemv(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
        torch.cuda.synchronize()
        compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"max K r{r} M{M}")


@pytest.mark.parametrize("M", [1, 8, 16, 64, 65, 255, 256, 300])
def test_single_row_and_minimum_k(M):
    """N = 1 and the smallest K (64 per-channel, 128 grouped), across the M
    ranges that route to the decode, small-batch, tiled and prefill kernels."""
    note(f"degenerate shapes M={M}")
    for (n, k, g) in ((1, 64, 64), (1, 128, 128), (3, 64, 64), (33, 128, 128)):
        m = quantized("tiny_linear", n, k, g, matrix=31)
        xb = inputs.activations_bf16("tiny_linear", M, k, matrix=31)
        for r in (8, 2):
            y = mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
            torch.cuda.synchronize()
            compare_linear(y, xb, m["q"], m["alpha"], m["zero"], g, r, f"N{n} K{k} g{g} r{r} M{M}")


def test_constant_rows_quantize_and_product():
    """Rows (and groups) with a single value: alpha = 1, z = -min, codes 0
    (the reading for a zero range); quantize bit-exact, products exact."""
    note("constant rows")
    n, k = 40, 512
    w = inputs.gaussian_weights("tiny_linear", n, k, matrix=32)
    w[3] = 0.25
    w[7] = -1.5
    w[11, 128:256] = 0.0   # one constant group of 128
    for g in (k, 128):
        q, a, z = oracle.quantize_minmax(w, g)
        codes, alpha, zero = mq.quantize(torch.from_numpy(w).to(dev()), g)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), q)
        assert np.array_equal(alpha.cpu().numpy().view(np.uint32), a.view(np.uint32))
        assert np.array_equal(zero.cpu().numpy().view(np.uint32), z.view(np.uint32))
        xb = inputs.activations_bf16("tiny_linear", 2, k, matrix=32)
        for r in (8, 4, 2):
            y = mq.gemv(mq.pack(codes, r), r, alpha, zero, g, n, k, x_device(xb))
            torch.cuda.synchronize()
            compare_linear(y, xb, q, a, z, g, r, f"constant rows g{g} r{r}")


def _constant_group_weights(n, k, seed):
    """Gaussian weights with constant vectors where the GEMM kernels change
    groups: a constant row, a zero row, a constant first, middle and last
    group of 128, and a row whose even groups are constant (the scale then
    alternates between 1 and about 5e-4 from group to group)."""
    w = inputs.gaussian_weights("mistral_small", n, k, matrix=seed)
    w[3] = 0.25
    w[5] = 0.0
    w[7, 128:256] = 0.0
    w[11, :128] = -1.5
    w[13, k - 128:] = 0.5
    for g0 in range(0, k, 256):
        w[17, g0:g0 + 128] = 0.1
    w[n - 1, 1024:1152] = -0.03125
    return w


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("M", [16, 64, 300, 2048])
def test_gemm_constant_groups(r, M):
    """Constant rows and groups (alpha = 1, z = -min) next to Gaussian groups
    (alpha about 5e-4) through mq_gemm at group 128: the panel kernel's group
    restarts (M = 16, 64; K split in 4), and the prefill kernel's rescale of
    its accumulators by alpha_g / alpha_{g+1} (M = 300, 2048; K split over
    workgroups).  Every output element against the oracle."""
    n, k = 300, 4096
    note(f"gemm constant groups r={r} M={M}")
    w = _constant_group_weights(n, k, 40)
    q, a, z = oracle.quantize_minmax(w, 128)
    assert np.sum(a == 1.0) == 2 * 32 + 16 + 4
    m = upload(q, a, z, 128)
    xb = inputs.activations_bf16("mistral_small", M, k, matrix=40, heavy_channels=8)
    y, check = guarded_f32(M, n)
    mq.gemm(mq.pack(m["q_d"], r), r, m["alpha_d"], m["zero_d"], 128, n, k, x_device(xb), out=y)
    torch.cuda.synchronize()
    check(f"constant groups r{r} M{M}")
    compare_linear(y, xb, q, a, z, 128, r, f"constant groups r{r} M{M}")
    # the constant rows alone (a whole-matrix norm would hide one of them)
    rows = [3, 5, 7, 11, 13, 17, n - 1]
    compare_linear(y[:, rows], xb, q[rows], a[rows], z[rows], 128, r, f"constant rows r{r} M{M}")


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", ["K", 128])
def test_one_hot_rows_read_back_every_weight(r, group):
    """Activation rows that are one-hot (x[m, k_m] = 1) make each output
    element a single dequantized weight: y[m, n] = (S(q[n, k_m], r) - z) *
    alpha.  Every weight of an 80 x 1536 matrix is read back this way through
    every route of mq_gemm (the decode kernel at M = 1 and 8 on a sample of
    columns, the small-batch kernel at M = 16 and 64, the tiled kernel at
    M = 128, 300 and 2048, K splits included), each within a few fp32
    roundings of its own size, far below one slice level alpha * 2^(8-r)."""
    n, k = 80, 1536
    g = k if group == "K" else 128
    note(f"one-hot read-back r={r} g={g}")
    m = quantized("mistral_small", n, k, g, matrix=60, outlier_frac=1e-2)
    plane = mq.pack(m["q_d"], r)
    w = oracle.dequant(m["q"], m["alpha"], m["zero"], g, r)
    s = oracle.slice_value(m["q"], r).astype(np.float64)
    abar = np.repeat(m["alpha"].astype(np.float64), g, axis=1)
    zbar = np.repeat(m["zero"].astype(np.float64), g, axis=1)
    tol = 2.0 ** -18 * abar * (np.abs(s - zbar) + 512.0)
    one = np.uint16(0x3F80)  # bf16 1.0
    rg = np.random.default_rng(r)
    sampled = np.unique(np.concatenate([np.arange(128), np.arange(k - 128, k),
                                        rg.choice(k, 128, replace=False)]))
    for M in (1, 8, 16, 64, 128, 300, 2048):
        cols = sampled if M <= 8 else np.arange(k)
        got = np.zeros((n, cols.size))
        outs = []
        for start in range(0, cols.size, M):
            chunk = cols[start:start + M]
            xb = np.zeros((M, k), dtype=np.uint16)
            xb[np.arange(chunk.size), chunk] = one
            y = mq.gemm(plane, r, m["alpha_d"], m["zero_d"], g, n, k, x_device(xb))
            outs.append((start, chunk.size, y))
        torch.cuda.synchronize()
        for start, c, y in outs:
            got[:, start:start + c] = y[:c].double().cpu().numpy().T
        err = np.abs(got - w[:, cols])
        ratio = err / tol[:, cols]
        worst = np.unravel_index(np.argmax(ratio), ratio.shape)
        note(f"  M={M}: max error / tolerance {ratio.max():.3e} at row {worst[0]} "
             f"col {cols[worst[1]]}")
        assert ratio.max() <= 1.0, f"r{r} g{g} M{M}: weight {worst} read back off by {err[worst]}"
