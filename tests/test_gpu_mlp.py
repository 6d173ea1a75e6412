"""GPU parity of the decode MLP block (mq_mlp_decode): up and gate in one
launch writing bf16(u * act(g)), then down, against the float64 oracle.

Teacher-forced checks use the GPU's own intermediates (u, g, the bf16 product)
so that a rounding decision taken in fp32 on the GPU does not propagate; the
end-to-end result is also compared with the oracle's block.
"""

import numpy as np
import pytest
import torch

import nested_int_matmul_amd as mq
import oracle
from nested_int_matmul_amd import inputs

from gpu_helpers import compare, compare_linear, dev, note, quantized, x_device

pytestmark = pytest.mark.gpu


def _mats(H, F, group, r, workload="gemma9b_mlp", outlier_frac=0.0):
    host, devm = {}, {}
    for i, (name, (n, k)) in enumerate((("up", (F, H)), ("gate", (F, H)), ("down", (H, F)))):
        g = k if group == "K" else 128
        m = quantized(workload, n, k, g, matrix=10 + i, outlier_frac=outlier_frac)
        host[name] = {"q": m["q"], "alpha": m["alpha"], "zero": m["zero"], "group": g}
        devm[name] = {"packed": mq.pack(m["q_d"], r), "alpha": m["alpha_d"], "zero": m["zero_d"],
                      "N": n, "K": k, "group": g}
    return host, devm


def _split_workspace(ws, M, F):
    fb = -(-(M * F * 4) // 256) * 256
    u = ws[0:M * F * 4].view(torch.float32).reshape(M, F)
    g = ws[fb:fb + M * F * 4].view(torch.float32).reshape(M, F)
    a = ws[2 * fb:2 * fb + M * F * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(M, F)
    return u, g, a


def _check_product_bits(a_bits, u, g, act, what):
    """The bf16 product the GPU wrote is the nearest-even rounding of its own
    fp32 u * act(g).  With the identity the decision is taken in the same
    precision on both sides (fp32 product, then bf16), so it is bit-exact.
    With SiLU / GELU the GPU evaluates the activation in fp32: its result may
    fall on the other side of a bf16 rounding boundary (one bf16 step), or
    flush a vanishing product to zero where float64 keeps a tiny value."""
    uu = u.double().cpu().numpy()
    gg = g.double().cpu().numpy()
    want_bits = oracle.bf16_bits_from_float(uu * oracle.mlp_activation(gg, act))
    if act == "identity":
        assert np.array_equal(a_bits, want_bits), f"{what}: differs from bf16(u * g)"
        return
    got = oracle.float_from_bf16_bits(a_bits)
    want = oracle.float_from_bf16_bits(want_bits)
    step = np.maximum(np.abs(got), np.abs(want)) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= step + 1e-30), f"{what}: product off by more than one step"
    bad = int(np.count_nonzero(got != want))
    note(f"  {what}: {bad} of {a_bits.size} bf16 products differ by one step")
    assert bad <= max(2, a_bits.size // 200), f"{what}: {bad} one-step differences"


@pytest.mark.parametrize("act", ["identity", "silu", "gelu_tanh"])
@pytest.mark.parametrize("group", ["K", 128])
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
def test_mlp_decode_small(r, M, group, act):
    H, F = 256, 640
    note(f"mlp decode r={r} M={M} g={group} act={act}")
    host, devm = _mats(H, F, group, r)
    xb = inputs.activations_bf16("gemma9b_mlp", M, H, matrix=10)
    y, ws = mq.mlp_decode(devm["up"], devm["gate"], devm["down"], r, x_device(xb), act=act)
    torch.cuda.synchronize()
    u, g, a = _split_workspace(ws, M, F)
    for name, t in (("up", u), ("gate", g)):
        p = host[name]
        compare_linear(t, xb, p["q"], p["alpha"], p["zero"], p["group"], r, f"mlp {name}")
    _check_product_bits(a, u, g, act, f"mlp r{r} M{M} {act}")
    p = host["down"]
    compare_linear(y, a, p["q"], p["alpha"], p["zero"], p["group"], r, "mlp down")
    compare(y, oracle.mlp_decode(xb, host["up"], host["gate"], host["down"], r, act),
            f"mlp end-to-end r{r} M{M} {act}", reg=1e-3)


@pytest.mark.parametrize("r", [8, 4, 2])
def test_mlp_decode_gemma_full_size(r):
    """Gemma-2-9B MLP (H = 3584, F = 14336), per-channel, GELU gate, batch 1;
    checked teacher-forced on sampled rows."""
    F, H = inputs.GEMMA9B_MLP["up"]
    note(f"mlp decode gemma full r={r}")
    host, devm = _mats(H, F, "K", r, outlier_frac=1e-3)
    xb = inputs.activations_bf16("gemma9b_mlp", 1, H, matrix=10)
    y, ws = mq.mlp_decode(devm["up"], devm["gate"], devm["down"], r, x_device(xb),
                          act="gelu_tanh")
    torch.cuda.synchronize()
    u, g, a = _split_workspace(ws, 1, F)
    rg = np.random.default_rng(r)
    rows = np.unique(np.concatenate([[0, F - 1], rg.choice(F, 200, replace=False)]))
    for name, t in (("up", u), ("gate", g)):
        p = host[name]
        compare(t[:, rows], oracle.linear(xb, p["q"][rows], p["alpha"][rows], p["zero"][rows],
                                          p["group"], r), f"gemma mlp {name} r{r}")
    _check_product_bits(a, u, g, "gelu_tanh", f"gemma mlp r{r}")
    cols = np.unique(np.concatenate([[0, H - 1], rg.choice(H, 100, replace=False)]))
    p = host["down"]
    compare(y[:, cols], oracle.linear(a, p["q"][cols], p["alpha"][cols], p["zero"][cols],
                                      p["group"], r), f"gemma mlp down r{r}")


def test_mlp_decode_matches_separate_products():
    """The fused block agrees with three mq_gemv calls with the product formed
    by torch in between (identity activation; the split of K, and so the
    summation order, may differ, hence the tolerance)."""
    H, F, r, M = 512, 1024, 4, 2
    host, devm = _mats(H, F, 128, r)
    xb = inputs.activations_bf16("gemma9b_mlp", M, H, matrix=11)
    x = x_device(xb)
    y, ws = mq.mlp_decode(devm["up"], devm["gate"], devm["down"], r, x)
    d = devm
    u2 = mq.gemv(d["up"]["packed"], r, d["up"]["alpha"], d["up"]["zero"], 128, F, H, x)
    g2 = mq.gemv(d["gate"]["packed"], r, d["gate"]["alpha"], d["gate"]["zero"], 128, F, H, x)
    a2 = (u2 * g2).to(torch.bfloat16).view(torch.int16)
    y2 = mq.gemv(d["down"]["packed"], r, d["down"]["alpha"], d["down"]["zero"], 128, H, F, a2)
    torch.cuda.synchronize()
    u, g, a = _split_workspace(ws, M, F)
    compare(u, u2.double().cpu().numpy(), "fused vs separate up")
    compare(y, y2.double().cpu().numpy(), "fused vs separate y")


@pytest.mark.parametrize("r", [2, 4, 8])
def test_mlp_decode_grouped_repeated_identical(r):
    """The paired up/gate launch at group 128, 20 times: every intermediate
    and the output bit-identical to the first call (fixed order), the first
    call's up output against the oracle."""
    H, F, M = 1536, 512, 2
    note(f"mlp repeated r={r}")
    host, devm = _mats(H, F, 128, r, workload="mistral_small")
    xb = inputs.activations_bf16("mistral_small", M, H, matrix=12, heavy_channels=8)
    x = x_device(xb)
    y0, ws0 = mq.mlp_decode(devm["up"], devm["gate"], devm["down"], r, x, act="silu")
    torch.cuda.synchronize()
    u0 = ws0.clone()
    p = host["up"]
    u, _, _ = _split_workspace(ws0, M, F)
    compare_linear(u, xb, p["q"], p["alpha"], p["zero"], p["group"], r, f"mlp repeated up r{r}")
    for i in range(20):
        y, ws = mq.mlp_decode(devm["up"], devm["gate"], devm["down"], r, x, act="silu")
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"call {i}: output differs"
        assert torch.equal(ws, u0), f"call {i}: intermediates differ"


def test_mlp_decode_error_enqueues_nothing():
    H, F, r = 256, 512, 4
    host, devm = _mats(H, F, "K", r)
    _, devg = _mats(H, F, 128, r)
    bad = devg["gate"]                    # a consistent gate at group 128: up's group differs
    x = x_device(inputs.activations_bf16("gemma9b_mlp", 1, H))
    y = torch.full((1, H), 3.0, device=dev())
    with pytest.raises(mq.MQError):
        mq.mlp_decode(devm["up"], bad, devm["down"], r, x, out=y)   # groups differ
    with pytest.raises(mq.MQError):
        mq.mlp_decode(devm["up"], devm["gate"], devm["down"], 5, x, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
