"""GPU parity of the Mix'n'Match stack at the Mistral-7B shapes of the
benchmark (H = 4096, Hkv = 1024, F = 14336, per-channel scales, one slice
precision per layer from the 32-layer pattern): layers 7-10 of that pattern,
r = 8, 4, 4, 2, so the run crosses 8 -> 4 -> 2 ("Matryoshka Quantization"
explainer, §3.4 "Mix'n'Match and Interpolative Slicing").

Weights are drawn and quantized on the host by the oracle (the same seeds
per layer and matrix as the stack of the benchmark; its device-drawn weights
follow the same law), then uploaded and packed.  Every linear of every layer
is checked teacher-forced on sampled rows against the oracle with the GPU's
own bf16 input, and the four layers end to end against the float64 stack on
all 4096 outputs.
"""

import numpy as np
import pytest
import torch

import nested_int_matmul_amd as mq
import oracle
from nested_int_matmul_amd import inputs

from gpu_helpers import compare, compare_linear, dev, note, x_device

pytestmark = pytest.mark.gpu

LAYERS = (7, 8, 9, 10)
ROWS = 200


@pytest.fixture(scope="module")
def stack():
    rs_all = inputs.mixnmatch_pattern(32)
    assert [rs_all[i] for i in LAYERS] == [8, 4, 4, 2]
    host, devl = [], []
    for li in LAYERS:
        r = rs_all[li]
        note(f"stack layer {li} (r={r}): weights, oracle quantization, upload")
        hl, dl = {"r": r}, {"r": r}
        for mi, name in enumerate(mq.LAYER_LINEARS):
            n, k = inputs.MISTRAL_LAYER[name]
            w = inputs.gaussian_weights("mistral_stack", n, k, layer=li, matrix=mi)
            q, a, z = oracle.quantize_minmax(w, k)
            del w
            hl[name] = {"q": q, "alpha": a, "zero": z, "group": k}
            qd = torch.from_numpy(q).to(dev())
            dl[name] = {"packed": mq.pack(qd, r), "alpha": torch.from_numpy(a).to(dev()),
                        "zero": torch.from_numpy(z).to(dev()), "N": n, "K": k, "group": k}
            del qd
        host.append(hl)
        devl.append(dl)
    torch.cuda.synchronize()
    H = inputs.MISTRAL_LAYER["q"][0]
    xb = inputs.activations_bf16("mistral_stack", 1, H)
    return {"host": host, "dev": devl, "xb": xb, "H": H}


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("pos", range(len(LAYERS)))
def test_stack_mistral_teacher_forced(stack, pos):
    """Layer LAYERS[pos] run alone (in-place form) on the residual stream the
    GPU computed for the layers before it; each of its seven products against
    the oracle on the GPU's own bf16 input, on ROWS sampled output rows; the
    bf16 copies of q and u * g bit-exact against the rounding of the GPU's
    own fp32 outputs; the residual update exact in fp32."""
    host, devl, xb, H = stack["host"], stack["dev"], stack["xb"], stack["H"]
    L, r = host[pos], host[pos]["r"]
    note(f"stack teacher-forced layer {LAYERS[pos]} r={r}")
    arr_before = mq.make_layers(devl[:pos]) if pos else None
    one = mq.make_layers(devl[pos:pos + 1])
    ws = torch.empty(mq.mixnmatch_workspace_bytes(one, 1), dtype=torch.uint8, device=dev())
    off = mq.mixnmatch_workspace_offsets(one, 1)
    if pos:
        h = mq.mixnmatch_forward(arr_before, x_device(xb), ws)
    else:
        h = x_device(xb).view(torch.bfloat16).float()
    h_in = h.clone()
    mq.mixnmatch_forward_inplace(one, h, ws)
    torch.cuda.synchronize()

    Hkv, F = inputs.MISTRAL_LAYER["k"][0], inputs.MISTRAL_LAYER["up"][0]
    a_bits = _bits(ws[off[0]:off[0] + H * 2]).reshape(1, H)
    want_a = oracle.bf16_bits_from_float(oracle.rms_normalize(h_in.double().cpu().numpy()))
    mism = int(np.count_nonzero(a_bits != want_a))
    assert mism <= H // 200, f"{mism} bf16 rounding differences in the normalized input"

    def fetch(i, n):
        return ws[off[i]:off[i] + n * 4].view(torch.float32).reshape(1, n)

    outs = {"q": fetch(1, H), "k": fetch(2, Hkv), "v": fetch(3, Hkv), "up": fetch(4, F),
            "gate": fetch(5, F)}
    rg = np.random.default_rng(LAYERS[pos])
    for name, y in outs.items():
        p = L[name]
        n = y.shape[1]
        rows = np.unique(np.concatenate([[0, n - 1], rg.choice(n, ROWS, replace=False)]))
        compare_linear(y[:, rows], a_bits, p["q"][rows], p["alpha"][rows], p["zero"][rows],
                       p["group"], r, f"layer {LAYERS[pos]} {name}")
    qb = _bits(outs["q"].to(torch.bfloat16))
    ugb = _bits((outs["up"] * outs["gate"]).to(torch.bfloat16))
    np.testing.assert_array_equal(_bits(ws[off[8]:off[8] + H * 2]).reshape(1, H), qb)
    np.testing.assert_array_equal(_bits(ws[off[9]:off[9] + F * 2]).reshape(1, F), ugb)
    o, d = fetch(6, H), fetch(7, H)
    for name, y, xin in (("o", o, qb), ("down", d, ugb)):
        p = L[name]
        rows = np.unique(np.concatenate([[0, H - 1], rg.choice(H, ROWS, replace=False)]))
        compare_linear(y[:, rows], xin, p["q"][rows], p["alpha"][rows], p["zero"][rows],
                       p["group"], r, f"layer {LAYERS[pos]} {name}")
    assert torch.equal(h, (h_in + o) + d), "residual update"


def _forward_perturbed(weights, rs, xb, eps, seed):
    """The oracle's layer loop (oracle.mixnmatch_layer: a = bf16(h/rms(h)),
    q, k, v, u, g = W a, o = W_o bf16(q), d = W_down bf16(u g), h += o + d)
    on dequantized float64 weights, with every product's float64 result
    multiplied by (1 + eps * N(0, 1)) before it is rounded or added: how far
    the stack moves when each product carries a relative error of about eps.
    k and v are not consumed and are skipped."""
    rg = np.random.default_rng(seed)
    h = oracle.float_from_bf16_bits(xb).reshape(1, -1)
    for W in weights:
        a = oracle.float_from_bf16_bits(oracle.bf16_bits_from_float(oracle.rms_normalize(h)))

        def lin(name, x):
            y = x @ W[name].T
            return y * (1.0 + eps * rg.standard_normal(y.shape)) if eps else y

        q, u, g = lin("q", a), lin("up", a), lin("gate", a)
        qb = oracle.float_from_bf16_bits(oracle.bf16_bits_from_float(q))
        ub = oracle.float_from_bf16_bits(oracle.bf16_bits_from_float(u * g))
        h = h + lin("o", qb) + lin("down", ub)
    return h


def test_stack_mistral_end_to_end(stack):
    """Layers 7-10 in one call from the bf16 input against the float64 stack,
    all 4096 outputs.

    Each layer rounds a, q and u * g to bf16, so two correct evaluations
    whose products differ at the fp32 level (relative 1e-7 to 1e-6) round a
    few near-tie values apart; the next layers amplify those flips until the
    stack's outputs differ at the bf16 noise level.  The oracle measures that
    floor itself: the same float64 layers with each product perturbed by
    1e-6 (two seeds) land 3e-3 to 4e-3 (rel-L2) away from the unperturbed
    result at these shapes.  So the bound end to end is twice that floor (and
    never below the 1e-3 bar); each product is held to the bar and the
    regression bounds in the teacher-forced test, and one layer end to end
    to the bar."""
    host, devl, xb, H = stack["host"], stack["dev"], stack["xb"], stack["H"]
    note("stack end to end, layers 7-10")
    arr = mq.make_layers(devl)
    ws = torch.empty(mq.mixnmatch_workspace_bytes(arr, 1), dtype=torch.uint8, device=dev())
    h = mq.mixnmatch_forward(arr, x_device(xb), ws)
    h1 = mq.mixnmatch_forward(mq.make_layers(devl[:1]), x_device(xb), ws)
    torch.cuda.synchronize()
    note("  oracle: one and four float64 layers")
    ref1 = oracle.mixnmatch_forward(host[:1], xb)
    compare(h1, ref1, "stack mistral layer 7 alone, end to end", reg=1e-3)
    ref = oracle.mixnmatch_forward(host, xb)
    note("  oracle sensitivity floor (products perturbed by 1e-6)")
    weights = [{nm: oracle.dequant(L[nm]["q"], L[nm]["alpha"], L[nm]["zero"], L[nm]["group"],
                                   L["r"]) for nm in ("q", "o", "up", "gate", "down")}
               for L in host]
    rs = [L["r"] for L in host]
    base = _forward_perturbed(weights, rs, xb, 0.0, 0)
    assert np.allclose(base, ref, rtol=1e-12, atol=1e-12)  # the loop above is the oracle's
    floor = max(float(np.linalg.norm(_forward_perturbed(weights, rs, xb, 1e-6, s) - ref)
                      / np.linalg.norm(ref)) for s in (1, 2))
    del weights
    bound = max(1e-3, 2.0 * floor)
    note(f"  sensitivity floor {floor:.3e}: bound {bound:.3e}")
    got = h.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    note(f"  parity stack mistral layers 7-10 end to end: rel-L2 {rel:.3e} "
         f"max-abs {np.abs(got - ref).max():.3e} (bound {bound:.3e})")
    assert rel <= bound
