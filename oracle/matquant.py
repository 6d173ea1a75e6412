"""Float64 CPU oracle for the Matryoshka-nested integer matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP library and imports
nothing from it.

Sources (the pages this restates, by title and section):
  [MQX]  "Matryoshka Quantization" explainer (paper-graph-ui, training-methods),
         §3.4 Detailed Breakdown: "Quantization Primitives" (Eq. 1),
         "The Bit-Slicing Operator" (Eq. 6, worked examples, errata Eq. 8),
         "Mix'n'Match and Interpolative Slicing".
  [MQR]  "Pith review of Matryoshka Quantization", "What carries the argument".
  [ROSAQ] "Pith review of ROSAQ", method summary (per-group granularity of 128).

Everything is computed in float64 (plain Python integers for the integer
steps), step by step in the order the pages state, with no blocking, fusion or
reordering.  Readings taken where the pages are silent or ambiguous are marked
READING and listed in the design notes of the repository.
"""

from __future__ import annotations

import numpy as np

C_BITS = 8  # the stored code width c (int8 codes, [MQX] "The Bit-Slicing Operator")


# --------------------------------------------------------------------------
# bf16 (used for the activations, which the pages keep in bfloat16)
# --------------------------------------------------------------------------

def bf16_bits_from_float(v) -> np.ndarray:
    """Round float values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.

    Written from the IEEE definition: a bf16 is the upper half of an fp32;
    the value is first rounded to fp32, then the low 16 bits are rounded away
    to nearest, ties to even.  NaN is not expected in any input.
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    high = u >> 16
    round_up = (low > 0x8000) | ((low == 0x8000) & ((high & 1) == 1))
    high = high + round_up.astype(np.uint64)
    return high.astype(np.uint16)


def float_from_bf16_bits(b) -> np.ndarray:
    """The float64 value of bf16 bit patterns (exact)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Eq. 1: min-max asymmetric quantizer Q_MM(w, c)
# --------------------------------------------------------------------------

def quantize_minmax(w, group: int):
    """Min-max quantization of weights to c = 8-bit unsigned codes ([MQX] Eq. 1).

    w: float32 [N, K] (a real weight matrix stored out-channel major, K = input
    dimension contiguous).  Each "real-valued weight vector" of Eq. 1 is one
    group of `group` consecutive entries of a row (group == K: per output
    channel; group == 128: per group along K, the granularity of [ROSAQ]).

    Per vector:  alpha = (max - min) / (2^c - 1),  z = -min / alpha,
                 q = clamp(round(w / alpha + z), 0, 2^c - 1).
    READINGS: alpha and z are stored as fp32 (z is real, not rounded); alpha is
    the float64 quotient rounded to fp32, z the float64 quotient -min/alpha32
    rounded to fp32; the codes use those stored fp32 values, evaluated in
    float64; round() is floor(v + 1/2); a constant vector (max == min) takes
    alpha = 1, z = -min, so every code is 0 and dequantizes to min exactly.
    The same holds for a vector whose range is too small for a normal fp32
    alpha (alpha32 zero or subnormal, below 2^-126): Eq. 1 divides by alpha,
    and such an alpha is no usable scale, so the vector is treated as
    constant (every code 0, dequantized to min, off by less than 2^-118).

    Returns (q uint8 [N, K], alpha float32 [N, G], zero float32 [N, G]).
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if group <= 0 or k % group:
        raise ValueError("group must divide K")
    g = k // group
    levels = 2 ** C_BITS - 1
    wv = w.reshape(n, g, group).astype(np.float64)
    mn = wv.min(axis=2)
    mx = wv.max(axis=2)
    alpha64 = (mx - mn) / float(levels)
    alpha32 = alpha64.astype(np.float32)
    constant = (mx == mn) | (alpha32 < np.float32(2.0 ** -126))
    alpha32 = np.where(constant, np.float32(1.0), alpha32)
    zero32 = (-mn / alpha32.astype(np.float64)).astype(np.float32)
    a = alpha32.astype(np.float64)[:, :, None]
    z = zero32.astype(np.float64)[:, :, None]
    v = wv / a + z
    q = np.floor(v + 0.5)
    q = np.clip(q, 0, levels)
    return q.astype(np.uint8).reshape(n, k), alpha32, zero32


# --------------------------------------------------------------------------
# Eq. 6 (and the erratum Eq. 8): the bit-slicing operator S(q_c, r)
# --------------------------------------------------------------------------

def _round_half_up(v: np.ndarray) -> np.ndarray:
    # The first discarded bit decides: 1 rounds up, 0 rounds down.  For a
    # quotient by a power of two this is "round half up" ([MQX] "The
    # Bit-Slicing Operator", the tie-breaking rule stated after Eq. 6).
    return np.floor(v + 0.5)


def slice_value(q, r: int) -> np.ndarray:
    """S(q, r) = clamp(round(q / 2^(c-r)), 0, 2^r - 1) * 2^(c-r)  ([MQX] Eq. 6).

    q: integer codes in [0, 2^c - 1].  Returns int64 values on the int8 scale
    (multiples of 2^(c-r) with c - r trailing zero bits).  q / 2^(c-r) is exact
    in float64, so the rounding is exact.
    """
    if not 1 <= r <= C_BITS:
        raise ValueError("r must be in 1..8")
    step = float(2 ** (C_BITS - r))
    t = _round_half_up(np.asarray(q, dtype=np.float64) / step)
    t = np.clip(t, 0, 2 ** r - 1)
    return (t * step).astype(np.int64)


def slice_index(q, r: int) -> np.ndarray:
    """The r-bit index t with S(q, r) = t * 2^(c-r); t in [0, 2^r - 1]."""
    return slice_value(q, r) // (2 ** (C_BITS - r))


def slice_value_noclamp(q, r: int) -> np.ndarray:
    """The erratum operator without the clamp ([MQX] "The errata correction",
    Eq. 8): round(q / 2^(c-r)) * 2^(c-r).  Takes 2^r + 1 levels; the top one is
    2^c = 256, which needs an extra bit ("Extra-Precision MatQuant")."""
    if not 1 <= r <= C_BITS:
        raise ValueError("r must be in 1..8")
    step = float(2 ** (C_BITS - r))
    t = _round_half_up(np.asarray(q, dtype=np.float64) / step)
    return (t * step).astype(np.int64)


# --------------------------------------------------------------------------
# Storage of a sliced plane (the pages fix values only; this is the layout)
# --------------------------------------------------------------------------

# r = 3 and r = 6 ("interpolative" precisions between the nested 2/4/8, served
# from the same codes: [MQX] "Mix'n'Match and Interpolative Slicing") are not
# byte-aligned.  Their index t is stored as two planes of the word layout
# below: the high bits t >> r_lo, then the low bits t & (2^r_lo - 1).
SPLIT_WIDTHS = {3: (2, 1), 6: (4, 2)}  # r -> (r_hi, r_lo)


def pack_indices(t, r: int) -> np.ndarray:
    """Pack r-bit indices t [N, K] into bytes [N, K*r/8].

    LAYOUT (a reading; the pages define values, not storage): rows stay rows;
    each row is cut into 32-bit words of 32/r consecutive elements.  Inside a
    word, the elements at even positions 0, 2, 4, ... fill the low 16 bits and
    the elements at odd positions 1, 3, 5, ... fill the high 16 bits; in each
    half, the j-th of them occupies bits [j*r, j*r + r) of that half.  Words
    are stored little-endian.  K must be a multiple of 32/r.

    LAYOUT for r = 3 and r = 6 (also a reading): the N*K*r/8 bytes are two
    planes back to back, first the r_hi-bit plane of t >> r_lo for all rows,
    then the r_lo-bit plane of t & (2^r_lo - 1) for all rows (each as above;
    (r_hi, r_lo) = (2, 1) for r = 3 and (4, 2) for r = 6).  The result is that
    byte sequence viewed as [N, K*r/8]; its rows are not the weight rows.
    """
    if r in SPLIT_WIDTHS:
        t = np.asarray(t, dtype=np.int64)
        n, k = t.shape
        if t.min(initial=0) < 0 or t.max(initial=0) >= 2 ** r:
            raise ValueError("index out of range for r bits")
        r_hi, r_lo = SPLIT_WIDTHS[r]
        hi = pack_indices(t >> r_lo, r_hi)
        lo = pack_indices(t & ((1 << r_lo) - 1), r_lo)
        return np.concatenate([hi.reshape(-1), lo.reshape(-1)]).reshape(n, k * r // 8)
    if r not in (1, 2, 4, 8):
        raise ValueError("packing needs r in {1,2,3,4,6,8}")
    t = np.asarray(t, dtype=np.int64)
    n, k = t.shape
    per_word = 32 // r
    half = 16 // r
    if k % per_word:
        raise ValueError("K must be a multiple of 32/r")
    if t.min(initial=0) < 0 or t.max(initial=0) >= 2 ** r:
        raise ValueError("index out of range for r bits")
    elems = t.reshape(n, k // per_word, per_word)
    word = np.zeros((n, k // per_word), dtype=np.int64)
    for j in range(half):
        word |= elems[:, :, 2 * j] << (j * r)            # even position 2j: low half
        word |= elems[:, :, 2 * j + 1] << (16 + j * r)   # odd position 2j+1: high half
    out = np.zeros((n, k // per_word, 4), dtype=np.uint8)
    for b in range(4):
        out[:, :, b] = (word >> (8 * b)) & 0xFF          # little-endian bytes
    return out.reshape(n, k * r // 8)


def unpack_indices(packed, r: int, k: int) -> np.ndarray:
    """Inverse of pack_indices: bytes [N, K*r/8] -> indices int64 [N, K]."""
    if r in SPLIT_WIDTHS:
        p = np.asarray(packed, dtype=np.int64)
        n = p.shape[0]
        if p.shape[1] * 8 != k * r:
            raise ValueError("packed width does not match K")
        r_hi, r_lo = SPLIT_WIDTHS[r]
        flat = p.reshape(-1)
        cut = n * k * r_hi // 8
        hi = unpack_indices(flat[:cut].reshape(n, k * r_hi // 8), r_hi, k)
        lo = unpack_indices(flat[cut:].reshape(n, k * r_lo // 8), r_lo, k)
        return (hi << r_lo) | lo
    if r not in (1, 2, 4, 8):
        raise ValueError("packing needs r in {1,2,3,4,6,8}")
    p = np.asarray(packed, dtype=np.int64)
    n = p.shape[0]
    per_word = 32 // r
    half = 16 // r
    if p.shape[1] * 8 != k * r or k % per_word:
        raise ValueError("packed width does not match K")
    b = p.reshape(n, k // per_word, 4)
    word = b[:, :, 0] | (b[:, :, 1] << 8) | (b[:, :, 2] << 16) | (b[:, :, 3] << 24)
    mask = (1 << r) - 1
    out = np.zeros((n, k // per_word, per_word), dtype=np.int64)
    for j in range(half):
        out[:, :, 2 * j] = (word >> (j * r)) & mask
        out[:, :, 2 * j + 1] = (word >> (16 + j * r)) & mask
    return out.reshape(n, k)


def pack_codes(q, r: int) -> np.ndarray:
    """Slice stored codes to r bits and pack them: the plane a server at
    precision r reads ([MQX] §2: lower precisions are obtained from the one
    stored int8 model by slicing)."""
    return pack_indices(slice_index(q, r), r)


# --------------------------------------------------------------------------
# Bit-plane storage: one stored copy of the codes that serves every r
# --------------------------------------------------------------------------

BITPLANE_SUPERBLOCK = 512  # codes per superblock of a plane row (64 bytes)


def pack_bitplanes(q) -> np.ndarray:
    """The eight bit-planes of the stored codes: uint8 [8, N, K/8], plane p
    holding bit p of every code (p = 0 is the least significant bit).

    The pages store one int8 model and obtain every lower precision from its
    most significant bits ([MQX] "The Bit-Slicing Operator"; §2 on slicing the
    one stored model).  Stored by bit, a server at precision r reads only the
    planes it needs.

    LAYOUT (a reading; the pages define no storage): each row of a plane is cut
    into superblocks of 512 codes (64 bytes = 16 little-endian 32-bit words);
    word 4*s + G of a superblock holds, at bit 16*h + i, the bit of code
    128*G + 32*s + 2*i + h of that superblock (s, G in 0..3, i in 0..15,
    h in 0..1).  K must be a multiple of 512.
    """
    q = np.asarray(q)
    if q.ndim != 2 or np.any(q < 0) or np.any(q > 255):
        raise ValueError("codes must be a 2-D array of values in 0..255")
    n, k = q.shape
    if k % BITPLANE_SUPERBLOCK:
        raise ValueError("K must be a multiple of 512")
    qi = q.astype(np.int64)
    out = np.zeros((8, n, k // 8), dtype=np.uint8)
    for p in range(8):
        bits = (qi >> p) & 1
        words = np.zeros((n, k // 32), dtype=np.int64)
        for sb in range(k // BITPLANE_SUPERBLOCK):
            for s in range(4):
                for g in range(4):
                    w = 0
                    for i in range(16):
                        for h in range(2):
                            code = sb * 512 + 128 * g + 32 * s + 2 * i + h
                            w = w | (bits[:, code] << (16 * h + i))
                    words[:, sb * 16 + 4 * s + g] = w
        for b in range(4):
            out[p, :, b::4] = (words >> (8 * b)) & 0xFF
    return out


def unpack_bitplanes(planes) -> np.ndarray:
    """Inverse of pack_bitplanes: uint8 [8, N, K/8] -> codes int64 [N, K]."""
    pl = np.asarray(planes, dtype=np.int64)
    if pl.ndim != 3 or pl.shape[0] != 8:
        raise ValueError("planes must be [8, N, K/8]")
    _, n, kb = pl.shape
    k = kb * 8
    if k % BITPLANE_SUPERBLOCK:
        raise ValueError("K must be a multiple of 512")
    q = np.zeros((n, k), dtype=np.int64)
    for p in range(8):
        words = pl[p, :, 0::4] | (pl[p, :, 1::4] << 8) | (pl[p, :, 2::4] << 16) | (pl[p, :, 3::4] << 24)
        for sb in range(k // BITPLANE_SUPERBLOCK):
            for s in range(4):
                for g in range(4):
                    w = words[:, sb * 16 + 4 * s + g]
                    for i in range(16):
                        for h in range(2):
                            code = sb * 512 + 128 * g + 32 * s + 2 * i + h
                            q[:, code] |= ((w >> (16 * h + i)) & 1) << p
    return q


def slice_index_from_bitplanes(planes, r: int, extra: bool = False) -> np.ndarray:
    """The r-bit index read from bit-planes, int64 [N, K].

    The quotient q / 2^(8-r) splits into its integer part h (the r most
    significant bits, planes 8-r .. 7) and the first discarded bit c (plane
    7-r); rounding half up adds c ([MQX] "The Bit-Slicing Operator": the first
    discarded bit decides the rounding).  Eq. 6 clamps h + c to 2^r - 1, which
    matters only when h is all ones and c = 1; with extra=True the clamp is
    left out (the errata Eq. 8, Extra-Precision MatQuant) and the index can be
    2^r.  At r = 8 nothing is discarded: the index is q."""
    if not 1 <= r <= C_BITS:
        raise ValueError("r must be in 1..8")
    pl = np.asarray(planes, dtype=np.int64)
    _, n, kb = pl.shape
    bits = [None] * 8
    q = unpack_bitplanes(pl)
    for p in range(8):
        bits[p] = (q >> p) & 1
    h = np.zeros((n, kb * 8), dtype=np.int64)
    for j in range(r):
        h = h + (bits[C_BITS - r + j] << j)
    if r == C_BITS:
        return h
    c = bits[C_BITS - 1 - r]
    t = h + c
    if not extra:
        t = np.minimum(t, 2 ** r - 1)
    return t


def bitplane_bytes_read(n: int, k: int, r: int) -> int:
    """Bytes of planes a server at r reads: r + 1 planes (all 8 at r = 8)."""
    return n * (k // 8) * (min(r + 1, C_BITS))


# --------------------------------------------------------------------------
# Dequantization and the matrix product
# --------------------------------------------------------------------------

def dequant(q, alpha, zero, group: int, r: int) -> np.ndarray:
    """w_hat = (S(q, r) - z) * alpha, float64 [N, K]  ([MQX] Eq. 1's
    dequantization alpha*(q - z), applied to the sliced value, which is used
    "as if it were an int8 value", "The Bit-Slicing Operator").
    READING: the sliced model keeps the int8 alpha and z."""
    q = np.asarray(q)
    n, k = q.shape
    g = k // group
    s = slice_value(q, r).astype(np.float64).reshape(n, g, group)
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(n, g, 1)
    z = np.asarray(zero, dtype=np.float32).astype(np.float64).reshape(n, g, 1)
    return ((s - z) * a).reshape(n, k)


def dequant_rows(q_rows, alpha_rows, zero_rows, group: int, r: int) -> np.ndarray:
    """dequant() of a subset of rows (for sampled checks of large matrices)."""
    return dequant(q_rows, alpha_rows, zero_rows, group, r)


def linear(x_bf16_bits, q, alpha, zero, group: int, r: int) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w_hat[n, k]  in float64.

    x: bf16 bit patterns uint16 [M, K]; the weight matrix is stored [N, K]
    (the transpose of the pages' W in XW), so y = x @ w_hat^T.
    """
    x = float_from_bf16_bits(x_bf16_bits)
    if x.ndim == 1:
        x = x[None, :]
    return x @ dequant(q, alpha, zero, group, r).T


# --------------------------------------------------------------------------
# Extra-Precision MatQuant: the slice without the clamp (errata Eq. 8)
# --------------------------------------------------------------------------

def dequant_extra_precision(q, alpha, zero, group: int, r: int) -> np.ndarray:
    """w_hat = (S'(q, r) - z) * alpha with S' the unclamped slice of the
    errata Eq. 8 ([MQX] "The Bit-Slicing Operator"): 2^r + 1 levels, the top
    one 256 ("Extra-Precision MatQuant"; [MQX] §5 "Ablation Studies and
    Robustness Checks" on the few weights that use it).  Same alpha and z."""
    q = np.asarray(q)
    n, k = q.shape
    g = k // group
    s = slice_value_noclamp(q, r).astype(np.float64).reshape(n, g, group)
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(n, g, 1)
    z = np.asarray(zero, dtype=np.float32).astype(np.float64).reshape(n, g, 1)
    return ((s - z) * a).reshape(n, k)


def linear_extra_precision(x_bf16_bits, q, alpha, zero, group: int, r: int) -> np.ndarray:
    """y = x @ w_hat^T with the extra-precision w_hat, float64."""
    x = float_from_bf16_bits(x_bf16_bits)
    if x.ndim == 1:
        x = x[None, :]
    return x @ dequant_extra_precision(q, alpha, zero, group, r).T


def overflow_lists(q, r: int):
    """Positions of the codes whose unclamped slice reaches the extra level
    256 (the only codes where Eq. 8 and Eq. 6 differ), per row in increasing
    k: (row_ptr int64 [N + 1], col_idx int64 [nnz]).

    READING (storage of the extra bit; the pages note that a custom kernel
    would have to add it sparsely, [MQX] §5 "Critical Assessment"): the r-bit
    plane keeps the clamped index and these lists mark where one more level
    of 2^(8-r) is added."""
    mask = slice_value_noclamp(q, r) == 2 ** C_BITS
    row_ptr = np.concatenate([[0], np.cumsum(mask.sum(axis=1))]).astype(np.int64)
    col_idx = np.nonzero(mask)[1].astype(np.int64)  # row-major: increasing k in a row
    return row_ptr, col_idx


# --------------------------------------------------------------------------
# Mix'n'Match: a stack of linears, each layer at its own precision r
# --------------------------------------------------------------------------

LAYER_LINEARS = ("q", "k", "v", "o", "up", "gate", "down")


def rms_normalize(h) -> np.ndarray:
    """h / sqrt(mean(h^2)) per row (no gain, no epsilon).  READING: the pages
    give no layer dataflow for a Mix'n'Match stack; a gain-free RMS
    normalization keeps the activations bounded through the stack."""
    h = np.asarray(h, dtype=np.float64)
    rms = np.sqrt(np.mean(h * h, axis=-1, keepdims=True))
    return h / rms


def bf16_round(v) -> np.ndarray:
    """Round float values to the nearest bf16 value (ties to even), float64."""
    return float_from_bf16_bits(bf16_bits_from_float(v))


def mixnmatch_layer(h, layer, trace=None):
    """One layer of the Mix'n'Match stack ([MQX] "Mix'n'Match": one stored
    int8 model, a different slice precision r per layer).

    READING of the layer dataflow (the pages give none):
      a = bf16(rms_normalize(h));
      q, k, v, u, g = W_q a, W_k a, W_v a, W_up a, W_gate a;
      o = W_o bf16(q);  d = W_down bf16(u * g);
      h <- h + o + d.
    k and v are computed and not consumed (attention is out of scope).
    layer: dict with key "r" and, per linear name, a dict with q, alpha, zero,
    group (stored codes; the layer's r is applied by slicing).
    trace: optional dict that receives the intermediate values.
    """
    r = layer["r"]
    a_bits = bf16_bits_from_float(rms_normalize(h))

    def lin(name, xb):
        p = layer[name]
        return linear(xb, p["q"], p["alpha"], p["zero"], p["group"], r)

    outs = {name: lin(name, a_bits) for name in ("q", "k", "v", "up", "gate")}
    q_bits = bf16_bits_from_float(outs["q"])
    ug_bits = bf16_bits_from_float(outs["up"] * outs["gate"])
    o = lin("o", q_bits)
    d = lin("down", ug_bits)
    h_new = np.asarray(h, dtype=np.float64) + o + d
    if trace is not None:
        trace.update(a_bits=a_bits, q_bits=q_bits, ug_bits=ug_bits, o=o, d=d, **outs)
    return h_new


def mixnmatch_forward(layers, x_bf16_bits, traces=None) -> np.ndarray:
    """Run the stack: h0 = x (bf16 values), then every layer in order.
    Returns float64 h [M, H].  traces: optional list that receives one dict of
    intermediates per layer."""
    h = float_from_bf16_bits(x_bf16_bits)
    if h.ndim == 1:
        h = h[None, :]
    for layer in layers:
        tr = {} if traces is not None else None
        h = mixnmatch_layer(h, layer, tr)
        if traces is not None:
            traces.append(tr)
    return h


# --------------------------------------------------------------------------
# Decode MLP block: up and gate from one x, the gated product, then down
# --------------------------------------------------------------------------

MLP_ACTIVATIONS = ("identity", "silu", "gelu_tanh")


def mlp_activation(g, act: str) -> np.ndarray:
    """The gate activation of a gated MLP, float64.
    READING (the pages name the FFN as the main decode cost, [MQX] §5, but
    give no block): identity (the elementwise gate of the Mix'n'Match
    reading), SiLU g * sigmoid(g), or GELU in its tanh form
    g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))."""
    g = np.asarray(g, dtype=np.float64)
    if act == "identity":
        return g
    if act == "silu":
        return g / (1.0 + np.exp(-g))
    if act == "gelu_tanh":
        # g/2 * (1 + tanh(z)) written as g / (1 + exp(-2z)), the same function:
        # 1 + tanh(z) cancels to 0 in float64 once tanh(z) rounds to -1
        # (g below about -7), where the product is still about 1e-17
        z = np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)
        with np.errstate(over="ignore"):
            return g / (1.0 + np.exp(-2.0 * z))
    raise ValueError(f"unknown activation {act!r}")


def mlp_decode(x_bf16_bits, up, gate, down, r: int, act: str = "identity", trace=None):
    """y = W_down bf16(act(W_gate x) * W_up x) with every W the stored codes
    sliced to r ([MQX] Eq. 6 and dequantization as in linear()).
    up, gate: dicts q, alpha, zero, group of [F, H]; down: of [H, F].
    The gated product is formed in float64 and rounded to bf16 (nearest even),
    the precision of the activations the product takes."""
    u = linear(x_bf16_bits, up["q"], up["alpha"], up["zero"], up["group"], r)
    g = linear(x_bf16_bits, gate["q"], gate["alpha"], gate["zero"], gate["group"], r)
    a_bits = bf16_bits_from_float(mlp_activation(g, act) * u)
    y = linear(a_bits, down["q"], down["alpha"], down["zero"], down["group"], r)
    if trace is not None:
        trace.update(u=u, g=g, a_bits=a_bits)
    return y


def effective_bits(layers) -> float:
    """Average stored bits per weight of a Mix'n'Match assignment (the
    "effective bits per parameter" measure of [MQX] "Mix'n'Match")."""
    total = 0
    bits = 0
    for layer in layers:
        for name in LAYER_LINEARS:
            n = int(np.asarray(layer[name]["q"]).size)
            total += n
            bits += n * layer["r"]
    return bits / total
