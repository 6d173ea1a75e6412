"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, the rounding rule as the pages state it in words (a bit-level
formulation, independent of the oracle's division-based one), closed forms,
brute force over every code, exact rational arithmetic, and torch's own bf16
conversion.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL_CODES = np.arange(256)


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ---------------------------------------------------------------- slicing

def test_worked_examples():
    for q, r, s in _rows("slice_worked_examples.txt"):
        assert oracle.slice_value(int(q), int(r)) == int(s)


def test_ties_follow_the_rule_in_words():
    for q, r, s in _rows("slice_ties.txt"):
        assert oracle.slice_value(int(q), int(r)) == int(s)


def _slice_by_bits(q: int, r: int, clamp: bool = True) -> int:
    """The operator as the pages describe it in words: keep the r most
    significant bits, round up when the first discarded bit is 1, clamp to
    the r-bit range (not in the errata's unclamped form), shift back."""
    if r == 8:
        return q
    kept = q >> (8 - r)
    first_discarded = (q >> (7 - r)) & 1
    t = kept + first_discarded
    if clamp:
        t = min(t, 2 ** r - 1)
    return t << (8 - r)


@pytest.mark.parametrize("r", range(1, 9))
def test_bruteforce_against_bit_rule(r):
    got = oracle.slice_value(ALL_CODES, r)
    want = [_slice_by_bits(int(q), r) for q in ALL_CODES]
    assert got.tolist() == want


@pytest.mark.parametrize("r", range(1, 9))
def test_nearest_level_with_ties_up(r):
    # S(q, r) is the nearest level t * 2^(8-r), t in [0, 2^r - 1], with ties
    # going to the larger level (the rounding rule), by exhaustive search.
    levels = np.arange(2 ** r) * 2 ** (8 - r)
    for q in range(256):
        d = np.abs(levels - q)
        best = levels[d == d.min()].max()
        assert oracle.slice_value(q, r) == best


def test_r8_is_identity():
    assert oracle.slice_value(ALL_CODES, 8).tolist() == ALL_CODES.tolist()
    assert oracle.slice_index(ALL_CODES, 8).tolist() == ALL_CODES.tolist()


@pytest.mark.parametrize("r", range(1, 9))
def test_multiples_and_range(r):
    s = oracle.slice_value(ALL_CODES, r)
    step = 2 ** (8 - r)
    assert np.all(s % step == 0)
    assert s.min() >= 0 and s.max() <= (2 ** r - 1) * step <= 255
    t = oracle.slice_index(ALL_CODES, r)
    assert np.array_equal(t * step, s)


def test_level_sets():
    for row in _rows("slice_levels.txt"):
        variant, r, levels = row[0], int(row[1]), [int(v) for v in row[2:]]
        fn = oracle.slice_value if variant == "clamp" else oracle.slice_value_noclamp
        assert sorted(set(fn(ALL_CODES, r).tolist())) == levels


def test_r2_buckets():
    # Consequence of Eq. 6 over all codes: [0,31]->0, [32,95]->64,
    # [96,159]->128, [160,255]->192.
    s = oracle.slice_value(ALL_CODES, 2)
    want = np.select([ALL_CODES < 32, ALL_CODES < 96, ALL_CODES < 160], [0, 64, 128], 192)
    assert np.array_equal(s, want)


@pytest.mark.parametrize("r", range(1, 9))
def test_nesting_and_idempotence(r):
    s = oracle.slice_value(ALL_CODES, r)
    assert np.array_equal(oracle.slice_value(s, r), s)
    for r2 in range(r, 9):
        # the value set of a coarser slice lies inside every finer one
        assert np.array_equal(oracle.slice_value(s, r2), s)


def test_slicing_does_not_compose_downwards():
    # Slicing the int4 slice to int2 is not the int2 slice: double rounding
    # changes exactly the 24 codes 24-31, 88-95, 152-159.
    via4 = oracle.slice_value(oracle.slice_value(ALL_CODES, 4), 2)
    direct = oracle.slice_value(ALL_CODES, 2)
    diff = np.nonzero(via4 != direct)[0].tolist()
    assert diff == list(range(24, 32)) + list(range(88, 96)) + list(range(152, 160))


@pytest.mark.parametrize("r", range(1, 9))
def test_noclamp_overflow_count(r):
    # Without the clamp, round(q / 2^(8-r)) = 2^r exactly when
    # q >= 256 - 2^(7-r): 2^(7-r) codes for r <= 7, none for r = 8.
    s = oracle.slice_value_noclamp(ALL_CODES, r)
    n256 = int(np.sum(s == 256))
    assert n256 == (2 ** (7 - r) if r < 8 else 0)
    clamped = oracle.slice_value(ALL_CODES, r)
    assert np.array_equal(np.minimum(s, (2 ** r - 1) * 2 ** (8 - r)), clamped)


# ---------------------------------------------------------------- quantizer

def _hand():
    d = {}
    for row in _rows("hand_linear.txt"):
        d.setdefault(row[0], []).append(row[1:])
    return d


def test_hand_quantize():
    h = _hand()
    w = np.array([[float(v) for v in h["w"][0]]], dtype=np.float32)
    q, a, z = oracle.quantize_minmax(w, 4)
    assert q[0].tolist() == [int(v) for v in h["q"][0]]
    assert a[0, 0] == np.float32(2.0 / 255.0)
    assert z[0, 0] == np.float32(127.49999237060547)


@pytest.mark.parametrize("group", [128, 512])
def test_quantizer_invariants(group):
    rg = np.random.default_rng(7)
    w = (rg.standard_normal((16, 512)) * 0.02).astype(np.float32)
    q, a, z = oracle.quantize_minmax(w, group)
    g = 512 // group
    qv = q.reshape(16, g, group).astype(np.int64)
    wv = w.reshape(16, g, group)
    # the minimum of every vector maps to 0 and the maximum to 255
    assert np.all(qv[np.arange(16)[:, None], np.arange(g)[None, :], wv.argmin(2)] == 0)
    assert np.all(qv[np.arange(16)[:, None], np.arange(g)[None, :], wv.argmax(2)] == 255)
    # monotone within a vector
    order = np.argsort(wv, axis=2, kind="stable")
    qs = np.take_along_axis(qv, order, axis=2)
    assert np.all(np.diff(qs, axis=2) >= 0)
    # reconstruction error of the int8 model is at most half a step
    what = oracle.dequant(q, a, z, group, 8)
    step = np.repeat(a.astype(np.float64), group, axis=1)
    assert np.all(np.abs(what - w) <= 0.5 * step * (1 + 1e-6) + 1e-12)


def test_quantizer_exact_rationals():
    # q = floor(w/alpha + z + 1/2) with the stored fp32 alpha, z, in exact
    # rational arithmetic, agrees with the float64 evaluation.
    rg = np.random.default_rng(11)
    w = (rg.standard_normal((8, 256)) * 0.02).astype(np.float32)
    q, a, z = oracle.quantize_minmax(w, 128)
    for n in range(8):
        for k in range(256):
            g = k // 128
            v = Fraction(float(w[n, k])) / Fraction(float(a[n, g])) + Fraction(float(z[n, g]))
            want = min(max(int(np.floor(v + Fraction(1, 2))), 0), 255)
            assert q[n, k] == want


def test_tiny_range_vector_is_treated_as_constant():
    """A vector whose fp32 alpha would be subnormal or zero takes the
    constant-vector reading (alpha = 1, z = -min, every code 0); a range of
    exactly 255 * 2^-126 gives the smallest normal alpha, 2^-126, and the
    ordinary codes 0 and 255."""
    w = np.zeros((3, 128), dtype=np.float32)
    w[0, 1::2] = np.float32(1e-38)                   # alpha64 = 3.9e-41: subnormal in fp32
    w[1, 5] = np.float32(2.0 ** -149)                 # alpha64 rounds to 0 in fp32
    w[2, 7] = np.float32(255 * 2.0 ** -126)           # alpha = 2^-126 exactly
    q, a, z = oracle.quantize_minmax(w, 128)
    assert a[0, 0] == 1.0 and a[1, 0] == 1.0 and np.all(q[:2] == 0)
    assert z[0, 0] == 0.0 and z[1, 0] == 0.0
    assert a[2, 0] == np.float32(2.0 ** -126)
    assert q[2, 7] == 255 and np.count_nonzero(q[2]) == 1


def test_constant_vector():
    w = np.full((2, 128), -0.25, dtype=np.float32)
    w[1] = 0.0
    q, a, z = oracle.quantize_minmax(w, 128)
    assert np.all(q == 0) and np.all(a == 1.0)
    for r in (8, 4, 2):
        assert np.array_equal(oracle.dequant(q, a, z, 128, r), w.astype(np.float64))


# ---------------------------------------------------------------- packing

def test_hand_slice_indices():
    h = _hand()
    q = np.array([[int(v) for v in h["q"][0]]])
    for row in h["t"]:
        r = int(row[0])
        assert oracle.slice_index(q, r)[0].tolist() == [int(v) for v in row[1:]]


def test_hand_packed_words():
    for line in open(os.path.join(GOLDEN, "pack_layout.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split(";")
        vals = [int(v) for v in left.split()]
        r, t = vals[0], np.array([vals[1:]])
        assert oracle.pack_indices(t, r)[0].tolist() == [int(b, 16) for b in right.split()]
        assert oracle.unpack_indices(oracle.pack_indices(t, r), r, t.shape[1]).tolist() == t.tolist()


def test_hand_packed_split_planes():
    for line in open(os.path.join(GOLDEN, "pack_layout_split.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split(";")
        vals = [int(v) for v in left.split()]
        r, n, k = vals[:3]
        t = np.array(vals[3:]).reshape(n, k)
        got = oracle.pack_indices(t, r)
        assert got.shape == (n, k * r // 8)
        assert got.reshape(-1).tolist() == [int(b, 16) for b in right.split()]
        assert oracle.unpack_indices(got, r, k).tolist() == t.tolist()


def _golden_bitplane_cases():
    for line in open(os.path.join(GOLDEN, "pack_layout_bitplanes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split(";")
        head, codes = left.split("|")
        n, k = (int(v) for v in head.split())
        q = np.zeros((n, k), dtype=np.int64)
        for item in codes.split():
            where, v = item.split("=")
            row, cols = where.split(",")
            lo, _, hi = cols.partition("-")
            q[int(row), int(lo):int(hi or lo) + 1] = int(v)
        want = np.zeros((8, n, k // 8), dtype=np.uint8)
        for item in right.split():
            where, v = item.split("=")
            plane, byte = (int(x) for x in where.split(":"))
            want[plane].reshape(-1)[byte] = int(v, 16)
        yield q, want


def test_hand_packed_bitplanes():
    cases = list(_golden_bitplane_cases())
    assert len(cases) == 3
    for q, want in cases:
        got = oracle.pack_bitplanes(q)
        assert got.shape == want.shape and got.dtype == np.uint8
        assert np.array_equal(got, want)
        assert np.array_equal(oracle.unpack_bitplanes(got), q)


def test_bitplanes_roundtrip_and_shape_checks():
    rg = np.random.default_rng(77)
    q = rg.integers(0, 256, size=(3, 1024))
    pl = oracle.pack_bitplanes(q)
    assert pl.shape == (8, 3, 128)
    assert np.array_equal(oracle.unpack_bitplanes(pl), q)
    # plane p holds exactly the set bits p of the codes (population counts agree)
    for p in range(8):
        assert int(np.unpackbits(pl[p]).sum()) == int(((q >> p) & 1).sum())
    with pytest.raises(ValueError):
        oracle.pack_bitplanes(np.zeros((1, 256), dtype=np.int64))  # K not a multiple of 512


@pytest.mark.parametrize("extra", [False, True])
def test_slice_from_bitplanes_brute_force(extra):
    # every code at every r, through the planes (integer part + first discarded
    # bit) against Eq. 6 (clamped) or the errata Eq. 8 (unclamped) evaluated
    # as rounded quotients
    q = np.tile(ALL_CODES, 2).reshape(1, 512)
    pl = oracle.pack_bitplanes(q)
    for r in range(1, 9):
        t = oracle.slice_index_from_bitplanes(pl, r, extra=extra)
        if extra:
            want = oracle.slice_value_noclamp(q, r) // 2 ** (8 - r)
        else:
            want = oracle.slice_index(q, r)
        assert np.array_equal(t, want), r
    # the unclamped index exceeds 2^r - 1 for exactly 2^(7-r) codes (r < 8)
    for r in range(1, 8):
        t = oracle.slice_index_from_bitplanes(oracle.pack_bitplanes(ALL_CODES.reshape(1, 256).repeat(2, 1)), r, extra=True)
        assert int((t == 2 ** r).sum()) == 2 * 2 ** (7 - r)


def test_bitplane_bytes_read():
    # r + 1 planes of N*K/8 bytes; all eight at r = 8
    assert oracle.bitplane_bytes_read(14336, 3584, 2) == 3 * 14336 * 3584 // 8
    assert oracle.bitplane_bytes_read(14336, 3584, 4) == 5 * 14336 * 3584 // 8
    assert oracle.bitplane_bytes_read(14336, 3584, 8) == 14336 * 3584


@pytest.mark.parametrize("r", [3, 6])
def test_split_planes_roundtrip_and_sizes(r):
    rg = np.random.default_rng(40 + r)
    t = rg.integers(0, 2 ** r, size=(5, 128))
    p = oracle.pack_indices(t, r)
    assert p.shape == (5, 128 * r // 8)
    assert np.array_equal(oracle.unpack_indices(p, r, 128), t)
    with pytest.raises(ValueError):
        oracle.pack_indices(np.full((1, 64), 2 ** r), r)


def test_interpolated_precisions_sit_between_their_neighbours():
    # r = 3 and r = 6 are plain Eq. 6 slices: multiples of 2^(8-r) in range,
    # idempotent, and containing the value sets of the coarser slices
    for r in (3, 6):
        s = oracle.slice_value(ALL_CODES, r)
        assert np.all(s % 2 ** (8 - r) == 0) and s.min() == 0
        assert s.max() == (2 ** r - 1) * 2 ** (8 - r)
        assert np.array_equal(oracle.slice_value(s, r), s)
    assert set(oracle.slice_value(ALL_CODES, 2)) <= set(oracle.slice_value(ALL_CODES, 3))
    assert set(oracle.slice_value(ALL_CODES, 3)) <= set(oracle.slice_value(ALL_CODES, 6))
    # ties round up (the rule in words): q = 16 -> 32 at r = 3, q = 2 -> 4 at r = 6
    assert oracle.slice_value(np.array([16, 15, 2, 1]), 3).tolist() == [32, 0, 0, 0]
    assert oracle.slice_value(np.array([2, 1, 6, 5]), 6).tolist() == [4, 0, 8, 4]


@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_pack_bit_layout_and_roundtrip(r):
    rg = np.random.default_rng(r)
    t = rg.integers(0, 2 ** r, size=(3, 64))
    p = oracle.pack_indices(t, r)
    per_word = 32 // r
    for n in range(3):
        for w in range(64 // per_word):
            e = [int(v) for v in t[n, w * per_word:(w + 1) * per_word]]
            word = 0
            for j in range(per_word // 2):
                word += e[2 * j] * 2 ** (j * r) + e[2 * j + 1] * 2 ** (16 + j * r)
            assert p[n, 4 * w:4 * w + 4].tolist() == list(word.to_bytes(4, "little"))
    assert np.array_equal(oracle.unpack_indices(p, r, 64), t)


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch():
    rg = np.random.default_rng(3)
    v = np.concatenate([
        rg.standard_normal(20000).astype(np.float32) * 10.0 ** rg.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20,
                  3.0e38, 1e-40, -1e-39, 65504.0], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_from_float(v), want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    assert np.array_equal(oracle.float_from_bf16_bits(want), back)


# ---------------------------------------------------------------- the product

def test_hand_linear():
    h = _hand()
    w = np.array([[float(v) for v in h["w"][0]]], dtype=np.float32)
    q, a, z = oracle.quantize_minmax(w, 4)
    x = oracle.bf16_bits_from_float(np.ones((1, 4)))
    for r, num, den in h["y"]:
        y = oracle.linear(x, q, a, z, 4, int(r))
        # closed form with alpha = 2/255, z = 127.5; the fp32 storage of alpha
        # and z moves it by less than 3e-7
        assert abs(y[0, 0] - int(num) / int(den)) < 3e-7


def test_hand_linear_extra_precision():
    h = _hand()
    w = np.array([[float(v) for v in h["w"][0]]], dtype=np.float32)
    q, a, z = oracle.quantize_minmax(w, 4)
    x = oracle.bf16_bits_from_float(np.ones((1, 4)))
    for r, num, den in h["ye"]:
        y = oracle.linear_extra_precision(x, q, a, z, 4, int(r))
        assert abs(y[0, 0] - int(num) / int(den)) < 3e-7


@pytest.mark.parametrize("r", [2, 3, 4, 6, 8])
def test_overflow_lists_are_the_codes_above_the_last_midpoint(r):
    # the unclamped slice reaches 256 exactly for q >= 256 - 2^(7-r) (r < 8)
    rg = np.random.default_rng(70 + r)
    q = rg.integers(0, 256, size=(9, 192))
    q[2] = 255
    q[5] = 0
    row_ptr, col_idx = oracle.overflow_lists(q, r)
    assert row_ptr[0] == 0 and len(row_ptr) == 10
    for n in range(9):
        want = np.nonzero(q[n] >= 256 - 2 ** (7 - r))[0] if r < 8 else np.array([], int)
        assert col_idx[row_ptr[n]:row_ptr[n + 1]].tolist() == want.tolist()


def _exact_linear(x_bits, q, a, z, group, r, clamp=True):
    m, k = x_bits.shape
    n = q.shape[0]
    xs = [[Fraction(float(v)) for v in row] for row in oracle.float_from_bf16_bits(x_bits)]
    out = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                g = kk // group
                s = _slice_by_bits(int(q[j, kk]), r, clamp)
                acc += xs[i][kk] * (s - Fraction(float(z[j, g]))) * Fraction(float(a[j, g]))
            out[i, j] = float(acc)
    return out


@pytest.mark.parametrize("r", [8, 6, 4, 3, 2])
@pytest.mark.parametrize("group", [4, 8])
def test_linear_exact_rationals(r, group):
    rg = np.random.default_rng(100 + r + group)
    w = (rg.standard_normal((5, 8)) * 0.02).astype(np.float32)
    q, a, z = oracle.quantize_minmax(w, group)
    x = oracle.bf16_bits_from_float(rg.standard_normal((3, 8)))
    got = oracle.linear(x, q, a, z, group, r)
    want = _exact_linear(x, q, a, z, group, r)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("r", [6, 4, 3, 2])
def test_linear_extra_precision_exact_rationals(r):
    rg = np.random.default_rng(200 + r)
    w = (rg.standard_normal((6, 16)) * 0.02).astype(np.float32)
    w[:, 3] = 0.2  # a column at the top of every row's range: it rounds to the extra level
    q, a, z = oracle.quantize_minmax(w, 8)
    assert np.any(oracle.slice_value_noclamp(q, r) == 256)
    x = oracle.bf16_bits_from_float(rg.standard_normal((2, 16)))
    got = oracle.linear_extra_precision(x, q, a, z, 8, r)
    want = _exact_linear(x, q, a, z, 8, r, clamp=False)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- Mix'n'Match

def _const_layer(h_dim, f_dim, consts, r):
    layer = {"r": r}
    shapes = {"q": (h_dim, h_dim), "k": (4, h_dim), "v": (4, h_dim), "o": (h_dim, h_dim),
              "up": (f_dim, h_dim), "gate": (f_dim, h_dim), "down": (h_dim, f_dim)}
    for name, (n, k) in shapes.items():
        w = np.full((n, k), consts[name], dtype=np.float32)
        q, a, z = oracle.quantize_minmax(w, k)
        layer[name] = {"q": q, "alpha": a, "zero": z, "group": k}
    return layer


def _bf16(v):
    return torch.tensor(np.asarray(v, dtype=np.float64)).float().to(torch.bfloat16).double().numpy()


def test_rms_normalize_hand_values():
    """Hand values of the gain-free RMS normalization h / sqrt(mean(h^2)),
    per row: [3, 4] has mean square 12.5, so it maps to (sqrt(2)/5) [3, 4]
    (a sum instead of the mean would give [0.6, 0.8]); [0, 5] in a second
    row has the same mean square (rows are independent); [2, 2, 2, 2] maps to
    ones and [1, -1, 1, -1] to itself."""
    got = oracle.rms_normalize(np.array([[3.0, 4.0], [0.0, 5.0]]))
    c = np.sqrt(2.0) / 5.0
    assert np.allclose(got, [[3 * c, 4 * c], [0.0, 5 * c]], rtol=1e-15, atol=0)
    assert not np.allclose(got[0], [0.6, 0.8])
    assert np.array_equal(oracle.rms_normalize(np.array([[2.0, 2.0, 2.0, 2.0]])), [[1.0] * 4])
    assert np.array_equal(oracle.rms_normalize(np.array([[1.0, -1.0, 1.0, -1.0]])),
                          [[1.0, -1.0, 1.0, -1.0]])


def test_mixnmatch_constant_weights_closed_form():
    # Constant weight matrices quantize to code 0 with alpha = 1, z = -c, so
    # every slice dequantizes to c exactly and each linear returns
    # c * sum(input) in every output.  One layer, worked out directly.
    h_dim, f_dim = 8, 16
    consts = {"q": 0.125, "k": -0.5, "v": 0.25, "o": -0.0625, "up": 0.03125,
              "gate": 0.5, "down": 0.25}
    rg = np.random.default_rng(5)
    x = oracle.bf16_bits_from_float(rg.standard_normal((2, h_dim)))
    for r in (8, 4, 2):
        got = oracle.mixnmatch_forward([_const_layer(h_dim, f_dim, consts, r)], x)
        h0 = oracle.float_from_bf16_bits(x)
        a = _bf16(h0 / np.sqrt(np.mean(h0 ** 2, axis=1, keepdims=True)))
        sa = a.sum(axis=1, keepdims=True)
        qv, uv, gv = consts["q"] * sa, consts["up"] * sa, consts["gate"] * sa
        o = consts["o"] * h_dim * _bf16(qv)
        d = consts["down"] * f_dim * _bf16(uv * gv)
        assert np.allclose(got, h0 + o + d, rtol=1e-14, atol=1e-14)


def test_mixnmatch_zero_weights_is_identity():
    consts = {k: 0.0 for k in oracle.LAYER_LINEARS}
    rg = np.random.default_rng(6)
    x = oracle.bf16_bits_from_float(rg.standard_normal((1, 8)))
    layers = [_const_layer(8, 16, consts, r) for r in (8, 2, 4)]
    assert np.array_equal(oracle.mixnmatch_forward(layers, x), oracle.float_from_bf16_bits(x))


def test_mixnmatch_input_scale_property():
    # The normalization makes a layer's update o + d invariant to scaling its
    # input by a power of two, exactly.
    rg = np.random.default_rng(8)
    layer = {"r": 4}
    for name, (n, k) in {"q": (16, 16), "k": (4, 16), "v": (4, 16), "o": (16, 16),
                         "up": (32, 16), "gate": (32, 16), "down": (16, 32)}.items():
        q, a, z = oracle.quantize_minmax((rg.standard_normal((n, k)) * 0.02).astype(np.float32), k)
        layer[name] = {"q": q, "alpha": a, "zero": z, "group": k}
    x = oracle.bf16_bits_from_float(rg.standard_normal((1, 16)))
    x2 = oracle.bf16_bits_from_float(2.0 * oracle.float_from_bf16_bits(x))
    t1, t2 = [], []
    oracle.mixnmatch_forward([layer], x, t1)
    oracle.mixnmatch_forward([layer], x2, t2)
    assert np.array_equal(t1[0]["a_bits"], t2[0]["a_bits"])
    assert np.array_equal(t1[0]["o"], t2[0]["o"]) and np.array_equal(t1[0]["d"], t2[0]["d"])
    assert np.any(t1[0]["o"] != 0)


def test_effective_bits_of_the_stack_pattern():
    from nested_int_matmul_amd import inputs

    rs = inputs.mixnmatch_pattern(32)
    assert rs.count(8) == 16 and rs.count(4) == 11 and rs.count(2) == 5
    assert [i for i, r in enumerate(rs) if r == 2] == [10, 13, 16, 19, 22]
    layers = [{"r": r, **{nm: {"q": np.zeros((1, 1))} for nm in oracle.LAYER_LINEARS}} for r in rs]
    assert oracle.effective_bits(layers) == 5.6875


def test_oracle_and_library_share_no_code():
    root = os.path.dirname(GOLDEN)
    root = os.path.dirname(root)
    for dirpath, _, files in os.walk(os.path.join(root, "oracle")):
        for f in files:
            if f.endswith(".py"):
                src = open(os.path.join(dirpath, f)).read()
                assert "nested_int_matmul_amd" not in src.replace("(nested_int_matmul_amd)", "")
    for dirpath, _, files in os.walk(os.path.join(root, "nested_int_matmul_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src


# ---------------------------------------------------------------- decode MLP block

def test_mlp_activations_against_library_and_identities():
    from scipy import special

    g = np.linspace(-9.0, 9.0, 181)
    # SiLU is g * sigmoid(g) (scipy's logistic); GELU's tanh form is within
    # 1e-3 of the exact g * Phi(g) (scipy's erf)
    assert np.allclose(oracle.mlp_activation(g, "silu"), g * special.expit(g), rtol=1e-13, atol=1e-15)
    exact = 0.5 * g * (1.0 + special.erf(g / np.sqrt(2.0)))
    assert np.max(np.abs(oracle.mlp_activation(g, "gelu_tanh") - exact)) < 1e-3
    # both are x * (something in [0, 1]) with f(x) - f(-x) = x
    for act in ("silu", "gelu_tanh"):
        f = oracle.mlp_activation(g, act)
        assert np.allclose(f - oracle.mlp_activation(-g, act), g, rtol=0, atol=1e-12)
        assert oracle.mlp_activation(np.array([0.0]), act)[0] == 0.0
    assert np.array_equal(oracle.mlp_activation(g, "identity"), g)
    # the tanh form of GELU as written, where it does not cancel (g > -4)
    mid = g[g > -4.0]
    tanh_form = 0.5 * mid * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (mid + 0.044715 * mid ** 3)))
    assert np.allclose(oracle.mlp_activation(mid, "gelu_tanh"), tanh_form, rtol=1e-12, atol=1e-15)
    # far below, where tanh(z) rounds to -1: 1 + tanh(z) = 2 e^(2z) (1 - e^(2z) + ...),
    # so the value tends to g e^(2z) (not to the zero the tanh form gives in float64)
    far = np.array([-8.0, -9.0, -10.0])
    tail = oracle.mlp_activation(far, "gelu_tanh")
    z = np.sqrt(2.0 / np.pi) * (far + 0.044715 * far ** 3)
    assert np.all(1.0 + np.tanh(z) == 0.0)
    assert np.allclose(tail, far * np.exp(2.0 * z), rtol=1e-9, atol=0)
    with pytest.raises(ValueError):
        oracle.mlp_activation(g, "relu")


@pytest.mark.parametrize("act", ["identity", "silu", "gelu_tanh"])
def test_mlp_decode_constant_weights_closed_form(act):
    # constant matrices dequantize to their constant exactly (code 0, alpha 1,
    # z = -c), so u = c_u * sum(x), g = c_g * sum(x) in every output, and every
    # output of down is c_d * F * bf16(act(g) * u)
    h_dim, f_dim = 8, 24
    rg = np.random.default_rng(9)
    x = oracle.bf16_bits_from_float(rg.standard_normal((3, h_dim)))
    consts = {"up": 0.375, "gate": -0.75, "down": 0.0625}
    mats = {}
    for name, (n, k) in {"up": (f_dim, h_dim), "gate": (f_dim, h_dim), "down": (h_dim, f_dim)}.items():
        q, a, z = oracle.quantize_minmax(np.full((n, k), consts[name], dtype=np.float32), k)
        mats[name] = {"q": q, "alpha": a, "zero": z, "group": k}
    sx = oracle.float_from_bf16_bits(x).sum(axis=1, keepdims=True)
    gv = consts["gate"] * sx
    if act == "silu":
        gv = gv / (1.0 + np.exp(-gv))
    elif act == "gelu_tanh":
        from scipy import special
        gv = 0.5 * gv * (1.0 + np.tanh(np.sqrt(2 / np.pi) * (gv + 0.044715 * gv ** 3)))
        assert np.allclose(gv, 0.5 * (consts["gate"] * sx) * (1 + special.erf(consts["gate"] * sx / np.sqrt(2))), atol=1e-3)
        assert np.all(np.abs(consts["gate"] * sx) < 5)  # the tanh form has no cancellation here
    for r in (8, 4, 2):
        got = oracle.mlp_decode(x, mats["up"], mats["gate"], mats["down"], r, act)
        want = consts["down"] * f_dim * _bf16(gv * consts["up"] * sx)
        assert got.shape == (3, h_dim)
        assert np.allclose(got, np.broadcast_to(want, got.shape), rtol=1e-14, atol=1e-14)


def test_mlp_decode_is_the_mixnmatch_gated_branch():
    # with the identity activation the block is the u * g -> down branch of a
    # Mix'n'Match layer fed the same bf16 input
    rg = np.random.default_rng(10)
    layer = {"r": 4}
    for name, (n, k) in {"q": (16, 16), "k": (4, 16), "v": (4, 16), "o": (16, 16),
                         "up": (32, 16), "gate": (32, 16), "down": (16, 32)}.items():
        q, a, z = oracle.quantize_minmax((rg.standard_normal((n, k)) * 0.02).astype(np.float32), k)
        layer[name] = {"q": q, "alpha": a, "zero": z, "group": k}
    x = oracle.bf16_bits_from_float(rg.standard_normal((2, 16)))
    tr = []
    oracle.mixnmatch_forward([layer], x, tr)
    y = oracle.mlp_decode(tr[0]["a_bits"], layer["up"], layer["gate"], layer["down"], 4)
    assert np.array_equal(y, tr[0]["d"])
