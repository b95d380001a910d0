"""Pins for the oracle's rotation, quantizer and packer (CPU only).

Each test checks the oracle against something other than itself: dense Hadamard
matrices (scipy's Sylvester construction and the popcount definition), exact integer
arithmetic, closed forms, binary16 facts and hand-worked values (tests/golden/).
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_hand_worked.txt")


def _golden(kind):
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *fields = line.split()
            if tag != kind:
                continue
            rows.append(dict(kv.split("=", 1) for kv in fields))
    assert rows, kind
    return rows


# ------------------------------------------------------------------------------------
# rotation
# ------------------------------------------------------------------------------------
def test_c_constant_is_nearest_fp32_to_inv_sqrt128():
    c = oracle.C_F32
    assert c.view(np.uint32) == 0x3DB504F3
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(128).sqrt()
    c_exact = Decimal(Fraction(float(c)).numerator) / Decimal(Fraction(float(c)).denominator)
    ulp = Decimal(2) ** -27          # c is in [2^-4, 2^-3): 23 fraction bits -> 2^-27
    assert abs(c_exact - exact) <= ulp / 2


def test_hadamard_matches_sylvester_construction():
    H = oracle.hadamard_matrix()
    ref = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128)
    assert np.array_equal(H, ref)
    # natural order: row 1 alternates +,-; row 64 is + for k < 64 and - after
    assert np.all(np.sign(H[1]) == np.tile([1, -1], 64))
    assert np.all(np.sign(H[64]) == np.repeat([1, -1], 64))


def test_hadamard_is_symmetric_orthonormal():
    H = oracle.hadamard_matrix()
    assert np.array_equal(H, H.T)
    assert np.max(np.abs(H @ H.T - np.eye(128))) < 1e-14
    assert np.all(np.abs(np.abs(H) - 1 / math.sqrt(128)) < 1e-17)


def test_fwht_matches_dense_matrix_float64():
    x = np.random.default_rng(1).standard_normal((17, 128))
    dense = x @ scipy.linalg.hadamard(128).T.astype(np.float64)
    assert np.max(np.abs(oracle.fwht(x) - dense)) < 1e-12


def test_fwht_exact_on_integers():
    x = np.random.default_rng(2).integers(-1000, 1001, size=(9, 128))
    exact = x @ scipy.linalg.hadamard(128).T.astype(np.int64)   # |entries| <= 128000
    got = oracle.fwht(x.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), exact)


def test_fwht_float32_stage_order_matches_scalar_definition():
    """The vectorised butterflies equal a scalar loop over stages h = 1, 2, ..., 64 in
    fp32, pair (i, i+h) -> (a+b, a-b), bit for bit (rounding order is part of the codec)."""
    rows = np.random.default_rng(3).standard_normal((4, 128)).astype(np.float32) * 7
    got = oracle.fwht(rows)
    for r, g in zip(rows, got):
        v = [np.float32(t) for t in r]
        h = 1
        while h < 128:
            for i in range(128):
                if i & h == 0:
                    a, b = v[i], v[i + h]
                    v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
            h *= 2
        assert np.array_equal(np.array(v, dtype=np.float32).view(np.uint32), g.view(np.uint32))


def test_fwht_float32_close_to_dense():
    x = np.random.default_rng(4).standard_normal((32, 128)).astype(np.float32)
    ref = x.astype(np.float64) @ oracle.hadamard_matrix().T
    got = oracle.rotate_f32(x).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 2e-6 * np.max(np.abs(ref))


def test_fwht_twice_is_identity():
    x = np.random.default_rng(5).standard_normal((3, 128))
    y = oracle.fwht(oracle.fwht(x)) / 128.0
    assert np.max(np.abs(y - x)) < 1e-13


def test_rotation_closed_forms():
    e0 = np.zeros(128, np.float32)
    e0[0] = 1
    assert np.all(oracle.rotate_f32(e0) == oracle.C_F32)
    ones = np.ones(128, np.float32)
    r = oracle.rotate_f32(ones)
    assert abs(float(r[0]) - math.sqrt(128)) < 2e-6
    assert np.all(r[1:] == 0)


def test_rotation_preserves_dot_products():
    g = np.random.default_rng(6)
    q, k = g.standard_normal(128), g.standard_normal(128)
    H = oracle.hadamard_matrix()
    assert abs((H @ q) @ (H @ k) - q @ k) < 1e-12 * (abs(q @ k) + 1)
    fq = oracle.fwht(q) / math.sqrt(128)
    fk = oracle.fwht(k) / math.sqrt(128)
    assert abs(fq @ fk - q @ k) < 1e-12 * (abs(q @ k) + 1)


# ------------------------------------------------------------------------------------
# binary16 conversion and the quantizer
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("row", _golden("fp16"), ids=lambda r: r["value"])
def test_fp16_rne_facts(row):
    v = np.float32(float(row["value"]))
    got = oracle.f32_to_f16_saturating(np.array([v]))[0].view(np.uint16)
    assert got == int(row["bits"], 16)


def test_fp16_saturates():
    got = oracle.f32_to_f16_saturating(np.array([70000.0, 65519.0, 1e30], np.float32))
    assert np.all(got.view(np.uint16) == 0x7BFF)


@pytest.mark.parametrize("row", _golden("quantize"), ids=lambda r: f"b{r['bits']}-{r['s16']}")
def test_quantizer_hand_worked(row):
    bits = int(row["bits"])
    vals = [float(t) for t in row["x"].split(",")]
    x = np.zeros(128, np.float32)
    x[: len(vals)] = vals
    codes, s16 = oracle.quantize_rotated(x[None], bits)
    want = [int(t) for t in row["codes"].split(",")]
    assert s16[0].view(np.uint16) == int(row["s16"], 16)
    assert list(codes[0, : len(want)]) == want
    assert np.all(codes[0, len(want):] == 0)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_quantizer_round_trip_on_grid(bits):
    g = np.random.default_rng(10 + bits)
    qmax = oracle.QMAX[bits]
    for _ in range(50):
        s = np.float16(g.uniform(1e-3, 100.0))
        c = g.integers(-qmax, qmax + 1, size=128)
        c[g.integers(128)] = qmax * (1 if g.integers(2) else -1)
        x = (np.float32(s) * c.astype(np.float32))
        codes, s16 = oracle.quantize_rotated(x[None], bits)
        assert s16[0] == s
        assert np.array_equal(codes[0], c.astype(np.int8))


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_quantizer_error_bound_and_full_range(bits):
    g = np.random.default_rng(20 + bits)
    x = (g.standard_normal((500, 128)) * g.uniform(0.01, 50, size=(500, 1))).astype(np.float32)
    codes, s16 = oracle.quantize_rotated(x, bits)
    s = s16.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - s * codes)
    assert np.all(err <= s / 2 + 1e-12)
    assert np.all(np.max(np.abs(codes), axis=1) == oracle.QMAX[bits])
    assert codes.min() >= -oracle.QMAX[bits]


def test_quantizer_zero_row():
    codes, s16 = oracle.quantize_rotated(np.zeros((2, 128), np.float32), 4)
    assert np.all(s16 == 0) and np.all(codes == 0)


def test_quantizer_rejects_nonfinite():
    x = np.zeros((1, 128), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_rotated(x, 4)


def test_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    got = oracle.bf16_bits_to_f32(bits)
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == np.float32(3.140625)
    assert got[3] == np.float32(2.0 ** -133)        # smallest bf16 subnormal
    assert got[4] == np.float32(3.3895313892515355e38)


def test_rotation_spreads_outliers():
    """The pages' reason for the rotation: outlier channels inflate the absmax of an
    unrotated row. Reconstruction error with the rotation is far below without it."""
    g = np.random.default_rng(30)
    x = g.standard_normal((2000, 128)).astype(np.float32)
    x[:, [5, 40, 77, 100]] *= 20
    c_rot, s_rot = oracle.quantize_rotated(oracle.rotate_f32(x), 4)
    rec_rot = oracle.dequantize(c_rot, s_rot) @ oracle.hadamard_matrix()   # H symmetric
    c_raw, s_raw = oracle.quantize_rotated(x, 4)
    rec_raw = oracle.dequantize(c_raw, s_raw)
    mse_rot = np.mean((rec_rot - x) ** 2)
    mse_raw = np.mean((rec_raw - x) ** 2)
    assert mse_rot < 0.5 * mse_raw


# ------------------------------------------------------------------------------------
# packing
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("row", _golden("pack"), ids=lambda r: f"b{r['bits']}")
def test_pack_hand_worked(row):
    bits = int(row["bits"])
    codes = np.zeros(128, np.int8)
    vals = [int(t) for t in row["codes"].split(",")]
    codes[: len(vals)] = vals
    packed = oracle.pack_codes(codes[None], bits)[0]
    want = [int(t, 16) for t in row["bytes"].split(",")]
    assert packed.shape == (16 * bits,)
    assert list(packed[: len(want)]) == want
    assert np.all(packed[len(want):] == 0)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_pack_matches_bigint_bitstream(bits):
    g = np.random.default_rng(40 + bits)
    q = oracle.QMAX[bits]
    codes = g.integers(-q, q + 1, size=(20, 128))
    packed = oracle.pack_codes(codes, bits)
    for c, p in zip(codes, packed):
        stream = 0
        for d, v in enumerate(c):
            stream |= (int(v) & ((1 << bits) - 1)) << (bits * d)
        assert int.from_bytes(bytes(p), "little") == stream


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_pack_unpack_exhaustive(bits):
    vals = np.arange(-(1 << (bits - 1)), 1 << (bits - 1))
    for shift in range(len(vals)):
        row = np.roll(np.resize(vals, 128), shift)        # every value at every position
        got = oracle.unpack_codes(oracle.pack_codes(row[None], bits), bits)[0]
        assert np.array_equal(got, row.astype(np.int8))


def test_row_bytes_reproduce_capacity_ratio():
    """66 bytes per turbo4 row (64 code bytes + fp16 scale) against 256 bytes of bf16
    reproduces the xInfer page's 7 GB example, 112k -> 434k tokens (section "What
    actually sits between the request and the tokens"), to within 0.2%."""
    assert oracle.row_bytes(4) == 66
    assert abs(256 / oracle.row_bytes(4) / (434 / 112) - 1) < 2e-3
    assert oracle.row_bytes(8) == 130 and oracle.row_bytes(3) == 50
