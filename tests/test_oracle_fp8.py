"""Pins of the oracle's fp8 (OCP FP8 E4M3) cache type against things other than itself:
hand-worked values (tests/golden/fp8_hand_worked.txt), torch's own float8_e4m3fn type (a
library routine) for decoding every code and for casting every finite bf16 value it casts
without overflow, the saturation reading beyond that range, and attention over fp8 rows
against the textbook bf16 attention where the rows lie on the fp8 grid.

Cache type from "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com),
section "Getting a server up: the commands in the README" (fp8 among the KV cache types; its
compression table gives fp8 2x against BF16)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_hand_worked.txt")


def _golden(kind):
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] != kind:
                continue
            rows.append(dict(p.split("=", 1) for p in parts[1:]))
    assert rows, kind
    return rows


@pytest.mark.parametrize("row", _golden("value"), ids=lambda r: r["code"])
def test_value_hand_worked(row):
    assert oracle.fp8_e4m3_value(int(row["code"], 16)) == float(row["x"])


@pytest.mark.parametrize("row", _golden("encode"), ids=lambda r: r["x"])
def test_encode_hand_worked(row):
    assert int(oracle.fp8_e4m3_encode(float(row["x"]))) == int(row["code"], 16)


def test_every_code_decodes_as_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))   # 0x80 is -0.0
    assert np.sum(np.isnan(got)) == 2 and np.nanmax(np.abs(got)) == 448.0


def test_every_finite_bf16_casts_as_torch_below_the_overflow_range():
    """torch's cast rounds to nearest-even like the reading, but returns NaN past the range
    (from 464 on), where the reading saturates; below that the two agree on every bf16."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(bits)
    keep = np.isfinite(x) & (np.abs(x) < 464.0)
    x = x[keep]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.fp8_e4m3_encode(x)
    assert np.array_equal(got, want)


def test_saturation_past_448():
    x = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e4, 3.0e38])
    assert np.all(oracle.fp8_e4m3_encode(x) == 0x7E)
    assert np.all(oracle.fp8_e4m3_encode(-x) == 0xFE)


def test_codes_round_trip_and_the_error_is_within_half_a_step():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_value(codes)), codes)
    r = np.random.default_rng(5)
    x = np.concatenate([r.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0, 120.0)])
    x = x[np.abs(x) <= 448.0]                 # beyond: saturation, tested above
    c = oracle.fp8_e4m3_encode(x)
    v = oracle.fp8_e4m3_value(c)
    # step of the binade of |x|: 2^(e-3) for normal values, 2^-9 in the subnormal range
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
    step = np.exp2(e - 3)
    assert np.all(np.abs(x - v) <= step / 2 + 1e-300)
    assert np.all(np.sign(v[v != 0]) == np.sign(x[v != 0]))


def test_non_finite_input_is_rejected():
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode(np.array([1.0, np.nan]))


def test_fp8_attention_equals_bf16_attention_on_grid_values():
    """Rows whose bf16 values are E4M3 values are cached exactly, so fp8 attention must equal
    the textbook bf16 attention over the same rows (which is pinned to float64 softmax)."""
    r = np.random.default_rng(9)
    L, hkv, hq = 37, 2, 8
    on_grid = oracle.fp8_e4m3_value(np.array([c for c in range(256) if c & 0x7F != 0x7F]))
    on_grid = on_grid[np.abs(on_grid) <= 8]
    k = workloads.round_to_bf16_bits(r.choice(on_grid, size=(L, hkv, 128)).astype(np.float32))
    v = workloads.round_to_bf16_bits(r.choice(on_grid, size=(L, hkv, 128)).astype(np.float32))
    q = workloads.round_to_bf16_bits(r.standard_normal((hq, 128)).astype(np.float32))
    got, (kf, vf) = oracle.decode_sequence(oracle.FP8, q, k, v, 0.1)
    want, _ = oracle.decode_sequence(0, q, k, v, 0.1)
    assert np.max(np.abs(got - want)) < 1e-12
    assert np.array_equal(oracle.fp8_e4m3_value(kf), oracle.bf16_bits_to_f32(k).astype(np.float64))


def test_fp8_attention_error_against_bf16_is_small():
    """Quality sanity (the page's "near-lossless" column): N(0,1) rows, 3 significant bits."""
    r = np.random.default_rng(11)
    L, hkv, hq = 200, 2, 8
    k = workloads.round_to_bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    v = workloads.round_to_bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    q = workloads.round_to_bf16_bits(r.standard_normal((hq, 128)).astype(np.float32))
    got, _ = oracle.decode_sequence(oracle.FP8, q, k, v, 1 / np.sqrt(128))
    want, _ = oracle.decode_sequence(0, q, k, v, 1 / np.sqrt(128))
    err = np.max(np.abs(got - want))
    assert 0 < err < 0.05, err
