"""Pins of the oracle's chunked prefill (infero landing page, section "Beyond plain text decode",
item "Continuous batching": prefill fills what a step leaves and may split across steps):
against a dense causal-masked attention written as one matrix product per head (a different
formulation from the oracle's per-query loop), a one-token chunk against decode, and causality
(rows past a query's position cannot change it)."""
import numpy as np
import pytest

import oracle
import workloads


def _rows(seed, n, h):
    r = np.random.default_rng(seed)
    return workloads.round_to_bf16_bits(r.standard_normal((n, h, 128)).astype(np.float32))


def test_bf16_prefill_equals_dense_causal_attention():
    start, c, hq, hkv = 29, 11, 8, 2
    q = _rows(1, c, hq)
    k, v = _rows(2, start + c, hkv), _rows(3, start + c, hkv)
    scale = 0.11
    got = oracle.prefill_sequence(0, q, k, v, start, scale)
    qf = oracle.bf16_bits_to_f32(q).astype(np.float64)
    kf = oracle.bf16_bits_to_f32(k).astype(np.float64)
    vf = oracle.bf16_bits_to_f32(v).astype(np.float64)
    qpos = start + np.arange(c)[:, None]
    kpos = np.arange(start + c)[None, :]
    mask = kpos <= qpos                                        # [c, L]
    g = hq // hkv
    for j in range(hq):
        s = scale * qf[:, j, :] @ kf[:, j // g, :].T            # [c, L]
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        want = (p / p.sum(axis=1, keepdims=True)) @ vf[:, j // g, :]
        assert np.max(np.abs(got[:, j, :] - want)) < 1e-12


@pytest.mark.parametrize("dtype", [4, 3, 8, 2, oracle.FP8])
def test_one_token_chunk_is_decode(dtype):
    L, hq, hkv = 40, 4, 2
    q = _rows(4, 1, hq)
    k, v = _rows(5, L, hkv), _rows(6, L, hkv)
    got = oracle.prefill_sequence(dtype, q, k, v, L - 1, 0.09)
    want, _ = oracle.decode_sequence(dtype, q[0], k, v, 0.09)
    assert np.array_equal(got[0], want)


@pytest.mark.parametrize("dtype", [0, 4, oracle.FP8])
def test_rows_past_a_query_do_not_change_it(dtype):
    start, c, hq, hkv = 10, 6, 4, 1
    q = _rows(7, c, hq)
    k, v = _rows(8, start + c, hkv), _rows(9, start + c, hkv)
    a = oracle.prefill_sequence(dtype, q, k, v, start, 0.09)
    k2, v2 = k.copy(), v.copy()
    k2[start + 3:] = _rows(10, c - 3, hkv)
    v2[start + 3:] = _rows(11, c - 3, hkv)
    b = oracle.prefill_sequence(dtype, q, k2, v2, start, 0.09)
    assert np.array_equal(a[:3], b[:3])           # queries at positions <= start + 2
    assert not np.array_equal(a[3:], b[3:])


def test_chunk_split_across_steps_equals_one_chunk():
    """Two chunks (the second attending to the first through the cache) equal one long chunk."""
    start, c, hq, hkv = 5, 12, 4, 2
    q = _rows(12, c, hq)
    k, v = _rows(13, start + c, hkv), _rows(14, start + c, hkv)
    whole = oracle.prefill_sequence(4, q, k, v, start, 0.09)
    first = oracle.prefill_sequence(4, q[:7], k[:start + 7], v[:start + 7], start, 0.09)
    second = oracle.prefill_sequence(4, q[7:], k, v, start + 7, 0.09)
    assert np.array_equal(np.concatenate([first, second]), whole)
