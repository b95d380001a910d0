"""Pins for the oracle's decode attention (CPU only).

Checked against textbook softmax attention written with scipy.special.softmax, against
attention in the original (unrotated) space over rows reconstructed with the dense
Hadamard matrix, and against closed-form special cases.
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle
import workloads


def _bits(x):
    return workloads.round_to_bf16_bits(np.asarray(x, np.float32))


def _textbook(q, k, v, scale, g):
    """softmax(scale * q K^T) V per head, vectorised, float64."""
    hq = q.shape[0]
    kk = np.repeat(k.transpose(1, 0, 2), g, axis=0)       # [Hq, L, D]
    vv = np.repeat(v.transpose(1, 0, 2), g, axis=0)
    z = scale * np.einsum("hd,hld->hl", q, kk)
    p = scipy.special.softmax(z, axis=-1)
    return np.einsum("hl,hld->hd", p, vv).reshape(hq, -1)


@pytest.mark.parametrize("L,hq,hkv", [(1, 4, 4), (37, 8, 2), (300, 10, 2)])
def test_bf16_mode_is_textbook_attention(L, hq, hkv):
    g = np.random.default_rng(L)
    q, k, v = _bits(g.standard_normal((hq, 128))), _bits(g.standard_normal((L, hkv, 128)) * 2), \
        _bits(g.standard_normal((L, hkv, 128)))
    scale = 1 / np.sqrt(128)
    got = oracle.decode_attention_bf16(q, k, v, scale)
    f = oracle.bf16_bits_to_f32
    want = _textbook(f(q).astype(np.float64), f(k).astype(np.float64), f(v).astype(np.float64),
                     scale, hq // hkv)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_turbo_equals_attention_over_unrotated_reconstruction(bits):
    """out = H softmax(s q'K'^T) V' with q' = Hq must equal plain attention of q over
    the rows rotated back to the original space, K'H and V'H (H symmetric orthonormal)."""
    g = np.random.default_rng(100 + bits)
    L, hq, hkv = 50, 6, 3
    q = _bits(g.standard_normal((hq, 128)))
    k = _bits(g.standard_normal((L, hkv, 128)) * 3)
    v = _bits(g.standard_normal((L, hkv, 128)))
    kc, ks = oracle.quantize_rows_bf16(k, bits)
    vc, vs = oracle.quantize_rows_bf16(v, bits)
    scale = 0.1
    got = oracle.decode_attention_turbo(q, kc, ks, vc, vs, scale)
    Hs = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128)
    k_back = (kc.astype(np.float64) * ks.astype(np.float64)[..., None]) @ Hs
    v_back = (vc.astype(np.float64) * vs.astype(np.float64)[..., None]) @ Hs
    want = _textbook(oracle.bf16_bits_to_f32(q).astype(np.float64), k_back, v_back, scale,
                     hq // hkv)
    assert np.max(np.abs(got - want)) < 1e-12


def test_gqa_group_mapping():
    """Query head j reads kv head j // g: heads of one group agree with single-head runs
    on their own kv head, and kv heads are made very different so a wrong map shows."""
    g = np.random.default_rng(7)
    L, hq, hkv = 20, 8, 2
    q = _bits(g.standard_normal((hq, 128)))
    k = _bits(g.standard_normal((L, hkv, 128)))
    v = _bits(np.stack([np.full((L, 128), 5.0), np.full((L, 128), -5.0)], axis=1)
              + g.standard_normal((L, hkv, 128)) * 0.1)
    out = oracle.decode_attention_bf16(q, k, v, 0.2)
    for j in range(hq):
        one = oracle.decode_attention_bf16(q[j:j + 1], k[:, j // 4:j // 4 + 1], v[:, j // 4:j // 4 + 1], 0.2)
        assert np.max(np.abs(out[j] - one[0])) < 1e-13
    assert np.all(out[:4] > 4) and np.all(out[4:] < -4)


def test_empty_context_gives_zeros():
    q = _bits(np.ones((4, 128)))
    e = np.zeros((0, 2, 128), np.uint16)
    assert np.all(oracle.decode_attention_bf16(q, e, e, 1.0) == 0)
    kc = np.zeros((0, 2, 128), np.int8)
    ks = np.zeros((0, 2), np.float16)
    assert np.all(oracle.decode_attention_turbo(q, kc, ks, kc, ks, 1.0) == 0)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_single_token_returns_its_value(bits):
    """With one cached token the softmax weight is 1, so out = H (s_v c_v)."""
    g = np.random.default_rng(200 + bits)
    q = _bits(g.standard_normal((2, 128)))
    k = _bits(g.standard_normal((1, 1, 128)))
    v = _bits(g.standard_normal((1, 1, 128)))
    out, (kc, ks, vc, vs) = oracle.decode_sequence(bits, q, k, v, 0.5)
    want = scipy.linalg.hadamard(128) @ (vc[0, 0].astype(np.float64) * float(vs[0, 0])) / np.sqrt(128)
    assert np.max(np.abs(out - want[None])) < 1e-13


def test_identical_keys_average_values():
    g = np.random.default_rng(9)
    L = 33
    q = _bits(g.standard_normal((3, 128)))
    k = np.repeat(_bits(g.standard_normal((1, 1, 128))), L, axis=0)
    v = _bits(g.standard_normal((L, 1, 128)))
    out = oracle.decode_attention_bf16(q, k, v, 1.0)
    mean = oracle.bf16_bits_to_f32(v)[:, 0].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out - mean[None])) < 1e-13


def test_token_order_does_not_matter():
    """Attention is a function of the set of cached tokens; the page order in which a
    paged cache stores them cannot change the result."""
    g = np.random.default_rng(11)
    L = 64
    q = _bits(g.standard_normal((4, 128)))
    k = _bits(g.standard_normal((L, 2, 128)) * 4)
    v = _bits(g.standard_normal((L, 2, 128)))
    perm = g.permutation(L)
    a, _ = oracle.decode_sequence(4, q, k, v, 0.125)
    b, _ = oracle.decode_sequence(4, q, k[perm], v[perm], 0.125)
    assert np.max(np.abs(a - b)) < 1e-12


def test_quality_orders_by_code_width():
    """Quality sanity on the 8B-class distribution (8 outlier channels x30 in K): turbo8
    stays within a few percent of the unquantized cache, and error grows as codes get
    narrower (turbo8 < turbo4 < turbo3 < turbo2). Reported behaviour, not a parity bar."""
    W = workloads.config(2, batch=1, context_scale=1 / 32)
    q = W.q_bits()[0]
    k, v = W.kv_bits(0)
    ref, _ = oracle.decode_sequence(0, q, k, v, W.softmax_scale)
    err = {b: np.mean(np.abs(oracle.decode_sequence(b, q, k, v, W.softmax_scale)[0] - ref))
           for b in (8, 4, 3, 2)}
    assert err[8] < 0.03 * np.mean(np.abs(ref))
    assert err[8] < err[4] < err[3] < err[2]


def test_softmax_stable_for_large_logits():
    q = _bits(np.full((1, 128), 8.0))
    k = _bits(np.full((3, 1, 128), 8.0))
    v = _bits(np.arange(3 * 128).reshape(3, 1, 128) % 7)
    out = oracle.decode_attention_bf16(q, k, v, 1.0)          # logits ~ 8192: no overflow
    assert np.all(np.isfinite(out))
