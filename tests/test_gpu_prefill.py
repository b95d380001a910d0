"""GPU parity of the chunked prefill (xq_paged_prefill_attention) against the oracle's
prefill_sequence: a chunk's queries attending causally to the sequence's cache, its own rows
included (infero landing page, section "Beyond plain text decode", item "Continuous batching").
Bar: within 2e-3 max-abs of the float64 oracle; with fixed partitions, query i bitwise equals
the decode of the same sequence cut at start + i + 1 tokens."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import dominant_queries, fill, make_cache, to_dev, upload_tables

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _case(*a):
    print("CASE", *a, flush=True)


def _setup(dtype, start, chunk, hq, hkv, ps, cfg):
    W = workloads.make(f"prefill-{dtype}-{ps}", cfg, dtype, [start + chunk], hq, hkv, ps)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    kv = {0: W.kv_bits(0)}
    fill(cache, W, bt, kv=kv)                  # the prefix and the chunk's own rows
    r = np.random.default_rng(cfg)
    q = workloads.round_to_bf16_bits(r.standard_normal((chunk, hq, 128)).astype(np.float32))
    return W, cache, bt, kv, q


@pytest.mark.parametrize("dtype,start,chunk,hq,hkv,ps", [
    (4, 0, 77, 8, 2, 16), (4, 100, 77, 16, 8, 16), (4, 333, 40, 32, 8, 64), (8, 50, 33, 32, 8, 16),
    (3, 200, 65, 40, 8, 64), (2, 17, 50, 8, 8, 16), (0, 90, 45, 8, 2, 32), (16, 120, 60, 32, 8, 16),
    (4, 700, 1, 8, 2, 16), (4, 37, 50, 8, 8, 16), (3, 64, 29, 40, 8, 64), (8, 5, 70, 16, 1, 32),
    (0, 30, 47, 24, 8, 16), (16, 3, 61, 8, 1, 16), (4, 3000, 20, 32, 8, 16), (4, 1, 300, 40, 8, 32)])
def test_prefill_matches_oracle(dtype, start, chunk, hq, hkv, ps):
    _case("prefill", dtype, start, chunk, hq, hkv, ps)
    W, cache, bt, kv, q = _setup(dtype, start, chunk, hq, hkv, ps, 800 + dtype)
    k, v = kv[0]
    want = oracle.prefill_sequence(dtype, q, k, v, start, W.softmax_scale)
    for splits in (0, 3):
        out = cache.prefill(to_dev(q), bt[0], start, W.softmax_scale, splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = np.max(np.abs(got - want), axis=(1, 2))
        assert np.all(err <= TOL), f"splits {splits}: worst query {int(np.argmax(err))} err {err.max():.3e}"


@pytest.mark.parametrize("dtype,hq,hkv,ps", [(8, 32, 8, 16), (4, 32, 8, 16), (3, 40, 8, 64), (2, 8, 8, 16),
                                            (4, 16, 1, 32), (16, 32, 8, 16)])
def test_prefill_queries_with_a_dominant_rotated_element(dtype, hq, hkv, ps):
    """Chunk queries whose rotation has one dominant element (constant offsets 3 and 30, Hadamard
    rows): a prefill unit packs up to 16 (query, head) columns, so its queries are prepared in two
    passes of eight rows; every query against the oracle."""
    _case("prefill-dominant", dtype, hq, hkv, ps)
    start, chunk = 100, 40
    W = workloads.make(f"prefill-dom-{dtype}", 880 + dtype, dtype, [start + chunk], hq, hkv, ps,
                       outlier_channels=8, outlier_scale=30.0)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    k, v = W.kv_bits(0)
    fill(cache, W, bt, kv={0: (k, v)})
    r = np.random.default_rng(dtype)
    q0 = workloads.round_to_bf16_bits(r.standard_normal((chunk, hq, 128)).astype(np.float32))
    for kind in (3, 30, "had"):
        q = dominant_queries(q0, kind, seed=dtype)
        want = oracle.prefill_sequence(dtype, q, k, v, start, W.softmax_scale)
        for splits in (0, 3):
            out = cache.prefill(to_dev(q), bt[0], start, W.softmax_scale, splits)
            torch.cuda.synchronize()
            err = np.max(np.abs(out.cpu().numpy().astype(np.float64) - want), axis=(1, 2))
            assert np.all(err <= TOL), f"query {kind} splits {splits}: worst {int(np.argmax(err))} err {err.max():.3e}"


@pytest.mark.parametrize("hq,hkv,exact", [(16, 1, True), (16, 8, False), (32, 8, False)])
def test_prefill_rows_equal_decode_cut_at_their_position(hq, hkv, exact):
    """Query i of a chunk against a decode of the same sequence with context start + i + 1, both
    with fixed partitions. With 16 query heads per kv head a prefill unit holds one query, in the
    decode's layout, so the two are bitwise equal; with fewer, the prefill packs 16 / g queries
    into a unit's 16 columns where the decode uses its paired layout, and the sums are rounded in
    another order."""
    _case("prefill-vs-decode", hq, hkv)
    dtype, start, chunk = 4, 300, 40
    W, cache, bt, kv, q = _setup(dtype, start, chunk, hq, hkv, 16, 820)
    qd = to_dev(q)
    out = cache.prefill(qd, bt[0], start, W.softmax_scale, -256)
    rows = [0, 1, 17, chunk - 1]
    cl = to_dev(np.array([start + i + 1 for i in rows], np.int32))
    btr = bt[0:1].repeat(len(rows), 1).contiguous()
    dec = cache.decode(qd[rows].contiguous(), btr, cl, start + chunk, W.softmax_scale, -256)
    torch.cuda.synchronize()
    for j, i in enumerate(rows):
        a, d = out[i].cpu(), dec[j].cpu()
        if exact:
            assert torch.equal(a, d), f"query {i}"
        else:
            assert float((a - d).abs().max()) < 1e-4, f"query {i}"


def test_prefill_full_chunk_of_the_mixed_step():
    """The mixed step's 2,048-token chunk (32q/8kv, turbo4, page 16, pages shuffled over the
    2M-token pool) attending to itself from position 0; sampled queries against the oracle."""
    _case("prefill-c4-chunk")
    W = workloads.config(4)
    cache = make_cache(W, fill_byte=None)
    bt, _ = upload_tables(W)
    b = W.batch                                  # the chunk's sequence
    k, v = W.kv_bits(b)
    fill(cache, W, bt, seqs=[b], kv={b: (k, v)})
    r = np.random.default_rng(4)
    q = workloads.round_to_bf16_bits(r.standard_normal((W.chunk_tokens, W.num_q_heads, 128)).astype(np.float32))
    out = cache.prefill(to_dev(q), bt[b], 0, W.softmax_scale, 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    for i in (0, 1, 15, 16, 1000, W.chunk_tokens - 1):
        want = oracle.prefill_sequence(W.dtype, q[i:i + 1], k[: i + 1], v[: i + 1], i, W.softmax_scale)
        err = np.max(np.abs(got[i] - want[0]))
        assert err <= TOL, f"query {i}: {err:.3e}"


@pytest.mark.parametrize("dtype,start,chunk,hq,hkv,ps", [(16, 200, 90, 16, 8, 256), (0, 300, 33, 8, 1, 256),
                                                         (2, 0, 130, 32, 8, 64), (4, 700, 100, 32, 8, 256),
                                                         (3, 1000, 40, 40, 8, 128), (8, 260, 75, 16, 16, 256)])
def test_prefill_large_pages(dtype, start, chunk, hq, hkv, ps):
    _case("prefill-ps", dtype, start, chunk, hq, hkv, ps)
    W, cache, bt, kv, q = _setup(dtype, start, chunk, hq, hkv, ps, 860 + dtype)
    k, v = kv[0]
    want = oracle.prefill_sequence(dtype, q, k, v, start, W.softmax_scale)
    out = cache.prefill(to_dev(q), bt[0], start, W.softmax_scale, 0)
    torch.cuda.synchronize()
    err = np.max(np.abs(out.cpu().numpy().astype(np.float64) - want), axis=(1, 2))
    assert np.all(err <= TOL), f"worst query {int(np.argmax(err))} err {err.max():.3e}"
