"""The fused step (xq_append_decode_attention): appending each sequence's new row and decoding
in one launch must store the same bytes and give bitwise the same outputs as
xq_quantize_append followed by the decode, for every cache type, split policy and with or
without the host plan; and match the oracle within the 2e-3 bar. Unwritten slots (the new
rows' slots included, before the step) hold 0xFF bytes, so a read of a slot before its new row
has landed would show."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import make_cache, to_dev, upload_tables

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _fill_all_but_last(cache, W, bt, kv):
    ks, vs, ss, ps = [], [], [], []
    for b in range(W.batch):
        L = int(W.context_lens[b])
        if L <= 1:
            continue
        ks.append(kv[b][0][: L - 1])
        vs.append(kv[b][1][: L - 1])
        ss.append(np.full(L - 1, b, np.int32))
        ps.append(np.arange(L - 1, dtype=np.int32))
    cache.append(to_dev(np.concatenate(ks)), to_dev(np.concatenate(vs)), to_dev(np.concatenate(ss)),
                 to_dev(np.concatenate(ps)), bt)


@pytest.mark.parametrize("dtype,hq,hkv,ps", [(4, 16, 8, 16), (8, 32, 8, 16), (3, 40, 8, 64), (2, 16, 8, 16),
                                             (0, 16, 8, 16), (16, 32, 8, 16), (4, 32, 2, 32)])
def test_fused_step_equals_append_then_decode(dtype, hq, hkv, ps):
    print("CASE fused", dtype, hq, hkv, ps, flush=True)
    r = np.random.default_rng(dtype + 40)
    lens = list(r.integers(1, 900, 254)) + [0, 1]          # 256 sequences, with an empty and a 1-token one
    W = workloads.make(f"fused-{dtype}", 950 + dtype, dtype, lens, hq, hkv, ps)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    bt, cl = upload_tables(W)
    qb = W.q_bits()
    q = to_dev(qb)
    new_k = to_dev(np.stack([kv[b][0][-1] if lens[b] else np.zeros((hkv, 128), np.uint16)
                             for b in range(W.batch)]))
    new_v = to_dev(np.stack([kv[b][1][-1] if lens[b] else np.zeros((hkv, 128), np.uint16)
                             for b in range(W.batch)]))
    live = [b for b in range(W.batch) if lens[b] > 0]
    seq = to_dev(np.array(live, np.int32))
    pos = to_dev(np.array([lens[b] - 1 for b in live], np.int32))
    for splits in (0, 3, -256):
        for planned in (False, True):
            a, f = make_cache(W), make_cache(W)
            _fill_all_but_last(a, W, bt, kv)
            _fill_all_but_last(f, W, bt, kv)
            # the plan of these arguments: a permutation of the batch with one partition per
            # sequence, a unit placement with several
            so = a.plan([int(x) for x in lens], hq, W.max_context_len, splits) if planned else None
            a.append(new_k[live].contiguous(), new_v[live].contiguous(), seq, pos, bt)
            want = a.decode(q, bt, cl, W.max_context_len, W.softmax_scale, splits, seq_order=so)
            got = f.append_decode(new_k, new_v, q, bt, cl, W.max_context_len, W.softmax_scale, splits,
                                  seq_order=so)
            torch.cuda.synchronize()
            assert torch.equal(a.k_pool, f.k_pool) and torch.equal(a.v_pool, f.v_pool), (splits, planned)
            assert torch.equal(want, got), (splits, planned)
    out = got.cpu().numpy().astype(np.float64)
    assert np.all(out[lens.index(0)] == 0)
    for b in (0, 100, 253, 255):
        k, v = kv[b]
        ref, _ = oracle.decode_sequence(dtype, qb[b], k, v, W.softmax_scale)
        assert np.max(np.abs(out[b] - ref)) <= TOL, b


@pytest.mark.parametrize("dtype,hq,hkv,ps", [(4, 8, 8, 256), (16, 8, 8, 256), (3, 8, 1, 128)])
def test_fused_step_page_sizes_and_groups(dtype, hq, hkv, ps):
    """Large pages (the new row deep inside a page) and one query head per kv head."""
    print("CASE fused-ps", dtype, hq, hkv, ps, flush=True)
    lens = [700, 1, 256, 257, 513, 90, 1000, 31]
    W = workloads.make(f"fusedps-{dtype}", 990 + dtype, dtype, lens, hq, hkv, ps)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    bt, cl = upload_tables(W)
    qb = W.q_bits()
    q = to_dev(qb)
    new_k = to_dev(np.stack([kv[b][0][-1] for b in range(W.batch)]))
    new_v = to_dev(np.stack([kv[b][1][-1] for b in range(W.batch)]))
    seq = to_dev(np.arange(W.batch, dtype=np.int32))
    pos = to_dev(np.array([L - 1 for L in lens], np.int32))
    a, f = make_cache(W), make_cache(W)
    _fill_all_but_last(a, W, bt, kv)
    _fill_all_but_last(f, W, bt, kv)
    a.append(new_k, new_v, seq, pos, bt)
    want = a.decode(q, bt, cl, W.max_context_len, W.softmax_scale, 0)
    got = f.append_decode(new_k, new_v, q, bt, cl, W.max_context_len, W.softmax_scale, 0)
    torch.cuda.synchronize()
    assert torch.equal(a.k_pool, f.k_pool) and torch.equal(a.v_pool, f.v_pool)
    assert torch.equal(want, got)
    out = got.cpu().numpy().astype(np.float64)
    for b in range(W.batch):
        ref, _ = oracle.decode_sequence(dtype, qb[b], kv[b][0], kv[b][1], W.softmax_scale)
        assert np.max(np.abs(out[b] - ref)) <= TOL, b
