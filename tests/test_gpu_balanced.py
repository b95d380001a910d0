"""Decode over a length-aware plan (xq_decode_plan_balanced + xq_decode_attention_balanced): every
sequence gets its own partition size so that the work units are of about equal length (the infero
page, section "Beyond plain text decode", item "Continuous batching"). The outputs are checked
against the oracle at the parity bar and against the plain decode within the split-agreement bound
(a different partitioning changes only the rounding); the fused append must write the same bytes
as the plain one."""
import numpy as np
import pytest
import torch

import bit_quantized_paged_turbo_amd as xq
import oracle
import workloads
from tests.gpu_util import fill, make_cache, to_dev, upload_tables
from tests.test_gpu_parity import _codec_check

pytestmark = pytest.mark.gpu
TOL = 2e-3
# Two partitionings of one decode differ only in the order of fp32 additions: the matrix core's
# accumulation over a partition's tiles (one addition per 32 tokens) and the merge of partitions.
# Summing n terms in fp32 in another order moves the sum by at most (n - 1) 2^-24 of the sum of
# their magnitudes, here at most max|v| (a convex combination of the rotated values); the inverse
# rotation then adds the 128 rotated dimensions' errors into one output, times C = 1/sqrt(128):
# at most sqrt(128) (n - 1) 2^-24 max|v|. The longest sequence here has about 950 tiles and 20
# partitions and |v| stays below 8, a bound near 6e-3; the measured differences sit far below
# it (under 3e-5), so the check uses 1e-4, still an order of magnitude below the 2e-3 bar a
# missing or doubled tile would cross.
AGREE = 1e-4


def _agree(W, kv):
    """Bound on the difference between two partitionings of the same decode. Turbo caches: the
    split-agreement bound (fp16 high and low weight parts, ~22 bits). bf16 and fp8 caches carry
    their weights as bf16 high and low parts, 16 significant bits, so each output is within
    2^-16 max|v| of the exact weighted mean and two partitionings within 2^-15 max|v|."""
    if W.dtype in (workloads.BF16, workloads.FP8):
        vmax = max(float(np.max(np.abs((kv[b][1].astype(np.uint32) << 16).view(np.float32))))
                   for b in kv if W.seq_len(b) > 0)
        return 2.0 ** -15 * vmax + AGREE
    return AGREE


def _oracle(W, b, qb, kv):
    k, v = kv[b] if kv is not None else W.kv_bits(b)
    return oracle.decode_sequence(W.dtype, qb[b], k, v, W.softmax_scale)[0]


@pytest.mark.parametrize("dtype,hq,hkv,ps", [(4, 32, 8, 16), (4, 16, 2, 64), (3, 40, 8, 64), (8, 32, 8, 16),
                                             (2, 16, 8, 16), (16, 16, 8, 16), (0, 16, 8, 32), (4, 12, 1, 256)])
def test_balanced_decode_matches_oracle_and_plain(dtype, hq, hkv, ps):
    print("CASE balanced", dtype, hq, hkv, ps, flush=True)
    lens = [0, 1, 17, 300, 1029, 2000, 64, 5000, 33, 777, 4096, 2]
    W = workloads.make(f"bal-{dtype}-{ps}", 1200 + dtype, dtype, lens, hq, hkv, ps)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    q = to_dev(qb)
    plan = cache.plan_balanced(lens, hq, W.max_context_len)
    got = cache.decode_balanced(q, bt, cl, W.max_context_len, W.softmax_scale, plan)
    plain = cache.decode(q, bt, cl, W.max_context_len, W.softmax_scale, 0)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    plain = plain.cpu().numpy().astype(np.float64)
    assert np.all(got[0] == 0)                       # empty context -> zeros
    diff = np.max(np.abs(got - plain))
    print(f"stride {plan[0]}; balanced against plain: {diff:.3e}", flush=True)
    assert diff < _agree(W, kv)
    for b in range(1, W.batch):
        err = np.max(np.abs(got[b] - _oracle(W, b, qb, kv)))
        assert err <= TOL, f"seq {b} (L={lens[b]}): {err:.3e}"


@pytest.mark.parametrize("dtype", [4, 3])
def test_balanced_fused_step_writes_the_plain_bytes(dtype):
    """The step with its append: the same code bytes as the plain fused step, outputs within the
    split-agreement bound of it and within the bar of the oracle."""
    print("CASE balanced fused", dtype, flush=True)
    lens = [5, 700, 3000, 64, 1, 1500, 2049, 96]
    hq, hkv = 32, 8
    W = workloads.make(f"balf-{dtype}", 1300 + dtype, dtype, lens, hq, hkv, 16)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    qb = W.q_bits()
    q = to_dev(qb)
    outs, pools = [], []
    for balanced in (False, True):
        cache = make_cache(W)
        bt, cl = upload_tables(W)
        # every position but the last through the append kernel; the last one by the fused step
        rows = [(b, L - 1) for b, L in enumerate(lens) if L > 1]
        kk = to_dev(np.concatenate([kv[b][0][:n] for b, n in rows]))
        vv = to_dev(np.concatenate([kv[b][1][:n] for b, n in rows]))
        seq = to_dev(np.concatenate([np.full(n, b, np.int32) for b, n in rows]))
        pos = to_dev(np.concatenate([np.arange(n, dtype=np.int32) for b, n in rows]))
        cache.append(kk, vv, seq, pos, bt)
        k_new = to_dev(np.stack([kv[b][0][-1] for b in range(W.batch)]))
        v_new = to_dev(np.stack([kv[b][1][-1] for b in range(W.batch)]))
        if balanced:
            plan = cache.plan_balanced(lens, hq, W.max_context_len)
            out = cache.decode_balanced(q, bt, cl, W.max_context_len, W.softmax_scale, plan, k_new, v_new)
        else:
            out = cache.append_decode(k_new, v_new, q, bt, cl, W.max_context_len, W.softmax_scale, 0)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64))
        pools.append((cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()))
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
    assert np.max(np.abs(outs[0] - outs[1])) < AGREE
    for b in range(W.batch):
        err = np.max(np.abs(outs[1][b] - _oracle(W, b, qb, kv)))
        assert err <= TOL, f"seq {b} (L={lens[b]}): {err:.3e}"


FULL = [("mixed-32q8kv-turbo4", 4, None, [0, 13, 63]), ("batched-16q8kv-turbo4", 1, None, [0, 100, 255]),
        ("longctx-40q8kv-turbo3", 3, None, [0]), ("8b-32q8kv-ctx8192-turbo8", 2, 8, [0, 31])]


@pytest.mark.parametrize("name,cfg,dtype,sample", FULL, ids=[f[0] for f in FULL])
def test_balanced_full_size(name, cfg, dtype, sample):
    """The benchmark's step at full size with a length-aware plan: fused append (each sequence's
    last position again) and decode; sampled sequences against the oracle, every sequence against
    the plain planned step."""
    print("CASE balanced full", name, flush=True)
    W = workloads.config(cfg, dtype=dtype)
    cache = make_cache(W, fill_byte=None)
    bt, cl = upload_tables(W)
    last = {}
    fill(cache, W, bt, last=last)
    torch.cuda.synchronize()
    B, qb = W.batch, W.q_bits()
    q = to_dev(qb)
    k_new = to_dev(np.stack([last[b][0] for b in range(B)]))
    v_new = to_dev(np.stack([last[b][1] for b in range(B)]))
    lens = [int(x) for x in W.context_lens]
    plan = cache.plan_balanced(lens, W.num_q_heads, W.max_context_len)
    got = cache.decode_balanced(q, bt[:B], cl, W.max_context_len, W.softmax_scale, plan, k_new, v_new)
    order = cache.plan(lens, W.num_q_heads, W.max_context_len, W.num_splits)
    plain = cache.append_decode(k_new, v_new, q, bt[:B], cl, W.max_context_len, W.softmax_scale,
                                W.num_splits, seq_order=order)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    plain = plain.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    diff = np.max(np.abs(got - plain))
    print(f"stride {plan[0]}; balanced against plain: {diff:.3e}", flush=True)
    assert diff < AGREE
    for b in sample:
        err = np.max(np.abs(got[b] - oracle.decode_sequence(W.dtype, qb[b], *W.kv_bits(b), W.softmax_scale)[0]))
        assert err <= TOL, f"{name} seq {b}: {err:.3e}"


@pytest.mark.parametrize("dtype", [4, 3, 8, 2, 0, workloads.FP8])
def test_balanced_step_appends_a_chunk_in_the_same_launch(dtype, monkeypatch):
    """A prefill chunk of a sequence outside the decoded batch (continuous batching, infero page,
    section "Beyond plain text decode") appended by the decode's own launch: the pools hold the
    bytes of the separate append kernel, the chunk's rows equal the oracle's encoding, and the
    decode's outputs are bit-identical to the same plan's without the chunk."""
    print("CASE balanced chunk", dtype, flush=True)
    monkeypatch.setenv("XQ_DEBUG", "1")             # also checks that no chunk page is read
    lens = [5, 700, 3000, 64, 1, 1500, 2049, 96, 333]
    hq, hkv = 32, 8
    W = workloads.make(f"balc-{dtype}", 1400 + dtype, dtype, lens, hq, hkv, 16, chunk_tokens=1037)
    B = W.batch
    kv = {b: W.kv_bits(b) for b in range(W.num_seqs)}
    qb = W.q_bits()
    q = to_dev(qb)
    chunk = (to_dev(kv[B][0]), to_dev(kv[B][1]), to_dev(np.full(W.chunk_tokens, B, np.int32)),
             to_dev(np.arange(W.chunk_tokens, dtype=np.int32)))
    k_new = to_dev(np.stack([kv[b][0][-1] for b in range(B)]))
    v_new = to_dev(np.stack([kv[b][1][-1] for b in range(B)]))
    outs, pools = [], []
    for inline in (False, True):
        cache = make_cache(W)
        bt, cl = upload_tables(W)
        fill(cache, W, bt, seqs=range(B), kv=kv)      # the decoded sequences; the chunk's pages unwritten
        plan = cache.plan_balanced(lens, hq, W.max_context_len)
        if not inline:
            cache.append(*chunk[:2], chunk[2], chunk[3], bt)
        out = cache.decode_balanced(q, bt, cl, W.max_context_len, W.softmax_scale, plan, k_new, v_new,
                                    chunk=chunk if inline else None)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        pools.append((cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()))
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
    assert np.array_equal(outs[0], outs[1])
    _codec_check(W, cache, [B])
    got = outs[1].astype(np.float64)
    for b in range(B):
        err = np.max(np.abs(got[b] - _oracle(W, b, qb, kv)))
        assert err <= TOL, f"seq {b} (L={lens[b]}): {err:.3e}"


def test_balanced_chunk_into_a_read_page_is_rejected(monkeypatch):
    """Under XQ_DEBUG a chunk row that lands in a page the decode reads is refused before any
    launch (the decode's units and the appenders run in no fixed order)."""
    print("CASE balanced chunk rejected", flush=True)
    monkeypatch.setenv("XQ_DEBUG", "1")
    lens = [40, 90]
    W = workloads.make("balc-bad", 1500, 4, lens, 16, 8, 16, chunk_tokens=20)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    fill(cache, W, bt)
    q = to_dev(W.q_bits())
    k, v = W.kv_bits(2)
    # positions 70..89 of sequence 1: rows the decode reads
    chunk = (to_dev(k), to_dev(v), to_dev(np.full(20, 1, np.int32)), to_dev(np.arange(70, 90, dtype=np.int32)))
    plan = cache.plan_balanced(lens, 16, W.max_context_len)
    before = cache.k_pool.clone()
    with pytest.raises(xq.XqError) as e:
        cache.decode_balanced(q, bt, cl, W.max_context_len, W.softmax_scale, plan, chunk=chunk)
    assert e.value.status == xq.EINVAL and "which the decode reads" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(cache.k_pool, before)
