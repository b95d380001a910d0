"""XQ_DEBUG: with the variable set, both calls check the contents of their device index
arrays before launching and return XQ_EINVAL on a violation (include/xq.h, Errors).

Every rejected input here is one the kernels would still handle without a fault if the
check let it through: decode loads are range-checked buffer loads (out-of-range pages read
as zeros and context lengths are clamped to max_context_len), and the append cases write
either a duplicate slot or a page past the layout's num_pages that the pools still hold.
"""
import numpy as np
import pytest
import torch

import bit_quantized_paged_turbo_amd as xq
from bit_quantized_paged_turbo_amd import CacheLayout, xq_pool_bytes

pytestmark = pytest.mark.gpu

HKV, HQ, PS = 2, 8, 16


def _bf16(rng, *shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda().to(torch.bfloat16)


def _setup(num_pages=12, alloc_pages=None, dtype=4):
    """Layout of num_pages pages over pools that hold alloc_pages pages, filled for two
    sequences of 40 and 17 tokens on pages 0..2 and 3..4."""
    rng = np.random.default_rng(7)
    L = CacheLayout(dtype, HKV, PS, num_pages)
    big = CacheLayout(dtype, HKV, PS, alloc_pages or num_pages)
    kp = torch.zeros(xq_pool_bytes(big), dtype=torch.uint8, device="cuda")
    vp = torch.zeros_like(kp)
    bt = torch.tensor([[0, 1, 2, 0], [3, 4, 0, 0]], dtype=torch.int32, device="cuda")
    lens = [40, 17]
    seq = torch.tensor(sum(([b] * n for b, n in enumerate(lens)), []), dtype=torch.int32, device="cuda")
    pos = torch.tensor(sum((list(range(n)) for n in lens), []), dtype=torch.int32, device="cuda")
    k, v = _bf16(rng, len(seq), HKV, 128), _bf16(rng, len(seq), HKV, 128)
    xq.xq_quantize_append(L, k, v, len(seq), seq, pos, bt, bt.shape[1], kp, vp)
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = _bf16(rng, 2, HQ, 128)
    return L, kp, vp, bt, cl, q, rng


def _decode(L, kp, vp, bt, cl, q, max_ctx=64):
    out = torch.zeros(2, HQ, 128, dtype=torch.float32, device="cuda")
    xq.xq_paged_decode_attention(L, q, 2, HQ, kp, vp, bt, bt.shape[1], cl, max_ctx, 0.088, 1,
                                 None, 0, out)
    torch.cuda.synchronize()
    return out.cpu()


def test_debug_mode_gives_the_same_result(monkeypatch):
    L, kp, vp, bt, cl, q, _ = _setup()
    monkeypatch.setenv("XQ_DEBUG", "0")
    ref = _decode(L, kp, vp, bt, cl, q)
    monkeypatch.setenv("XQ_DEBUG", "1")
    got = _decode(L, kp, vp, bt, cl, q)
    assert torch.equal(ref, got)


@pytest.mark.parametrize("case", ["page_too_big", "page_negative", "len_above_max", "len_negative"])
def test_decode_rejects_bad_index_arrays(monkeypatch, case):
    L, kp, vp, bt, cl, q, _ = _setup()
    monkeypatch.setenv("XQ_DEBUG", "1")
    if case == "page_too_big":
        bt[1, 1] = 12                  # position 16 of sequence 1 (length 17) is on page 12
        msg = "block_tables[1][1] = 12"
    elif case == "page_negative":
        bt[0, 2] = -3
        msg = "block_tables[0][2] = -3"
    elif case == "len_above_max":
        cl[0] = 65
        msg = "context_lens[0] = 65"
    else:
        cl[1] = -1
        msg = "context_lens[1] = -1"
    print("CASE decode", case, flush=True)
    out = torch.full((2, HQ, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(xq.XqError) as e:
        xq.xq_paged_decode_attention(L, q, 2, HQ, kp, vp, bt, bt.shape[1], cl, 64, 0.088, 1, None,
                                     0, out)
    assert e.value.status == xq.EINVAL and msg in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())    # nothing was launched


def test_decode_ignores_entries_past_the_context(monkeypatch):
    """Only the pages holding positions below context_lens[b] are checked."""
    L, kp, vp, bt, cl, q, _ = _setup()
    monkeypatch.setenv("XQ_DEBUG", "1")
    bt[1, 3] = 999                      # page 3 of sequence 1 holds positions 48.. > 17
    _decode(L, kp, vp, bt, cl, q)


@pytest.mark.parametrize("case", ["duplicate_slot", "page_past_layout"])
def test_append_rejects_bad_index_arrays(monkeypatch, case):
    # the pools hold 16 pages, the layout says 12: page 13 is out of contract but in memory
    L, kp, vp, bt, cl, q, rng = _setup(num_pages=12, alloc_pages=16)
    monkeypatch.setenv("XQ_DEBUG", "1")
    before_k, before_v = kp.clone(), vp.clone()
    if case == "duplicate_slot":
        seq = torch.tensor([0, 1, 0], dtype=torch.int32, device="cuda")
        pos = torch.tensor([41, 17, 41], dtype=torch.int32, device="cuda")
        msg = "already written"
    else:
        bt[1, 1] = 13
        seq = torch.tensor([1], dtype=torch.int32, device="cuda")
        pos = torch.tensor([18], dtype=torch.int32, device="cuda")
        msg = "maps to page 13"
    print("CASE append", case, flush=True)
    k, v = _bf16(rng, len(seq), HKV, 128), _bf16(rng, len(seq), HKV, 128)
    with pytest.raises(xq.XqError) as e:
        xq.xq_quantize_append(L, k, v, len(seq), seq, pos, bt, bt.shape[1], kp, vp)
    assert e.value.status == xq.EINVAL and msg in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(kp, before_k) and torch.equal(vp, before_v)   # nothing was launched


def test_append_valid_batch_passes_the_checks(monkeypatch):
    L, kp, vp, bt, cl, q, rng = _setup()
    monkeypatch.setenv("XQ_DEBUG", "1")
    seq = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    pos = torch.tensor([40, 17], dtype=torch.int32, device="cuda")
    k, v = _bf16(rng, 2, HKV, 128), _bf16(rng, 2, HKV, 128)
    xq.xq_quantize_append(L, k, v, 2, seq, pos, bt, bt.shape[1], kp, vp)
    torch.cuda.synchronize()


def test_debug_prefill_rejects_a_page_past_the_pool(monkeypatch):
    """A prefill reads the chunk's block-table row for every position below start + n: an entry
    naming a page at or past num_pages is rejected under XQ_DEBUG before any launch, and the same
    call with a good row gives the unchecked result."""
    L, kp, vp, bt, cl, q, rng = _setup(num_pages=5, alloc_pages=12)
    qp = _bf16(rng, 10, HQ, 128)
    out = torch.zeros(10, HQ, 128, dtype=torch.float32, device="cuda")
    row = bt[0].clone()
    monkeypatch.setenv("XQ_DEBUG", "0")
    xq.xq_paged_prefill_attention(L, qp, 10, HQ, kp, vp, row, row.shape[0], 30, 0.088, 1, None, 0, out)
    torch.cuda.synchronize()
    ref = out.cpu().clone()
    monkeypatch.setenv("XQ_DEBUG", "1")
    xq.xq_paged_prefill_attention(L, qp, 10, HQ, kp, vp, row, row.shape[0], 30, 0.088, 1, None, 0, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref)
    bad = row.clone()
    bad[2] = 7                                    # page 7 >= num_pages = 5 (the pools hold 12)
    with pytest.raises(xq.XqError) as e:
        xq.xq_paged_prefill_attention(L, qp, 10, HQ, kp, vp, bad, bad.shape[0], 30, 0.088, 1, None, 0, out)
    assert e.value.status == xq.EINVAL and "block_table[2]" in str(e.value)


def test_debug_planned_decode_rejects_a_non_permutation(monkeypatch):
    L, kp, vp, bt, cl, q, _ = _setup()
    out = torch.zeros(2, HQ, 128, dtype=torch.float32, device="cuda")
    good = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    bad = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("XQ_DEBUG", "1")
    xq.xq_paged_decode_attention_planned(L, q, 2, HQ, kp, vp, bt, bt.shape[1], cl, 64, 0.088, 1, None, 0,
                                         out, good)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), _decode(L, kp, vp, bt, cl, q))
    with pytest.raises(xq.XqError) as e:
        xq.xq_paged_decode_attention_planned(L, q, 2, HQ, kp, vp, bt, bt.shape[1], cl, 64, 0.088, 1, None, 0,
                                             out, bad)
    assert e.value.status == xq.EINVAL and "seq_order" in str(e.value)
