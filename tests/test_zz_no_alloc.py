"""The allocation-free decode (xq_paged_decode_attention_noalloc, split partials in the library's
built-in scratch) against xq_paged_decode_attention with a caller workspace, through the C ABI:
bitwise equal outputs, and both within the 2e-3 bar of the oracle, on two calls in a row, the
second with a smaller input."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_quantized_paged_turbo_amd as xq
from tests.gpu_util import fill, make_cache, to_dev, upload_tables

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(W, splits):
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    q = to_dev(qb)
    need = cache.workspace_bytes(W.batch, W.num_q_heads, W.max_context_len, splits)
    assert 0 < need <= xq.NOALLOC_SCRATCH_BYTES          # the partials go through the scratch
    want = cache.decode(q, bt, cl, W.max_context_len, W.softmax_scale, splits)
    got = torch.full_like(want, float("nan"))
    xq.xq_paged_decode_attention_noalloc(cache.layout, q, W.batch, W.num_q_heads, cache.k_pool, cache.v_pool,
                                         bt, int(bt.shape[1]), cl, W.max_context_len, W.softmax_scale, splits,
                                         got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{W.name}: differs from the workspace decode"
    g = got.cpu().numpy().astype(np.float64)
    for b in range(W.batch):
        ref, _ = oracle.decode_sequence(W.dtype, qb[b], kv[b][0], kv[b][1], W.softmax_scale)
        err = np.max(np.abs(g[b] - ref))
        assert err <= TOL, f"{W.name} seq {b}: {err:.3e}"


def test_noalloc_decode_equals_the_workspace_decode_twice():
    print("CASE noalloc", flush=True)
    big = workloads.make("noalloc-big", 980, 4, [3000, 45, 1700, 2600, 900, 1, 2049, 700], 32, 8, 16)
    small = workloads.make("noalloc-small", 981, 3, [300, 130], 40, 8, 64)
    _run(big, 6)
    _run(small, 3)
