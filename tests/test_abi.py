"""The C-ABI library loads, exports every symbol include/xq.h declares, and validates
host-visible arguments without touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import bit_quantized_paged_turbo_amd as xq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(xq.LIB_PATH):
        from bit_quantized_paged_turbo_amd import build
        build.build()
    return xq.load()


def test_exports_match_header(lib):
    header = open(os.path.join(ROOT, "include", "xq.h")).read()
    declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(xq_\w+)\s*\(", header, re.M))
    assert declared == set(xq.EXPORTS)
    for name in declared:
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("dtype,ps,block", [(4, 16, 1056), (8, 16, 2080), (3, 64, 3200),
                                            (0, 16, 4096), (3, 16, 800), (4, 256, 16896),
                                            (2, 16, 544), (2, 64, 2176), (16, 16, 2048), (16, 64, 8192)])
def test_block_geometry(lib, dtype, ps, block):
    L = xq.CacheLayout(dtype, 8, ps, 10)
    assert xq.xq_block_bytes(L) == block
    assert xq.xq_page_stride_bytes(L) == 8 * block
    assert xq.xq_pool_bytes(L) == 80 * block


@pytest.mark.parametrize("bad", [dict(kv_dtype=5), dict(kv_dtype=1), dict(kv_dtype=17), dict(head_dim=64), dict(num_kv_heads=0),
                                 dict(page_size=24), dict(page_size=8), dict(page_size=512),
                                 dict(num_pages=0)])
def test_invalid_layouts(lib, bad):
    args = dict(kv_dtype=4, num_kv_heads=8, page_size=16, num_pages=10)
    head_dim = bad.pop("head_dim", 128)
    args.update(bad)
    L = xq.CacheLayout(head_dim=head_dim, **args)
    assert xq.xq_block_bytes(L) == -1
    assert xq.xq_pool_bytes(L) == -1


def test_split_planning(lib):
    L = xq.CacheLayout(3, 8, 64, 4096)
    assert xq.xq_decode_num_splits(L, 1, 40, 262144, 256) == 256
    # the partials: (m, l, pad, acc[128]) per (sequence, q head, split)
    assert xq.xq_decode_workspace_bytes(L, 1, 40, 262144, 256) == 40 * 256 * 132 * 4
    L = xq.CacheLayout(4, 8, 16, 9000)
    # library policy: whole pages / 32-token tiles per split, partials only when split
    n = xq.xq_decode_num_splits(L, 256, 16, 1022, 0)
    assert 1 <= n <= 16
    tps = -(-1022 // n)
    assert xq.xq_decode_num_splits(L, 256, 16, 1022, n) == n
    part = 256 * 16 * n * 132 * 4 if n > 1 else 0
    assert xq.xq_decode_workspace_bytes(L, 256, 16, 1022, 0) == part
    assert xq.xq_decode_num_splits(L, 256, 16, 1022, 1) == 1
    assert xq.xq_decode_workspace_bytes(L, 256, 16, 1022, 1) == 0
    assert xq.xq_decode_num_splits(L, 4, 16, 1000, 7) == 7
    assert xq.xq_decode_num_splits(L, 4, 16, 0, 0) == 1
    assert xq.xq_decode_num_splits(L, 4, 16, 100, -1) == -1
    # a split spans at most 128 pages, whatever the hint
    assert xq.xq_decode_num_splits(xq.CacheLayout(4, 8, 16, 9000), 1, 8, 65536, 1) == 32
    assert xq.xq_decode_num_splits(xq.CacheLayout(3, 8, 64, 9000), 1, 8, 262144, 4) == 32
    # fixed partitions (negative hint): -hint tokens each, independent of the batch
    L = xq.CacheLayout(4, 8, 16, 9000)
    assert xq.xq_decode_num_splits(L, 256, 16, 9000, -1024) == 9
    assert xq.xq_decode_num_splits(L, 1, 16, 9000, -1024) == 9
    assert xq.xq_decode_num_splits(L, 3, 16, 9000, -2048) == 5
    assert xq.xq_decode_num_splits(L, 3, 16, 9000, -1000) == -1     # not a multiple of 32
    assert xq.xq_decode_num_splits(L, 3, 16, 9000, -2080) == -1     # more than 128 pages
    assert xq.xq_decode_workspace_bytes(L, 4, 16, 1000, -256) == 4 * 16 * 4 * 132 * 4
    L = xq.CacheLayout(3, 8, 64, 4096)
    assert xq.xq_decode_num_splits(L, 1, 40, 262144, -32) == -1      # not whole pages
    assert xq.xq_decode_num_splits(L, 1, 40, 262144, -1024) == 256
    # bf16 needs no query preparation: no workspace for a single split
    L = xq.CacheLayout(0, 8, 16, 9000)
    assert xq.xq_decode_workspace_bytes(L, 256, 16, 1022, 1) == 0


def _decode_status(lib, L, **kw):
    a = dict(q=16, batch=1, hq=8, k=16, v=16, bt=16, maxp=4, cl=16, maxctx=64, scale=0.1,
             splits=0, ws=None, wsb=0, out=16, stream=None)
    a.update(kw)
    return lib.xq_paged_decode_attention(ctypes.byref(L), a["q"], a["batch"], a["hq"], a["k"],
                                         a["v"], a["bt"], a["maxp"], a["cl"], a["maxctx"],
                                         a["scale"], a["splits"], a["ws"], a["wsb"], a["out"],
                                         a["stream"])


def test_decode_argument_errors(lib):
    L = xq.CacheLayout(4, 2, 16, 10)
    assert _decode_status(lib, L, hq=7) == xq.EINVAL           # not a multiple of Hkv
    assert _decode_status(lib, L, hq=34) == xq.EUNSUPPORTED    # group 17 > 16
    assert _decode_status(lib, L, q=None) == xq.EINVAL
    assert _decode_status(lib, L, k=8) == xq.EINVAL            # misaligned pool
    assert _decode_status(lib, L, out=8) == xq.EINVAL          # misaligned output (16-byte stores)
    assert _decode_status(lib, L, maxctx=65) == xq.EINVAL      # > maxp * page_size
    assert _decode_status(lib, L, splits=2) == xq.EWORKSPACE   # partials of two splits
    assert b"workspace" in lib.xq_last_error()
    assert _decode_status(lib, L, splits=-48) == xq.EINVAL      # fixed partition not whole tiles
    assert b"fixed partition" in lib.xq_last_error()
    assert _decode_status(lib, L, batch=0) == xq.OK            # nothing to do
    bad = xq.CacheLayout(4, 2, 20, 10)
    assert _decode_status(lib, bad) == xq.EINVAL


def test_noalloc_decode_rejects_what_its_scratch_cannot_hold(lib):
    """The allocation-free decode checks its partials against the built-in 16 MiB before anything
    touches a device: too many (sequence, head, split) partials give XQ_EWORKSPACE."""
    L = xq.CacheLayout(4, 8, 16, 1 << 20)
    need = xq.xq_decode_workspace_bytes(L, 4096, 64, 16384, 16)
    assert need > xq.NOALLOC_SCRATCH_BYTES
    st = lib.xq_paged_decode_attention_noalloc(ctypes.byref(L), 16, 4096, 64, 16, 16, 16, 1024, 16, 16384,
                                               0.1, 16, 16, None)
    assert st == xq.EWORKSPACE
    assert b"16777216" in lib.xq_last_error()
    assert lib.xq_paged_decode_attention_noalloc(ctypes.byref(L), 16, 0, 64, 16, 16, 16, 1024, 16, 16384,
                                                 0.1, 16, 16, None) == xq.OK     # empty batch


def test_append_argument_errors(lib):
    L = xq.CacheLayout(4, 2, 16, 10)
    call = lambda **kw: lib.xq_quantize_append(
        ctypes.byref(L), kw.get("k", 16), kw.get("v", 16), kw.get("n", 4), kw.get("s", 16),
        kw.get("p", 16), kw.get("bt", 16), kw.get("maxp", 4), kw.get("kp", 16), kw.get("vp", 16), None)
    assert call(n=-1) == xq.EINVAL
    assert call(n=0) == xq.OK
    assert call(s=None) == xq.EINVAL
    assert call(kp=24) == xq.EINVAL
    assert call(maxp=0) == xq.EINVAL
    # 2^28 rows (tokens x kv heads) would need 2^32 work-items in one launch
    big = xq.CacheLayout(4, 16, 16, 10)
    call16 = lambda n: lib.xq_quantize_append(ctypes.byref(big), 16, 16, n, 16, 16, 16, 4, 16, 16, None)
    assert call16(1 << 24) == xq.EUNSUPPORTED
    assert b"2^28" in lib.xq_last_error()
    assert lib.xq_status_string(xq.EHIP) == b"HIP runtime error"


def _prefill_status(lib, L, **kw):
    a = dict(q=16, n=8, hq=8, k=16, v=16, bt=16, maxp=4, start=10, scale=0.1, splits=0, ws=None,
             wsb=0, out=16, stream=None)
    a.update(kw)
    return lib.xq_paged_prefill_attention(ctypes.byref(L), a["q"], a["n"], a["hq"], a["k"], a["v"],
                                          a["bt"], a["maxp"], a["start"], a["scale"], a["splits"],
                                          a["ws"], a["wsb"], a["out"], a["stream"])


def test_prefill_argument_errors(lib):
    """Argument checks of the chunked prefill; every case fails (or returns) before a launch."""
    L = xq.CacheLayout(4, 2, 16, 10)
    assert _prefill_status(lib, L, n=0) == xq.OK                # nothing to do
    assert _prefill_status(lib, L, n=-1) == xq.EINVAL
    assert _prefill_status(lib, L, start=-1) == xq.EINVAL
    assert _prefill_status(lib, L, start=60, n=5) == xq.EINVAL  # 65 positions > 4 pages of 16
    assert b"max_pages" in lib.xq_last_error()
    assert _prefill_status(lib, L, hq=7) == xq.EINVAL
    assert _prefill_status(lib, L, bt=None) == xq.EINVAL
    assert _prefill_status(lib, L, out=8) == xq.EINVAL          # misaligned output
    assert _prefill_status(lib, L, n=70000, maxp=5000, start=0) == xq.EUNSUPPORTED
    # 108 positions in 2 partitions of 64: both kernels need the partials
    assert _prefill_status(lib, L, start=100, maxp=8, splits=2) == xq.EWORKSPACE
    assert _prefill_status(lib, L, start=100, maxp=8, splits=-64) == xq.EWORKSPACE
    ws = xq.xq_prefill_workspace_bytes(L, 8, 8, 100, 2)
    assert ws == 8 * 8 * 2 * 132 * 4
    assert xq.xq_prefill_workspace_bytes(L, 8, 8, 100, -64) == ws
    assert xq.xq_prefill_workspace_bytes(L, 8, 8, 10, 0) == 0
    assert xq.xq_prefill_workspace_bytes(L, 8, 7, 10, 0) == -1
    assert xq.xq_prefill_workspace_bytes(L, -1, 8, 10, 0) == -1
    assert _prefill_status(lib, L, scale=float("nan")) == xq.EINVAL


def test_decode_plan_pairs_long_with_short(lib):
    """The host plan (no launch): a permutation of the batch; with one partition per sequence the
    slots b and b + 1024 / Hkv (which share SIMDs) get lengths that add up evenly; otherwise the
    identity."""
    import numpy as np
    L = xq.CacheLayout(4, 8, 16, 10000)
    lens = list(np.random.default_rng(1).integers(64, 1025, 256))
    order = xq.xq_decode_plan(L, 256, 16, max(lens), 0, lens)
    assert sorted(order) == list(range(256))
    period = 1024 // 8
    planned = [lens[order[b]] + lens[order[b + period]] for b in range(period)]
    plain = [lens[b] + lens[b + period] for b in range(period)]
    assert max(planned) - min(planned) < (max(plain) - min(plain)) / 4
    # the k-th longest shares its SIMDs with the k-th shortest
    srt = sorted(lens, reverse=True)
    assert lens[order[0]] == srt[0] and lens[order[period]] == srt[-1]
    # a batch that is not a multiple of 8: the identity
    assert xq.xq_decode_plan(L, 255, 16, max(lens), 0, lens[:255]) == list(range(255))
    assert xq.xq_decode_plan(L, 0, 16, 0, 0, []) == []
    assert xq.xq_decode_plan_entries(L, 256, 16, max(lens), 0) == 256


def test_unit_plan_balances_the_mixed_step(lib):
    """Several partitions per sequence (the mixed step's 64 sequences, 15 partitions of 2,048
    tokens): the plan holds one entry per work slot, every unit with tokens exactly once and -1
    elsewhere; the kv heads of a (sequence, partition) sit on one XCD (slot mod 8); the resident
    rounds (three waves a SIMD, slot i on SIMD i mod 1024 of the 1,024 this container assumes) give
    every SIMD within one partition's tiles of every other (the unplanned order, measured on MI355X,
    gave SIMDs from 17 to 192 tiles)."""
    import numpy as np
    import workloads
    W = workloads.config(4)
    L = xq.CacheLayout(4, 8, 16, W.num_pages)
    lens = [int(x) for x in W.context_lens]
    n = xq.xq_decode_plan_entries(L, 64, 32, W.max_context_len, 0)
    nsplits = xq.xq_decode_num_splits(L, 64, 32, W.max_context_len, 0)
    assert nsplits == 15 and n == 15 * 8 * 64
    plan = np.array(xq.xq_decode_plan(L, 64, 32, W.max_context_len, 0, lens))
    assert len(plan) == n
    tps = -(-W.max_context_len // nsplits)
    tps = -(-tps // 32) * 32
    real = {((b * nsplits + s) * 8 + k) for b in range(64) for s in range(-(-lens[b] // tps)) for k in range(8)}
    used = plan[plan >= 0]
    assert len(used) == len(set(used.tolist())) == len(real) and set(used.tolist()) == real
    tiles = {}
    for i, u in enumerate(plan):
        if u < 0:
            continue
        k, r = u % 8, u // 8
        s, b = r % nsplits, r // nsplits
        tiles[i] = -(-(min(lens[b], (s + 1) * tps) - s * tps) // 32)
        # the 8 kv heads of this unit's group share its slot's XCD
        assert all(plan[j] // 8 == r for j in range(i % 8, n, 8) if plan[j] >= 0 and plan[j] // 8 == r)
    load = np.zeros(1024, int)
    for i, t in tiles.items():
        assert i < 3 * 1024                      # 2,560 units fit the three resident rounds
        load[i % 1024] += t
    # longest-first placement: every SIMD within one partition (64 tiles) of every other
    assert load.max() - load.min() <= 64 and load.min() >= load.mean() - 32, (load.max(), load.min(), load.mean())
    # a planned decode must be given the plan's length
    st = lib.xq_paged_decode_attention_planned(ctypes.byref(L), 16, 64, 32, 16, 16, 16, 2048, 16,
                                               W.max_context_len, 0.1, 0, 16, 1 << 30, 16, 16, 64, None)
    assert st == xq.EINVAL and b"xq_decode_plan_entries" in lib.xq_last_error()
    # an empty sequence keeps its partition 0 (whose unit writes its zero output); a sequence of 500
    # tokens with 1,024-token partitions has only partition 0
    L = xq.CacheLayout(4, 2, 16, 4096)
    plan = xq.xq_decode_plan(L, 3, 4, 3000, 3, [0, 500, 3000])
    assert len(plan) == 3 * 3 * 2
    want = {((b * 3 + s) * 2 + k) for b, ns in ((0, 1), (1, 1), (2, 3)) for s in range(ns) for k in range(2)}
    assert set(u for u in plan if u >= 0) == want and sum(u >= 0 for u in plan) == len(want)


def test_balanced_plan_partitions_every_sequence(lib):
    """The length-aware plan (no launch) on the mixed step and the batched decode: every sequence's
    partition size is a whole number of pages and 32-token tiles within the block-table window;
    the units with work fill ids 0 .. n-1 (pairs {unit, its sequence's size}), each exactly once,
    and fit the three waves per SIMD the decode keeps resident (1,024 SIMDs when no device is
    there to ask); the kv heads of a partition share an XCD in the whole rounds."""
    import numpy as np
    import workloads
    for cfg in (4, 1):
        W = workloads.config(cfg)
        L = xq.CacheLayout(4, 8, W.page_size, W.num_pages)
        lens = [int(x) for x in W.context_lens]
        ns, tps, units = xq.xq_decode_plan_balanced(L, W.batch, W.num_q_heads, W.max_context_len, lens)
        u = np.array(units).reshape(-1, 2)
        assert len(u) == W.batch * ns * 8
        unit_tok = max(32, W.page_size)
        assert all(t % unit_tok == 0 and 0 < t <= 128 * W.page_size for t in tps)
        want = {((b * ns + s) * 8 + k) for b in range(W.batch)
                for s in range(max(1, -(-lens[b] // tps[b]))) for k in range(8)}
        real = int((u[:, 0] >= 0).sum())
        assert (u[:real, 0] >= 0).all() and (u[real:, 0] == -1).all()
        assert real == len(want) and set(u[:real, 0].tolist()) == want
        assert real <= 3 * 1024
        assert all(t == tps[x // 8 // ns] for x, t in u[:real])
        # partitions of about equal length: none above the first (longest) one's, and the units of the
        # whole rounds within a few tiles of each other
        sizes = np.array([-(-(min(lens[x // 8 // ns], (x // 8 % ns + 1) * t) - (x // 8 % ns) * t) // 32)
                          for x, t in u[:real]])
        assert sizes.max() <= 128 * W.page_size // 32
        # kv heads of one partition on one XCD (id mod 8) in the whole rounds of 1,024 ids
        full = real // 1024 * 1024
        xcd = {}
        for i in range(full):
            xcd.setdefault(int(u[i, 0]) // 8, set()).add(i % 8)
        assert all(len(v) == 1 for v in xcd.values())
    # an empty sequence keeps partition 0 (its zero output); a larger batch of one-token sequences
    L = xq.CacheLayout(4, 2, 16, 4096)
    ns, tps, units = xq.xq_decode_plan_balanced(L, 3, 4, 3000, [0, 500, 3000])
    u = np.array(units).reshape(-1, 2)
    assert {int(x) // 2 // ns for x in u[u[:, 0] >= 0, 0]} == {0, 1, 2}
    assert lib.xq_decode_plan_balanced(ctypes.byref(L), 3, 5, 3000, None, None, None) == -1   # 5 % 2 != 0
