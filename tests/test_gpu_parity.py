"""GPU parity: the HIP path against the oracle on the same seeded inputs.

Bar: packed codes and fp16 scales bit-exact; attention outputs within 2e-3 max-abs
(fp32 accumulation against the oracle's float64). Unused page slots are poisoned with
0xFF bytes (a NaN pattern in bf16 and fp16) before the cache is filled.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_quantized_paged_turbo_amd as xq
from bit_quantized_paged_turbo_amd import xq_block_bytes
from tests.gpu_util import dominant_queries, fill, gather, make_cache, to_dev, upload_tables

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _print_case(*a):
    print("CASE", *a, flush=True)


def _codec_check(W, cache, seqs):
    bb = xq_block_bytes(cache.layout)
    kp = cache.k_pool.cpu().numpy()
    vp = cache.v_pool.cpu().numpy()
    for b in seqs:
        L = W.seq_len(b)
        if L == 0:
            continue
        k, v = W.kv_bits(b)
        pos = np.arange(L)
        if L > 20000:   # sample positions of long sequences (first, last and random ones)
            pos = np.unique(np.concatenate([pos[:2048], pos[-2048:],
                                            np.random.default_rng(b).choice(L, 4096)]))
            k, v = k[pos], v[pos]
        for pool, rows in ((kp, k), (vp, v)):
            codes, scales = gather(pool, W, bb, b, pos)
            if W.dtype == 0:
                assert np.array_equal(codes.view(np.uint16).reshape(rows.shape), rows)
                continue
            if W.dtype == workloads.FP8:
                want = oracle.fp8_encode_rows_bf16(rows)
                bad = np.argwhere(codes != want)
                assert bad.size == 0, f"seq {b}: {len(bad)} fp8 bytes differ, first {bad[:3]}"
                continue
            c, s = oracle.quantize_rows_bf16(rows, W.dtype)
            want = oracle.pack_codes(c, W.dtype)
            bad = np.argwhere(codes != want)
            assert bad.size == 0, f"seq {b}: {len(bad)} code bytes differ, first {bad[:3]}"
            assert np.array_equal(scales, s.view(np.uint16)), f"seq {b}: scales differ"


def _decode(W, cache, bt, cl, num_splits=0, q=None):
    q = to_dev(W.q_bits()) if q is None else q
    out = cache.decode(q, bt[: W.batch], cl, W.max_context_len, W.softmax_scale, num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _oracle_out(W, b, q_bits, kv=None):
    k, v = kv if kv is not None else W.kv_bits(b)
    out, _ = oracle.decode_sequence(W.dtype, q_bits[b], k, v, W.softmax_scale)
    return out


# ------------------------------------------------------------------------------------
# codec
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,ps", [(4, 16), (4, 64), (8, 16), (8, 32), (3, 64), (3, 16), (0, 16),
                                      (2, 16), (2, 64), (16, 16), (16, 128)])
def test_append_codes_bit_exact(dtype, ps):
    _print_case("append", dtype, ps)
    W = workloads.make(f"codec-{dtype}-{ps}", 100 + dtype, dtype, [1, 37, 130, 16], 8, 2, ps)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    fill(cache, W, bt)
    torch.cuda.synchronize()
    _codec_check(W, cache, range(W.batch))
    # slots past each sequence's end keep the poison bytes
    bb = xq_block_bytes(cache.layout)
    kp = cache.k_pool.cpu().numpy().reshape(W.num_pages, W.num_kv_heads, bb)
    rowb = 256 if dtype == 0 else 128 if dtype == workloads.FP8 else 16 * dtype
    for b in range(W.batch):
        L = int(W.context_lens[b])
        if L % ps:
            page = W.block_tables[b, L // ps]
            assert np.all(kp[page, :, (L % ps) * rowb: ps * rowb] == 0xFF)


@pytest.mark.parametrize("dtype", [8, 4, 3, 2])
def test_append_edge_rows(dtype):
    """Zero rows, rows whose scale underflows or saturates, subnormal bf16 inputs, rows
    already on the quantization grid, and ties."""
    _print_case("edge-rows", dtype)
    rows = np.zeros((8, 1, 128), np.float32)
    g = np.random.default_rng(dtype)
    rows[1, 0] = g.standard_normal(128) * 1e-9          # scale rounds to 0 -> all-zero codes
    rows[2, 0] = g.standard_normal(128) * 1e35          # scale saturates at 65504
    rows[3, 0] = g.standard_normal(128) * 1e-39         # bf16 subnormals
    rows[4, 0, ::3] = 1.0                               # sparse, exact after rotation
    rows[5, 0] = g.standard_normal(128) * 1e4
    rows[6, 0] = np.arange(128) - 64.0
    rows[7, 0, 0] = 1.0
    bits = workloads.round_to_bf16_bits(rows)
    W = workloads.make("edge", 200 + dtype, dtype, [8], 1, 1, 16)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    k = to_dev(bits)
    pos = to_dev(np.arange(8, dtype=np.int32))
    seq = to_dev(np.zeros(8, np.int32))
    cache.append(k, k, seq, pos, bt)
    torch.cuda.synchronize()
    codes, scales = gather(cache.k_pool.cpu().numpy(), W, xq_block_bytes(cache.layout), 0, np.arange(8))
    c, s = oracle.quantize_rows_bf16(bits, dtype)
    assert np.array_equal(codes, oracle.pack_codes(c, dtype))
    assert np.array_equal(scales, s.view(np.uint16))


def test_fp8_append_every_bf16_value():
    """Every finite bf16 bit pattern (65,280 of them, both signs, subnormals, values far past
    the E4M3 range) through the fp8 append, against the oracle's nearest-value cast."""
    _print_case("fp8-all-bf16")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    vals = bits[finite]
    n = -(-vals.size // 128)
    rows = np.zeros(n * 128, np.uint16)
    rows[: vals.size] = vals
    rows = rows.reshape(n, 1, 128)
    W = workloads.make("fp8-all", 250, workloads.FP8, [n], 1, 1, 16)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    k = to_dev(rows)
    pos = to_dev(np.arange(n, dtype=np.int32))
    seq = to_dev(np.zeros(n, np.int32))
    cache.append(k, k, seq, pos, bt)
    torch.cuda.synchronize()
    for pool in (cache.k_pool, cache.v_pool):
        codes, _ = gather(pool.cpu().numpy(), W, xq_block_bytes(cache.layout), 0, np.arange(n))
        want = oracle.fp8_encode_rows_bf16(rows)
        bad = np.argwhere(codes != want)
        assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:3]}"


def test_fp8_decode_over_every_code():
    """K and V rows built from all 254 finite E4M3 values (subnormals, +-0, +-448), each
    stored exactly, so the decode widens every code; a query scaled by 2^-6 keeps the scores
    moderate."""
    _print_case("fp8-every-code")
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    vals = oracle.fp8_e4m3_value(codes)
    g = np.random.default_rng(17)
    L = 300
    k = g.choice(vals, size=(L, 2, 128))
    v = g.choice(vals, size=(L, 2, 128))
    for rows in (k, v):                                    # every code in both heads of both
        rows[:2, 0, :127] = vals[:127]
        rows[2:4, 1, :127] = vals[127:]
    kb = workloads.round_to_bf16_bits(k.astype(np.float32))
    vb = workloads.round_to_bf16_bits(v.astype(np.float32))
    W = workloads.make("fp8-codes", 251, workloads.FP8, [L], 8, 2, 16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    fill(cache, W, bt, kv={0: (kb, vb)})
    qb = workloads.round_to_bf16_bits(oracle.bf16_bits_to_f32(W.q_bits()) / np.float32(64.0))
    for splits in (0, 3):
        got = _decode(W, cache, bt, cl, splits, to_dev(qb))
        want, (kf, vf) = oracle.decode_sequence(W.dtype, qb[0], kb, vb, W.softmax_scale)
        assert np.array_equal(oracle.fp8_e4m3_value(kf), k)   # the rows were stored exactly
        rel = np.max(np.abs(got[0] - want)) / max(1.0, np.max(np.abs(want)))
        assert rel <= TOL / 4, f"splits {splits}: relative err {rel:.3e}"


# ------------------------------------------------------------------------------------
# decode on the presets (scaled-down versions run the oracle on every sequence)
# ------------------------------------------------------------------------------------
SMALL = [
    ("c0", 0, None, None, 1.0),
    ("c1-b24", 1, None, 24, 1.0),
    ("c2-turbo8-b2", 2, 8, 2, 1 / 8),
    ("c2-bf16-b2", 2, 0, 2, 1 / 8),
    ("c3-1/64", 3, None, None, 1 / 64),
    ("c4-b6-1/8", 4, None, 6, 1 / 8),
    ("c1-turbo2-b24", 1, 2, 24, 1.0),
    ("c3-turbo2-1/64", 3, 2, None, 1 / 64),
    ("c2-fp8-b2", 2, 16, 2, 1 / 8),
    ("c1-fp8-b24", 1, 16, 24, 1.0),
    ("c3-fp8-1/64", 3, 16, None, 1 / 64),
]


@pytest.mark.parametrize("name,cfg,dtype,batch,scale", SMALL, ids=[s[0] for s in SMALL])
def test_decode_matches_oracle(name, cfg, dtype, batch, scale):
    _print_case("decode", name)
    W = workloads.config(cfg, dtype=dtype, batch=batch, context_scale=scale)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.num_seqs)}
    fill(cache, W, bt, kv=kv)
    torch.cuda.synchronize()
    _codec_check(W, cache, range(W.num_seqs))
    qb = W.q_bits()
    splits = W.num_splits if W.num_splits and W.max_context_len >= W.num_splits * W.page_size else 0
    got = _decode(W, cache, bt, cl, splits, to_dev(qb))
    for b in range(W.batch):
        want = _oracle_out(W, b, qb, kv[b])
        err = np.max(np.abs(got[b] - want))
        assert err <= TOL, f"{name} seq {b}: max abs err {err:.3e}"


# ------------------------------------------------------------------------------------
# decode on the full presets, in the launch configuration the benchmark uses; the oracle
# recomputes a sample of sequences
# ------------------------------------------------------------------------------------
FULL = [("c1", 1, None, list(range(0, 256, 17))), ("c2-turbo8", 2, 8, [0, 31]),
        ("c2-bf16", 2, 0, [5]), ("c3", 3, None, [0]), ("c4", 4, None, [0, 13, 63]),
        ("c1-turbo2", 1, 2, [0, 100, 255]), ("c2-fp8", 2, 16, [0, 31])]


@pytest.mark.parametrize("name,cfg,dtype,sample", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(name, cfg, dtype, sample):
    """The benchmark's step: one fused launch appends every sequence's newest row (its last
    position again, so the cache stays what the oracle sees) and decodes, in the order of the
    host plan, with the preset's split hint."""
    _print_case("full", name)
    W = workloads.config(cfg, dtype=dtype)
    cache = make_cache(W, fill_byte=None)
    bt, cl = upload_tables(W)
    last = {}
    fill(cache, W, bt, last=last)
    torch.cuda.synchronize()
    B, qb = W.batch, W.q_bits()
    k_new = to_dev(np.stack([last[b][0] for b in range(B)]))
    v_new = to_dev(np.stack([last[b][1] for b in range(B)]))
    order = cache.plan([int(x) for x in W.context_lens], W.num_q_heads, W.max_context_len, W.num_splits)
    out = cache.append_decode(k_new, v_new, to_dev(qb), bt[:B], cl, W.max_context_len, W.softmax_scale,
                              W.num_splits, seq_order=order)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # the codes after the step (the fused append rewrote position L - 1 of every sequence)
    check_codes = sample[:1] + ([W.batch] if W.chunk_tokens else [])
    _codec_check(W, cache, check_codes)
    assert np.all(np.isfinite(got))
    for b in sample:
        want = _oracle_out(W, b, qb)
        err = np.max(np.abs(got[b] - want))
        assert err <= TOL, f"{name} seq {b}: max abs err {err:.3e}"


# ------------------------------------------------------------------------------------
# edge cases and properties
# ------------------------------------------------------------------------------------
# group sizes 1..8 take the paired-block QK layout for turbo4/turbo8, 9..16 the one-block one
@pytest.mark.parametrize("dtype,ps,hq,hkv", [(4, 16, 8, 8), (4, 32, 24, 8), (4, 128, 16, 2),
                                             (4, 256, 8, 1), (3, 64, 6, 2), (8, 64, 14, 2),
                                             (0, 32, 8, 1), (8, 16, 7, 7), (4, 16, 32, 2),
                                             (8, 32, 12, 1), (4, 64, 10, 1), (2, 16, 8, 8),
                                             (2, 64, 40, 8), (2, 32, 32, 2), (16, 16, 8, 8),
                                             (16, 64, 40, 8), (16, 32, 32, 2), (16, 128, 3, 1)])
def test_decode_shapes_and_ragged(dtype, ps, hq, hkv):
    _print_case("shapes", dtype, ps, hq, hkv)
    lens = [0, 1, 15, 17, ps + 3, 3 * ps - 1, 700]
    W = workloads.make(f"shape-{dtype}-{ps}", 300 + dtype, dtype, lens, hq, hkv, ps)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    for splits in (0, 1, 5):
        got = _decode(W, cache, bt, cl, splits, to_dev(qb))
        assert np.all(got[0] == 0)                       # empty context -> zeros
        for b in range(1, W.batch):
            want = _oracle_out(W, b, qb, kv[b])
            err = np.max(np.abs(got[b] - want))
            assert err <= TOL, f"splits {splits} seq {b} (L={lens[b]}): {err:.3e}"


@pytest.mark.parametrize("dtype,hq", [(4, 4), (8, 4), (4, 16), (3, 4), (0, 4), (2, 4), (16, 4), (16, 16)])
def test_query_and_scale_edge_cases(dtype, hq):
    """A zero query gives uniform weights (the mean of the values); a negative softmax scale
    flips the scores; both against the oracle."""
    _print_case("qedge", dtype, hq)
    W = workloads.make(f"qedge-{dtype}-{hq}", 500 + dtype, dtype, [45, 300], hq, 1, 16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    qb[0, :] = 0                       # sequence 0: all-zero query
    for scale in (W.softmax_scale, -W.softmax_scale, 0.0):
        out = cache.decode(to_dev(qb), bt[: W.batch], cl, W.max_context_len, scale, 0)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for b in range(W.batch):
            k, v = kv[b]
            want, _ = oracle.decode_sequence(W.dtype, qb[b], k, v, scale)
            err = np.max(np.abs(got[b] - want))
            assert err <= TOL, f"scale {scale} seq {b}: {err:.3e}"


# The presets (reduced) plus shapes with more than 8 query heads per kv head, whose queries are
# prepared in two passes of eight rows.
DOMINANT = [
    ("c0-turbo4", dict(cfg=0)),
    ("c1-turbo4-b16", dict(cfg=1, batch=16)),
    ("c2-turbo8-b2", dict(cfg=2, dtype=8, batch=2, scale=1 / 8)),
    ("c2-turbo4-b2", dict(cfg=2, dtype=4, batch=2, scale=1 / 8)),
    ("c3-turbo3", dict(cfg=3, scale=1 / 64)),
    ("c3-turbo2", dict(cfg=3, dtype=2, scale=1 / 64)),
    ("c2-fp8-b2", dict(cfg=2, dtype=16, batch=2, scale=1 / 8)),
    ("c2-bf16-b2", dict(cfg=2, dtype=0, batch=2, scale=1 / 8)),
    ("g16-turbo4", dict(dtype=4, hq=16, hkv=1)),
    ("g12-turbo8", dict(dtype=8, hq=12, hkv=1)),
    ("g16-turbo3", dict(dtype=3, hq=32, hkv=2)),
    ("g10-turbo2", dict(dtype=2, hq=10, hkv=1)),
]


@pytest.mark.parametrize("name,spec", DOMINANT, ids=[d[0] for d in DOMINANT])
def test_queries_with_a_dominant_rotated_element(name, spec):
    """The score precision must hold relative to each rotated query element, not only to the
    head's largest: constant offsets 1, 2, 3, 10, 30 on the preset draw and Hadamard-row queries,
    over keys with outlier channels (x20 on the c0/c1 shapes, x30 on c2's), at split counts 0
    and 5, every sequence against the oracle."""
    _print_case("dominant", name)
    if "cfg" in spec:
        W = workloads.config(spec["cfg"], dtype=spec.get("dtype"), batch=spec.get("batch"),
                             context_scale=spec.get("scale", 1.0))
    else:
        W = workloads.make(name, 450 + spec["dtype"], spec["dtype"], [1, 130, 700], spec["hq"],
                           spec["hkv"], 16, outlier_channels=8, outlier_scale=30.0)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.num_seqs)}
    fill(cache, W, bt, kv=kv)
    worst = 0.0
    for kind in (1, 2, 3, 10, 30, "had"):
        qb = dominant_queries(W.q_bits(), kind, seed=W.cfg)
        for splits in (0, 5):
            got = _decode(W, cache, bt, cl, splits, to_dev(qb))
            for b in range(W.batch):
                want = _oracle_out(W, b, qb, kv[b])
                err = np.max(np.abs(got[b] - want))
                worst = max(worst, err)
                assert err <= TOL, f"{name} query {kind} splits {splits} seq {b}: max abs err {err:.3e}"
    print(f"{name}: worst max abs err {worst:.3e}", flush=True)


@pytest.mark.parametrize("dtype,hq", [(4, 16), (4, 96), (3, 40), (0, 16), (2, 16), (16, 32)])
def test_pool_beyond_4gib(dtype, hq):
    """Pools larger than 4 GiB take per-page buffer descriptors and 64-bit page offsets; the
    sequences here live in the pages above the 4 GiB mark."""
    _print_case("bigpool", dtype, hq)
    lens = [300, 45, 1]
    hkv, ps = 8, 16
    block = xq_block_bytes(xq.CacheLayout(dtype, hkv, ps, 1))
    pages = (1 << 32) // (block * hkv) + 64
    W = workloads.make(f"bigpool-{dtype}", 600 + dtype, dtype, lens, hq, hkv, ps, pool_pages=pages)
    top = pages - 1 - np.arange(W.block_tables.size, dtype=np.int64)
    W.block_tables[:] = top.reshape(W.block_tables.shape).astype(W.block_tables.dtype)
    cache = make_cache(W, fill_byte=None)
    assert cache.pool_bytes > (1 << 32)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    for splits in (0, 5):
        got = _decode(W, cache, bt, cl, splits, to_dev(qb))
        for b in range(W.batch):
            want = _oracle_out(W, b, qb, kv[b])
            err = np.max(np.abs(got[b] - want))
            assert err <= TOL, f"splits {splits} seq {b}: {err:.3e}"
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,hq", [(4, 16), (4, 32), (8, 32), (3, 40), (0, 16), (2, 16), (16, 32)])
def test_fixed_partitions_are_batch_invariant(dtype, hq):
    """A negative split hint fixes the partitions: a sequence's output is then bitwise the
    same alone, in the full batch and in a reordered batch with another max_context_len."""
    _print_case("fixed", dtype, hq)
    lens = [700, 33, 1500, 0, 256, 1029, 64, 900]
    W = workloads.make(f"fixed-{dtype}", 700 + dtype, dtype, lens, hq, 8, 16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    q = to_dev(qb)
    hint = -256
    # 64 more table columns (page 0, never read) allow a max_context_len up to 2528
    bt = torch.cat([bt, torch.zeros((bt.shape[0], 64), dtype=bt.dtype, device=bt.device)], 1)

    def run(rows, max_ctx):
        idx = torch.tensor(rows, dtype=torch.long, device="cuda")
        out = cache.decode(q[idx].contiguous(), bt[idx].contiguous(), cl[idx].contiguous(), max_ctx,
                           W.softmax_scale, hint)
        torch.cuda.synchronize()
        return out.cpu()

    full = run(list(range(W.batch)), 2048)
    for b in range(W.batch):
        if lens[b]:
            want = _oracle_out(W, b, qb, kv[b])
            assert np.max(np.abs(full[b].numpy().astype(np.float64) - want)) <= TOL
    for rows, max_ctx in (([2], 1500), ([5, 0, 7, 2], 1536), ([7, 6, 5, 4, 3, 2, 1, 0], 2496)):
        part = run(rows, max_ctx)
        for i, b in enumerate(rows):
            assert torch.equal(part[i], full[b]), f"seq {b} differs in batch {rows}"


def test_splits_agree_and_repeat_is_deterministic():
    _print_case("splits")
    W = workloads.config(1, batch=16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    fill(cache, W, bt)
    q = to_dev(W.q_bits())
    a = _decode(W, cache, bt, cl, 1, q)
    b = _decode(W, cache, bt, cl, 1, q)
    assert np.array_equal(a, b)
    # Split counts change which tokens share a softmax reference and an accumulator, so the
    # fp16 weight split (~22 bits) and the matrix-core accumulation (measured loss below 2^-18
    # of a code step per accumulation) round differently; the inverse rotation sums the 128
    # rotated dimensions into output dimension 0, where such same-signed rounding adds up.
    # Measured on MI355X: 1.4e-5 at most over 2, 8 and 64 splits.
    for s in (2, 8, 64):
        c = _decode(W, cache, bt, cl, s, q)
        print(f"splits {s} against 1: max abs difference {np.max(np.abs(c - a)):.3e}", flush=True)
        assert np.max(np.abs(c - a)) < 2e-5


def test_page_placement_does_not_change_output():
    """Two caches with the same logical content in different physical pages give
    bit-identical outputs (the kernel walks pages in logical order)."""
    _print_case("placement")
    W1 = workloads.make("placeA", 400, 4, [300, 45], 8, 2, 16, permute=False)
    W2 = workloads.make("placeA", 400, 4, [300, 45], 8, 2, 16, pool_pages=64)
    outs = []
    for W in (W1, W2):
        cache = make_cache(W)
        bt, cl = upload_tables(W)
        fill(cache, W, bt)
        outs.append(_decode(W, cache, bt, cl, 0))
    assert np.array_equal(outs[0], outs[1])


def test_shared_prefix_pages():
    """Two sequences may point at the same physical pages (a shared prefix)."""
    _print_case("shared")
    W = workloads.make("shared", 401, 4, [64, 64], 8, 2, 16)
    W.block_tables[1] = W.block_tables[0]
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    fill(cache, W, bt, seqs=[0])
    qb = W.q_bits()
    qb[1] = qb[0]
    got = _decode(W, cache, bt, cl, 0, to_dev(qb))
    assert np.array_equal(got[0], got[1])


@pytest.mark.parametrize("dtype", [4, 8, 3, 0, 16])
def test_planned_decode_is_bitwise_the_plain_decode(dtype):
    """xq_decode_plan only changes which wave runs which sequence: the planned decode equals the
    plain one bit for bit (and the oracle within the bar), on a batch large enough for the plan
    to move sequences."""
    _print_case("planned", dtype)
    W = workloads.config(1, dtype=dtype, context_scale=0.25)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    q = to_dev(qb)
    order = cache.plan([int(x) for x in W.context_lens], W.num_q_heads, W.max_context_len, 0)
    assert sorted(order.cpu().tolist()) == list(range(W.batch))
    assert order.cpu().tolist() != list(range(W.batch))
    plain = cache.decode(q, bt[: W.batch], cl, W.max_context_len, W.softmax_scale, 0)
    planned = cache.decode(q, bt[: W.batch], cl, W.max_context_len, W.softmax_scale, 0, seq_order=order)
    torch.cuda.synchronize()
    assert torch.equal(plain, planned)
    got = planned.cpu().numpy().astype(np.float64)
    for b in (0, 37, 128, 255):
        want = _oracle_out(W, b, qb, kv[b])
        assert np.max(np.abs(got[b] - want)) <= TOL


def test_planned_decode_with_identity_and_unit_plans():
    """A batch that is not a multiple of 8 with one partition per sequence: the plan is the identity;
    with several partitions it is a unit placement. Either way the planned call equals the plain one
    bit for bit, an empty sequence (whose output is zeros) included."""
    _print_case("planned-identity")
    lens = [300, 45, 700, 1, 1029, 0, 9]
    W = workloads.make("plan-id", 960, 4, lens, 16, 8, 16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    fill(cache, W, bt)
    q = to_dev(W.q_bits())
    for splits in (1, 4, 0):
        order = cache.plan(lens, 16, W.max_context_len, splits)
        if splits == 1:
            assert order.cpu().tolist() == list(range(len(lens)))
        else:
            # (the library's own choice for 7 sequences of up to 1,029 tokens: 17 partitions of 64)
            assert order.numel() == (4 if splits == 4 else 17) * 8 * len(lens)
        a = cache.decode(q, bt, cl, W.max_context_len, W.softmax_scale, splits)
        b = cache.decode(q, bt, cl, W.max_context_len, W.softmax_scale, splits, seq_order=order)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert not torch.any(b[5])
