"""Benchmark of one decode step over a TurboQuant paged KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--no-cpu]

A step is one pass of the whole hot path for one layer of a decode batch:
  1. the new K/V rows are rotated, quantized, packed and stored in their pages: every
     sequence's new row, plus the prefill chunk where the workload has one;
  2. decode attention over every sequence's paged, quantized context.
By default one xq_append_decode_attention launch does both for the decode batch (a chunk still
goes through xq_quantize_append first); --no-fuse runs xq_quantize_append and the decode as two
launches. The decode uses the host plan (xq_decode_plan) unless --no-plan.

Steps are timed twice, K each after W warm-up steps: eagerly, with HIP events around every
decode call (the roofline's launch duration), and replayed from HIP graphs captured per pool
replica, the way a serving engine replays its decode step; when every replica has its graph,
also from one graph holding a step on each replica in turn, as a model's decode graph holds one
step per layer (K steps = K // R replays of it + K mod R single-step replays). `value` and
`ms_per_step` come from that graph, else from the single-step graphs when every replica has
one, else (--no-graph) from the eager launches; all figures are in `step_timing`.
The new row of sequence b goes to position L_b - 1, so every step has the same shape and
the cache content stays what the oracle computes.

Inputs are seeded synthetic draws (workloads/), resident in HBM before timing starts.
Steps rotate over R copies of the K/V pools, R x footprint >= 1 GiB, so the 256 MB
Infinity Cache cannot serve the KV reads of one step from the previous ones.

Prints ONE JSON line. `value` is KV GB/s: the algorithmic KV bytes the decode reads per
step (sum_b L_b * Hkv * 2 * row_bytes) over the whole step time. `roofline` is for the
decode call, which is the dominant work of the step: decode_split_kernel and, when a
sequence spans several partitions, decode_combine_kernel, timed together with HIP events
around each decode call on its stream inside the timed region (the rocprofv3 summary under
profiles/ lists the kernels separately); `traffic` is the measured HBM bytes of
those kernels per call. `cpu_baseline` is the oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded inputs; no arithmetic of the method)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "bit_quantized_paged_turbo_amd", "csrc", "decode_attention.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, help="workload preset 0..4 (default 1)")
    ap.add_argument("--dtype", type=int, default=None, help="override the preset's cache type")
    ap.add_argument("--splits", type=int, default=None, help="override the split hint")
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunk-prefill timing")
    ap.add_argument("--no-plan", action="store_true", help="decode without the host plan")
    ap.add_argument("--no-fuse", action="store_true",
                    help="append the batch's new rows in their own launch instead of the decode's")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run plain 512 MiB device copies (a known byte count for "
                         "scaling HBM counters)")
    return ap.parse_args()


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def row_bytes(dtype: int) -> int:
    return 256 if dtype == 0 else 128 if dtype == workloads.FP8 else 16 * dtype + 2


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(kernel_tag: str):
    """HBM bytes per launch from a committed counter summary, or None when there is none
    or the decode kernel's source has changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel_tag}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_digest(DECODE_SRC):
        return None
    return float(t.group(1))


class Step:
    """Precomputed ctypes arguments for the two calls of one step on one replica."""

    def __init__(self, lib, layout, cache, app, dec):
        import ctypes
        self.lib = lib
        self.L = ctypes.byref(layout)
        self.cache = cache
        self.app, self.dec = app, dec

    def run(self, stream: int):
        if self.app is None:            # the fused step appends inside the decode launch
            return
        lib = self.lib
        c = self.cache
        kp, vp = c.k_pool.data_ptr(), c.v_pool.data_ptr()
        st = lib.xq_quantize_append(self.L, *self.app, kp, vp, stream)
        if st:
            raise RuntimeError(lib.xq_last_error().decode())

    def decode(self, stream: int):
        lib = self.lib
        c = self.cache
        q, batch, hq, bt, maxp, cl, maxctx, scale, splits, ws, wsb, out, order, fused = self.dec
        if fused is not None:
            st = lib.xq_append_decode_attention(self.L, fused[0], fused[1], q, batch, hq, c.k_pool.data_ptr(),
                                                c.v_pool.data_ptr(), bt, maxp, cl, maxctx, scale, splits,
                                                ws, wsb, out, order, stream)
        elif order is None:
            st = lib.xq_paged_decode_attention(self.L, q, batch, hq, c.k_pool.data_ptr(),
                                               c.v_pool.data_ptr(), bt, maxp, cl, maxctx, scale,
                                               splits, ws, wsb, out, stream)
        else:
            st = lib.xq_paged_decode_attention_planned(self.L, q, batch, hq, c.k_pool.data_ptr(),
                                                       c.v_pool.data_ptr(), bt, maxp, cl, maxctx,
                                                       scale, splits, ws, wsb, out, order, stream)
        if st:
            raise RuntimeError(lib.xq_last_error().decode())


def time_prefill(lib, cache, W, bt, to_dev, stream, K, Wm):
    """The chunk's queries attending causally to the chunk (xq_paged_prefill_attention from
    position 0 over the chunk's appended rows): HIP events around each call on its stream."""
    import torch
    n, hq = W.chunk_tokens, W.num_q_heads
    g = np.random.default_rng(7)
    q = to_dev(workloads.round_to_bf16_bits(g.standard_normal((n, hq, 128)).astype(np.float32)))
    row = bt[W.batch]
    for _ in range(Wm):
        cache.prefill(q, row, 0, W.softmax_scale)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        cache.prefill(q, row, 0, W.softmax_scale)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    pairs = n * (n + 1) // 2                      # (query, key) pairs of the causal chunk
    flops = 4 * 128 * hq * pairs                  # QK and PV multiply-adds
    rows_bytes = n * W.num_kv_heads * 2 * row_bytes(W.dtype)
    log(f"prefill of the {n}-token chunk: {ms * 1e3:.1f} us")
    return {"queries": n, "start": 0, "call_us": round(ms * 1e3, 2),
            "query_tokens_per_s": round(n / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 3), "flops_per_call": flops,
            "kv_bytes_once": rows_bytes,
            "note": "the decode kernel with 16/g query tokens x g heads in the 16 matrix-core "
                    "columns of a unit; each unit reads its causal prefix (from L2/MALL for this "
                    "chunk)"}


def cpu_baseline(W, seconds: float):
    """The oracle on the host: per sequence, quantize its new row and attend over its
    (already quantized) context, sequence after sequence, for about `seconds`."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):              # one host thread (numpy's own loops are serial)
        return _cpu_baseline(oracle, W, seconds)


def _cpu_baseline(oracle, W, seconds: float):
    qb = W.q_bits()
    rb = row_bytes(W.dtype)
    done_seqs = done_bytes = done_tokens = 0
    elapsed = 0.0
    prepared = {}                    # sequence -> its context rows, quantized once, untimed
    b = 0
    while elapsed < seconds:
        if b not in prepared:
            k, v = W.kv_bits(b)
            if W.dtype == workloads.FP8:
                prepared[b] = (k[-1:], v[-1:], oracle.fp8_encode_rows_bf16(k[:-1]),
                               oracle.fp8_encode_rows_bf16(v[:-1]))
            elif W.dtype:
                prepared[b] = (k[-1:], v[-1:], oracle.quantize_rows_bf16(k[:-1], W.dtype),
                               oracle.quantize_rows_bf16(v[:-1], W.dtype))
            else:
                prepared[b] = (k, v)
        t0 = time.perf_counter()
        if W.dtype == workloads.FP8:
            k1, v1, kf, vf = prepared[b]
            kf2 = np.concatenate([kf, oracle.fp8_encode_rows_bf16(k1)])
            vf2 = np.concatenate([vf, oracle.fp8_encode_rows_bf16(v1)])
            oracle.decode_attention_fp8(qb[b], kf2, vf2, W.softmax_scale)
        elif W.dtype:
            k1, v1, (kc, ks), (vc, vs) = prepared[b]
            nk = oracle.quantize_rows_bf16(k1, W.dtype)
            nv = oracle.quantize_rows_bf16(v1, W.dtype)
            kc2, ks2 = np.concatenate([kc, nk[0]]), np.concatenate([ks, nk[1]])
            vc2, vs2 = np.concatenate([vc, nv[0]]), np.concatenate([vs, nv[1]])
            oracle.decode_attention_turbo(qb[b], kc2, ks2, vc2, vs2, W.softmax_scale)
        else:
            k, v = prepared[b]
            oracle.decode_attention_bf16(qb[b], k, v, W.softmax_scale)
        elapsed += time.perf_counter() - t0
        L = int(W.context_lens[b])
        done_seqs += 1
        done_tokens += L
        done_bytes += L * W.num_kv_heads * 2 * rb
        if done_seqs % 256 == 0:
            log(f"oracle: {done_seqs} sequences, {elapsed:.1f} s timed")
        b = (b + 1) % W.batch
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s",
            "seq_tokens_per_s": round(done_tokens / elapsed, 1), "cores": 1, "kind": "oracle",
            "sample": f"{done_seqs} sequence-decodes cycling over sequences of the same "
                      f"workload: quantize the step's new K/V row, then float64 decode "
                      f"attention over the quantized context; {elapsed:.1f} s on 1 host thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode path runs on one GPU with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_paged_turbo_amd as xq
    import workloads
    from bit_quantized_paged_turbo_amd.cache import PagedKVCache

    lib = xq.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = "cuda"

    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 copies of {n} bytes")

    W = workloads.config(args.config, dtype=args.dtype)
    log(f"workload {W.name}: batch {W.batch}, {W.total_tokens()} context tokens")
    splits = W.num_splits if args.splits is None else args.splits

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # ---- fill one replica with every sequence's context through the append path --------
    base = PagedKVCache(W.dtype, W.num_kv_heads, W.page_size, W.num_pages)
    bt = to_dev(W.block_tables.astype(np.int32))
    last_k, last_v = [], []
    chunk_kv = None
    pend = []
    for b in range(W.num_seqs):
        L = W.seq_len(b)
        k, v = W.kv_bits(b)
        if b < W.batch:
            last_k.append(k[-1])
            last_v.append(v[-1])
        else:
            chunk_kv = (k, v)
        pend.append((k, v, np.full(L, b, np.int32), np.arange(L, dtype=np.int32)))
        if sum(len(p[2]) for p in pend) >= (1 << 19) or b == W.num_seqs - 1:
            cat = [np.concatenate([p[i] for p in pend]) for i in range(4)]
            base.append(to_dev(cat[0]), to_dev(cat[1]), to_dev(cat[2]), to_dev(cat[3]), bt)
            pend = []
    torch.cuda.synchronize()

    log("cache filled through xq_quantize_append")
    footprint = 2 * base.pool_bytes
    R = max(1, int(np.ceil(args.replica_bytes / footprint)))
    caches = [base]
    for _ in range(R - 1):
        c = PagedKVCache(W.dtype, W.num_kv_heads, W.page_size, W.num_pages)
        c.k_pool.copy_(base.k_pool)
        c.v_pool.copy_(base.v_pool)
        caches.append(c)
    torch.cuda.synchronize()

    # ---- step inputs -------------------------------------------------------------------
    B, hq, hkv = W.batch, W.num_q_heads, W.num_kv_heads
    new_k = to_dev(np.stack(last_k))
    new_v = to_dev(np.stack(last_v))
    new_seq = to_dev(np.arange(B, dtype=np.int32))
    new_pos = to_dev((W.context_lens - 1).astype(np.int32))
    q = to_dev(W.q_bits())
    cl = to_dev(W.context_lens.astype(np.int32))
    out = torch.empty((B, hq, 128), dtype=torch.float32, device=dev)
    wsb = base.workspace_bytes(B, hq, W.max_context_len, splits)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev)
    maxp = W.max_pages_per_seq
    app = (new_k.data_ptr(), new_v.data_ptr(), B, new_seq.data_ptr(), new_pos.data_ptr(),
           bt.data_ptr(), maxp)
    chunk = None
    fuse = not args.no_fuse
    if chunk_kv is not None:
        # one append per step takes every new row that the decode launch does not: the chunk's, and
        # without the fused step the decode batch's own too
        nb = 0 if fuse else B
        ck = to_dev(np.concatenate([chunk_kv[0]] + ([] if fuse else [np.stack(last_k)])))
        cv = to_dev(np.concatenate([chunk_kv[1]] + ([] if fuse else [np.stack(last_v)])))
        cs = to_dev(np.concatenate([np.full(W.chunk_tokens, W.batch, np.int32), np.arange(nb, dtype=np.int32)]))
        cp = to_dev(np.concatenate([np.arange(W.chunk_tokens, dtype=np.int32),
                                    (W.context_lens[:nb] - 1).astype(np.int32)]))
        keep = (ck, cv, cs, cp)
        app = (ck.data_ptr(), cv.data_ptr(), W.chunk_tokens + nb, cs.data_ptr(), cp.data_ptr(),
               bt.data_ptr(), maxp)
        chunk = True
    elif fuse:
        app = None
    # the host plan: long and short sequences share SIMDs (identity where it cannot help)
    order = None
    if not args.no_plan:
        order = base.plan([int(x) for x in W.context_lens], hq, W.max_context_len, splits, device=dev)
    dec = (q.data_ptr(), B, hq, bt.data_ptr(), maxp, cl.data_ptr(), W.max_context_len,
           W.softmax_scale, splits, ws.data_ptr(), wsb, out.data_ptr(),
           None if order is None else order.data_ptr(),
           (new_k.data_ptr(), new_v.data_ptr()) if fuse else None)
    runners = [Step(lib, c.layout, c, app, dec) for c in caches]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    log(f"{R} pool replicas of {footprint} bytes; timing")
    K, Wm = args.steps, args.warmup
    for i in range(Wm):
        r = runners[i % R]
        r.run(sp)
        r.decode(sp)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        r = runners[(Wm + i) % R]
        r.run(sp)
        ev[i][0].record(stream)
        r.decode(sp)
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / K
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec_avg_ms = float(dec_ms.mean())

    # ---- the same steps replayed from captured HIP graphs (one per pool replica): the library
    # allocates, clears and waits on nothing, so a step captures whole ---------------------------
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for r in runners[:64]:
                r.run(side.cuda_stream)
                r.decode(side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for r in runners[:64]:         # tiny workloads have thousands of replicas: cap the graphs
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                r.run(cs)
                r.decode(cs)
            graphs.append(g)
        torch.cuda.synchronize()
        NG = len(graphs)
        for i in range(Wm):
            graphs[i % NG].replay()
        torch.cuda.synchronize()
        gstart, gstop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gstart.record(stream)
        for i in range(K):
            graphs[(Wm + i) % NG].replay()
        gstop.record(stream)
        torch.cuda.synchronize()
        g_ms = gstart.elapsed_time(gstop) / K
        graph = {"ms_per_step": round(g_ms, 5), "replicas": NG}
        log(f"graph replay: {g_ms * 1e3:.1f} us/step")
        # One graph holding a step on every replica in turn, as a model's decode graph holds one
        # step per layer (the replicas' pools stand for the layers' caches): K steps are K // NG
        # replays of it plus K % NG single-step replays.
        if NG == R and R > 1:
            layers = torch.cuda.CUDAGraph()
            with torch.cuda.graph(layers):
                cs = torch.cuda.current_stream().cuda_stream
                for r in runners:
                    r.run(cs)
                    r.decode(cs)
            torch.cuda.synchronize()
            for _ in range(max(1, Wm // R)):
                layers.replay()
            torch.cuda.synchronize()
            gstart.record(stream)
            for _ in range(K // R):
                layers.replay()
            for i in range(K % R):
                graphs[i].replay()
            gstop.record(stream)
            torch.cuda.synchronize()
            m_ms = gstart.elapsed_time(gstop) / K
            graph["multi_step_ms_per_step"] = round(m_ms, 5)
            graph["steps_per_graph"] = R
            log(f"graph of {R} steps: {m_ms * 1e3:.1f} us/step")
            del layers
        del graphs

    rb = row_bytes(W.dtype)
    kv_bytes = int(W.context_lens.astype(np.int64).sum()) * hkv * 2 * rb
    tokens = int(W.context_lens.astype(np.int64).sum())
    nsplits = xq.xq_decode_num_splits(base.layout, B, hq, W.max_context_len, splits)
    # The reported step time: the steps replayed from HIP graphs (as a serving engine replays its
    # decode step), R to a graph where possible, when every pool replica has its graph; else the
    # eager launches.
    by_graph = graph is not None and graph["replicas"] == R
    by_layers = by_graph and "multi_step_ms_per_step" in graph
    timed_ms = graph["multi_step_ms_per_step"] if by_layers else graph["ms_per_step"] if by_graph else step_ms
    value = kv_bytes / (timed_ms * 1e-3) / 1e9
    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    tag = f"decode_call_{workloads.DTYPE_NAMES[W.dtype]}_{W.name}"
    traffic = committed_traffic(tag)

    result = {
        "metric": "quantized paged decode attn: KV GB/s (% of HBM peak) and seq-tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(timed_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {4: "i4xi16->i32 QK, f32 softmax/PV", 3: "i3xi16->i32 QK, f32 softmax/PV",
                  2: "i2xi16->i32 QK, f32 softmax/PV", 8: "i8xi16->i32 QK, f32 softmax/PV",
                  0: "bf16xbf16->f32", workloads.FP8: "e4m3->bf16, bf16xbf16->f32"}[W.dtype],
        "data": "synthetic",
        "config": {
            "workload": W.name, "description": W.note, "cache": workloads.DTYPE_NAMES[W.dtype],
            "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
            "page_size": W.page_size, "context_tokens": tokens, "max_context": W.max_context_len,
            "splits": nsplits, "chunk_append_tokens": W.chunk_tokens, "pool_replicas": R,
            "plan": order is not None and order.cpu().tolist() != list(range(B)),
            "fused_append": fuse,
        },
        "step_timing": {"method": (f"hip graph replay, {R} steps (one per pool replica, as one per layer) per graph"
                                   if by_layers else "hip graph replay of the captured step" if by_graph
                                   else "eager launches"),
                        "eager_ms_per_step": round(step_ms, 5),
                        "eager_value": round(kv_bytes / (step_ms * 1e-3) / 1e9, 2),
                        "graph_ms_per_step": graph["ms_per_step"] if graph is not None else None,
                        "multi_step_graph_ms_per_step": graph.get("multi_step_ms_per_step") if graph is not None else None,
                        "graph_replicas": graph["replicas"] if graph is not None else None},
        "seq_tokens_per_s": round(tokens / (timed_ms * 1e-3), 1),
        "decode_seqs_per_s": round(B / (timed_ms * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_call_us": {"mean": round(dec_avg_ms * 1e3, 2),
                           "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                           "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": ("xq_append_decode_attention" if fuse else "xq_paged_decode_attention")
                               + " call (decode_split_kernel"
                               + (" + decode_combine_kernel)" if nsplits > 1 else ")"),
                     "bytes_per_launch": kv_bytes},
    }
    if chunk is not None and not args.no_prefill:
        result["prefill"] = time_prefill(lib, base, W, bt, to_dev, stream, K, Wm)
    log(f"GPU: {step_ms * 1e3:.1f} us/step eager, "
        f"{'%.1f' % (graph['ms_per_step'] * 1e3) if graph is not None else '-'} us/step graph, "
        f"decode call {dec_avg_ms * 1e3:.1f} us")
    if not args.no_cpu:
        log("oracle baseline on the host")
        result["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
