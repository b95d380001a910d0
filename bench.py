"""Benchmark of one decode step over a TurboQuant paged KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--no-cpu]

A step is one pass of the whole hot path for one layer:
  1. new K/V rows are rotated, quantized, packed and stored in their pages: every decoded
     sequence's new row, plus the prefill chunk where the workload has one (the default, the
     mixed step: a 2,048-token chunk appended for a new sequence, then a batch of 64 decodes);
  2. decode attention over every sequence's paged, quantized context.
By default one decode launch does all of it: it appends the batch's new rows, decodes, and
appends the chunk's rows with workgroups after its units (--chunk-append kernel: the chunk goes
through xq_quantize_append first); --no-fuse runs xq_quantize_append and the decode as two
launches. The decode runs over a length-aware plan by default (xq_decode_plan_balanced: each
sequence gets its own partition size, all work units about equal); --plan uniform takes the split
hint's partitions placed by xq_decode_plan, --plan none (or --no-plan) neither.

Steps are timed twice, K each after W warm-up steps (and as many more untimed ones as bring the
warm-up to 30 ms of GPU work, so that the clocks have left idle): eagerly, with HIP events around every
decode call and every append call (on the stream they are launched on), and replayed from HIP
graphs captured per pool replica, the way a serving engine replays its decode step; when every
replica has its graph, also from one graph holding a step on each replica in turn (8 steps when
there is one replica), as a model's decode graph holds one step per layer. `value` and `ms_per_step` come from the graph replay,
else (--no-graph) from the eager launches; all figures are in `step_timing`. The new row of
sequence b goes to position L_b - 1, so every step has the same shape and the cache content
stays what the oracle computes.

Inputs are seeded synthetic draws (workloads/), resident in HBM before timing starts. Steps
rotate over R copies of the K/V pools, R x footprint >= 1 GiB, so the 256 MB Infinity Cache
cannot serve one step's KV reads from the previous ones.

Prints ONE JSON line. `value` is KV GB/s: the algorithmic KV bytes the decode reads per step
(sum_b L_b * Hkv * 2 * row_bytes) over the whole step time. `roofline` is for the decode call,
the dominant work of the step (decode_split_kernel, plus decode_combine_kernel when a sequence
spans several partitions): achieved = those bytes / the mean duration of the decode call, from
one HIP event pair around replays of a graph holding only decode calls back to back (eager
per-call events, also reported, include the host's launch gaps; without graphs they are used); `frac_kernel_trace` is the same bytes over the kernels' mean
duration in the committed rocprofv3 summary of this command (while the kernel sources are the
ones it was taken on); `traffic` is the HBM bytes the counters measured per call.
`hbm_reference` is a plain streaming-read kernel over 4 GiB (sequentially, and in 1 KiB blocks
gathered in a random order, the decode's pattern). `append` reports the quantize-append kernel's
own rate. `cpu_baseline` is the oracle (oracle/, float64 attention over the quantized cache) on
the host's cores, in worker processes started before anything touches the GPU.
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import multiprocessing as mp
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
CSRC = os.path.join(ROOT, "bit_quantized_paged_turbo_amd", "csrc")
DECODE_SOURCES = [os.path.join(CSRC, f) for f in ("decode_attention.hip", "row_codec.h")]
MAX_WORKERS = 16               # the machine's CPU share for one GPU


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4, help="workload preset 0..4 (default 4, the mixed step)")
    ap.add_argument("--dtype", type=int, default=None, help="override the preset's cache type")
    ap.add_argument("--splits", type=int, default=None, help="override the split hint")
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="oracle worker processes (default: the host's cores, at most 16)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="timed oracle repetitions (median)")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunk-prefill timing")
    ap.add_argument("--chunk-append", choices=("decode", "kernel"), default="decode",
                    help="where the prefill chunk's rows are appended with the length-aware plan and the "
                         "fused step: by the decode launch (default) or by a separate append kernel")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--plan", choices=("balanced", "uniform", "none"), default="balanced",
                    help="host plan of the decode: length-aware partitions (xq_decode_plan_balanced), "
                         "the split hint's partitions placed by xq_decode_plan, or none")
    ap.add_argument("--no-plan", action="store_true", help="the same as --plan none")
    ap.add_argument("--no-fuse", action="store_true",
                    help="append the batch's new rows in their own launch instead of the decode's")
    ap.add_argument("--serial-draws", action="store_true",
                    help="draw the inputs in this process (no worker pool; for profiler runs, whose "
                         "library has the GPU initialised before the program starts)")
    ap.add_argument("--inputs-cache", default=None,
                    help="an .npz of the drawn K/V rows: loaded if it exists, else written after drawing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run plain 512 MiB device copies (a known byte count for "
                         "scaling HBM counters)")
    return ap.parse_args()


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def row_bytes(dtype: int) -> int:
    return 256 if dtype == 0 else 128 if dtype == workloads.FP8 else 16 * dtype + 2


def sources_digest() -> str:
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_profile(tag: str):
    """Figures from the committed rocprofv3 summaries of this workload, or None where there is no
    summary or the decode sources have changed since it was taken: (kernel-trace mean
    microseconds of the decode call's kernels, HBM bytes per call from the counters)."""
    out = {}
    for kind, key in (("kernel_trace", "decode_call_kernel_us"), ("pmc", "hbm_bytes_per_launch")):
        path = os.path.join(PROFILES, f"{tag}_{kind}.txt")
        if not os.path.exists(path):
            continue
        text = open(path).read()
        m = re.search(r"sources_sha256_16:\s*([0-9a-f]{16})", text)
        t = re.search(key + r":\s*([0-9.eE+]+)", text)
        if m and t and m.group(1) == sources_digest():
            out[key] = float(t.group(1))
    return out


def host_info() -> dict:
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


# ---------------------------------------------------------------------------------------------
# Host work in worker processes, forked before the GPU is touched: the seeded draws (which the
# GPU's cache is filled from) and the oracle baseline.
# ---------------------------------------------------------------------------------------------
_W = None


def _pool_init(cfg, dtype):
    global _W
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    _W = workloads.config(cfg, dtype=dtype)


def _draw(b):
    return b, _W.kv_bits(b)


def _balanced(lens, n):
    """Sequences dealt to n workers, longest first, each to the least loaded."""
    loads, parts = [0] * n, [[] for _ in range(n)]
    for b in sorted(range(len(lens)), key=lambda i: -int(lens[i])):
        w = int(np.argmin(loads))
        parts[w].append(b)
        loads[w] += int(lens[b])
    return parts


def _oracle_worker(wid, cfg, dtype, seqs, chunk_rows, reps, barrier, results):
    """One oracle worker: its sequences' context rows quantized once (untimed), then per
    repetition (the first a warm-up), between barriers: (a) quantize the step's new rows (each of
    its sequences' row L - 1 and its slice of the chunk), (b) decode its sequences in float64 over
    the quantized context."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    import oracle
    W = workloads.config(cfg, dtype=dtype)
    fp8 = W.dtype == workloads.FP8
    ctx, new = {}, {}
    for b in seqs:
        k, v = W.kv_bits(b)
        new[b] = (k[-1:], v[-1:])
        if W.dtype == 0:
            ctx[b] = (k[:-1], v[:-1])
        elif fp8:
            ctx[b] = (oracle.fp8_encode_rows_bf16(k[:-1]), oracle.fp8_encode_rows_bf16(v[:-1]))
        else:
            ctx[b] = (oracle.quantize_rows_bf16(k[:-1], W.dtype), oracle.quantize_rows_bf16(v[:-1], W.dtype))
    chunk = None
    if chunk_rows is not None:
        k, v = W.kv_bits(W.batch)
        chunk = (k[chunk_rows[0]:chunk_rows[1]], v[chunk_rows[0]:chunk_rows[1]])
    qb = W.q_bits()

    def encode(rows):
        if W.dtype == 0:
            return rows
        if fp8:
            return oracle.fp8_encode_rows_bf16(rows)
        return oracle.quantize_rows_bf16(rows, W.dtype)

    times = []
    for _ in range(reps + 1):
        barrier.wait()
        t0 = time.perf_counter()
        enc = {b: (encode(new[b][0]), encode(new[b][1])) for b in seqs}
        if chunk is not None:
            encode(chunk[0])
            encode(chunk[1])
        t1 = time.perf_counter()
        barrier.wait()
        t2 = time.perf_counter()
        for b in seqs:
            (kc, vc), (kn, vn) = ctx[b], enc[b]
            if W.dtype == 0:
                oracle.decode_attention_bf16(qb[b], np.concatenate([kc, kn]), np.concatenate([vc, vn]),
                                             W.softmax_scale)
            elif fp8:
                oracle.decode_attention_fp8(qb[b], np.concatenate([kc, kn]), np.concatenate([vc, vn]),
                                            W.softmax_scale)
            else:
                oracle.decode_attention_turbo(qb[b], np.concatenate([kc[0], kn[0]]), np.concatenate([kc[1], kn[1]]),
                                              np.concatenate([vc[0], vn[0]]), np.concatenate([vc[1], vn[1]]),
                                              W.softmax_scale)
        t3 = time.perf_counter()
        times.append((t0, t1, t2, t3))
    results.put((wid, times))


def cpu_baseline(W, workers: int, reps: int) -> dict:
    """The oracle on `workers` host processes (one thread each) over the whole step of the
    workload: quantize the step's new rows, then decode every sequence; each phase timed across
    all workers (earliest start to latest end), median of `reps` after one warm-up."""
    ctx = mp.get_context("fork")
    parts = _balanced(W.context_lens, workers)
    chunk_parts = [None] * workers
    if W.chunk_tokens:
        edges = np.linspace(0, W.chunk_tokens, workers + 1).astype(int)
        chunk_parts = [(int(edges[i]), int(edges[i + 1])) for i in range(workers)]
    barrier = ctx.Barrier(workers)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(w, W.cfg, W.dtype, parts[w], chunk_parts[w], reps, barrier,
                                                      results)) for w in range(workers)]
    t_start = time.perf_counter()
    for p in procs:
        p.start()
    got = [results.get() for _ in procs]
    for p in procs:
        p.join()
        if p.exitcode != 0:
            raise RuntimeError(f"oracle worker exited with {p.exitcode}")
    wall = time.perf_counter() - t_start
    quant, dec = [], []
    for r in range(1, reps + 1):
        quant.append(max(t[r][1] for _, t in got) - min(t[r][0] for _, t in got))
        dec.append(max(t[r][3] for _, t in got) - min(t[r][2] for _, t in got))
    tq, td = float(np.median(quant)), float(np.median(dec))
    kv_bytes = int(W.context_lens.astype(np.int64).sum()) * W.num_kv_heads * 2 * row_bytes(W.dtype)
    tokens = int(W.context_lens.sum())
    new_rows = (W.batch + W.chunk_tokens) * W.num_kv_heads * 2
    return {"value": round(kv_bytes / (tq + td) / 1e9, 4), "unit": "GB/s",
            "seq_tokens_per_s": round(tokens / (tq + td), 1), "cores": workers, "kind": "oracle",
            "quantize_s": round(tq, 5), "decode_s": round(td, 5),
            "quantize_rows_per_s": round(new_rows / tq, 1), "decode_kv_GBps": round(kv_bytes / td / 1e9, 4),
            "reps": reps, "wall_s_incl_setup": round(wall, 2), **host_info(),
            "sample": f"the whole step of {W.name}: quantize its {new_rows} new K/V rows "
                      f"({W.chunk_tokens}-token chunk + one row per sequence), then float64 decode of "
                      f"all {W.batch} sequences ({tokens} context tokens) over the quantized cache; "
                      f"{workers} worker processes x 1 thread, each phase timed from the earliest "
                      f"worker start to the latest end, median of {reps} after a warm-up; the "
                      f"context rows are quantized once beforehand, untimed"}


# ---------------------------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------------------------
class Step:
    """Precomputed ctypes arguments for the calls of one step on one replica."""

    def __init__(self, lib, layout, cache, app, dec):
        import ctypes
        self.lib = lib
        self.L = ctypes.byref(layout)
        self.cache = cache
        self.app, self.dec = app, dec

    def run(self, stream: int):
        if self.app is None:            # the fused step appends inside the decode launch
            return
        c = self.cache
        st = self.lib.xq_quantize_append(self.L, *self.app, c.k_pool.data_ptr(), c.v_pool.data_ptr(), stream)
        if st:
            raise RuntimeError(self.lib.xq_last_error().decode())

    def decode(self, stream: int):
        lib = self.lib
        c = self.cache
        q, batch, hq, bt, maxp, cl, maxctx, scale, splits, ws, wsb, out, order, n_order, fused, bal, chunk = self.dec
        if bal is not None:
            kn, vn = fused if fused is not None else (None, None)
            ck, cv, cn, cs, cp = chunk if chunk is not None else (None, None, 0, None, None)
            st = lib.xq_decode_attention_balanced(self.L, q, batch, hq, c.k_pool.data_ptr(), c.v_pool.data_ptr(),
                                                  bt, maxp, cl, maxctx, scale, bal[0], bal[1], bal[2], kn, vn,
                                                  ck, cv, cn, cs, cp, ws, wsb, out, stream)
        elif fused is not None:
            st = lib.xq_append_decode_attention(self.L, fused[0], fused[1], q, batch, hq, c.k_pool.data_ptr(),
                                                c.v_pool.data_ptr(), bt, maxp, cl, maxctx, scale, splits,
                                                ws, wsb, out, order, n_order, stream)
        elif order is None:
            st = lib.xq_paged_decode_attention(self.L, q, batch, hq, c.k_pool.data_ptr(),
                                               c.v_pool.data_ptr(), bt, maxp, cl, maxctx, scale,
                                               splits, ws, wsb, out, stream)
        else:
            st = lib.xq_paged_decode_attention_planned(self.L, q, batch, hq, c.k_pool.data_ptr(),
                                                       c.v_pool.data_ptr(), bt, maxp, cl, maxctx,
                                                       scale, splits, ws, wsb, out, order, n_order, stream)
        if st:
            raise RuntimeError(lib.xq_last_error().decode())


def warm(step, n: int, stream, min_ms: float = 30.0) -> int:
    """The W untimed warmup steps (step(i) runs step i), then more untimed steps until the warmup
    has kept the GPU busy for min_ms, so that its clocks have left idle (the host's oracle run and
    the graph captures leave it idle for seconds) before the timed steps. -> steps run."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    i = 0
    while i < max(n, 1):
        step(i)
        i += 1
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    if ms < min_ms:
        for _ in range(int(math.ceil((min_ms - ms) / max(ms / i, 1e-3)))):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return i


def event_pairs(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def hbm_reference(xq, stream, reps: int = 5) -> dict:
    """A plain streaming-read kernel over 4 GiB: one sequential stream, and 1 KiB blocks in a
    random order (the decode's gather of page blocks). Best and median of `reps` launches.
    `stream` is the torch stream: events are recorded on it, the library gets its handle."""
    import torch
    assert isinstance(stream, torch.cuda.Stream)
    sh = stream.cuda_stream
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nblk = nbytes // 1024
    order_h = np.random.default_rng(11).permutation(nblk).astype(np.int32)
    assert order_h.min() >= 0 and order_h.max() < nblk          # every block inside buf
    order = torch.from_numpy(order_h).cuda()
    out = {}
    # sequential: 64 KiB blocks back to back; gather: 1 KiB blocks in a random order
    for name, blocks, bb, od in (("sequential", nbytes // 65536, 65536, None), ("gather_1KiB", nblk, 1024, order)):
        for _ in range(2):
            xq.xq_hbm_read_probe(buf, nbytes, blocks, bb, bb, od, sink, sh)
        ev = event_pairs(reps)
        for a, b in ev:
            a.record(stream)
            xq.xq_hbm_read_probe(buf, nbytes, blocks, bb, bb, od, sink, sh)
            b.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        out[name + "_GBps"] = {"best": round(nbytes / (ms.min() * 1e-3) / 1e9, 1),
                               "median": round(nbytes / (np.median(ms) * 1e-3) / 1e9, 1)}
    del buf, order
    torch.cuda.empty_cache()
    out["bytes"] = nbytes
    out["note"] = ("xq_hbm_read_probe: non-temporal 16 B loads, 1 KiB per wave instruction, four in "
                   "flight per lane; HIP events around each launch")
    log(f"HBM reference: {out}")
    return out


def time_prefill(cache, W, bt, to_dev, stream, K, Wm):
    """The chunk's queries attending causally to the chunk (xq_paged_prefill_attention from
    position 0 over the chunk's appended rows): HIP events around each call on its stream, and
    one event pair around replays of a graph holding 8 calls back to back."""
    import torch
    import bit_quantized_paged_turbo_amd as xq
    n, hq = W.chunk_tokens, W.num_q_heads
    g = np.random.default_rng(7)
    q = to_dev(workloads.round_to_bf16_bits(g.standard_normal((n, hq, 128)).astype(np.float32)))
    row = bt[W.batch]
    out = torch.empty((n, hq, 128), dtype=torch.float32, device=q.device)
    need = xq.xq_prefill_workspace_bytes(cache.layout, n, hq, 0, 0)
    ws = torch.empty((max(16, need),), dtype=torch.uint8, device=q.device)

    def call(_=0):
        cache.prefill(q, row, 0, W.softmax_scale, out=out, workspace=ws)

    warm(call, Wm, stream)
    ev = event_pairs(K)
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(8):
            call()
    torch.cuda.synchronize()
    warm(lambda i: graph.replay(), 1, stream)
    nrep = max(1, K // 8)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(nrep):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    gms = a.elapsed_time(b) / (8 * nrep)
    del graph
    pairs = n * (n + 1) // 2                      # (query, key) pairs of the causal chunk
    flops = 4 * 128 * hq * pairs                  # QK and PV multiply-adds
    log(f"prefill of the {n}-token chunk: {ms * 1e3:.1f} us per call, {gms * 1e3:.1f} us replayed 8 a graph")
    return {"queries": n, "start": 0, "call_us": round(ms * 1e3, 2), "call_graph_us": round(gms * 1e3, 2),
            "query_tokens_per_s": round(n / (gms * 1e-3), 1),
            "tflops": round(flops / (gms * 1e-3) / 1e12, 3), "flops_per_call": flops,
            "method": "call_us: HIP events around each eager call; call_graph_us (the rates' time): one event "
                      "pair around replays of a graph of 8 calls"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode path runs on one GPU with no collectives)", file=sys.stderr)
        sys.exit(2)

    W = workloads.config(args.config, dtype=args.dtype)
    log(f"workload {W.name}: batch {W.batch}, {W.total_tokens()} context tokens")
    splits = W.num_splits if args.splits is None else args.splits
    workers = max(1, min(MAX_WORKERS, args.cpu_workers or len(os.sched_getaffinity(0))))

    # ---- host work first, in processes forked before any GPU call --------------------------------
    cpu = None
    if not args.no_cpu:
        log(f"oracle baseline on {workers} host processes")
        cpu = cpu_baseline(W, workers, args.cpu_reps)
        log(f"oracle: quantize {cpu['quantize_s'] * 1e3:.1f} ms, decode {cpu['decode_s'] * 1e3:.1f} ms per step")
    t0 = time.perf_counter()
    if args.inputs_cache and os.path.exists(args.inputs_cache):
        with np.load(args.inputs_cache) as z:
            drawn = {b: (z[f"k{b}"], z[f"v{b}"]) for b in range(W.num_seqs)}
        log(f"inputs loaded from {args.inputs_cache} in {time.perf_counter() - t0:.1f} s")
    else:
        if args.serial_draws:
            drawn = {b: W.kv_bits(b) for b in range(W.num_seqs)}
        else:
            with mp.get_context("fork").Pool(workers, initializer=_pool_init, initargs=(W.cfg, W.dtype)) as pool:
                drawn = dict(pool.imap_unordered(_draw, range(W.num_seqs), chunksize=1))
        log(f"inputs drawn in {time.perf_counter() - t0:.1f} s")
        if args.inputs_cache:
            np.savez(args.inputs_cache, **{f"{n}{b}": a for b, kv in drawn.items() for n, a in zip("kv", kv)})

    import torch
    import bit_quantized_paged_turbo_amd as xq
    from bit_quantized_paged_turbo_amd.cache import PagedKVCache

    lib = xq.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = "cuda"
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 copies of {n} bytes")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # ---- fill one replica with every sequence's context through the append path, timed ---------
    base = PagedKVCache(W.dtype, W.num_kv_heads, W.page_size, W.num_pages)
    bt = to_dev(W.block_tables.astype(np.int32))
    last_k, last_v = [], []
    chunk_kv = None
    pend, batches = [], []
    for b in range(W.num_seqs):
        L = W.seq_len(b)
        k, v = drawn.pop(b)
        if b < W.batch:
            last_k.append(k[-1])
            last_v.append(v[-1])
        else:
            chunk_kv = (k, v)
        pend.append((k, v, np.full(L, b, np.int32), np.arange(L, dtype=np.int32)))
        if sum(len(p[2]) for p in pend) >= (1 << 19) or b == W.num_seqs - 1:
            batches.append(tuple(to_dev(np.concatenate([p[i] for p in pend])) for i in range(4)))
            pend = []
    for k, v, s, p in batches:          # fills the cache (the first launches also load the kernel)
        base.append(k, v, s, p, bt)
    torch.cuda.synchronize()
    # timed: the same rows again (same slots, same bytes), as a steady-state bulk append
    fill_ev = event_pairs(len(batches))
    for (a, b), (k, v, s, p) in zip(fill_ev, batches):
        a.record(stream)
        base.append(k, v, s, p, bt)
        b.record(stream)
    torch.cuda.synchronize()
    fill_ms = sum(a.elapsed_time(b) for a, b in fill_ev)
    fill_rows = sum(int(x[0].shape[0]) for x in batches) * W.num_kv_heads * 2
    rb = row_bytes(W.dtype)
    del batches
    log(f"cache filled through xq_quantize_append: {fill_rows} rows in {fill_ms:.2f} ms")

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
    if args.no_plan:
        args.plan = "none"
    bal = None
    if args.plan == "balanced":
        bal = base.plan_balanced([int(x) for x in W.context_lens], hq, W.max_context_len, device=dev)
        wsb = xq.xq_decode_workspace_bytes_balanced(base.layout, B, hq, bal[0])
    else:
        wsb = base.workspace_bytes(B, hq, W.max_context_len, splits)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev)
    maxp = W.max_pages_per_seq
    fuse = not args.no_fuse
    chunk = None
    app = (new_k.data_ptr(), new_v.data_ptr(), B, new_seq.data_ptr(), new_pos.data_ptr(), bt.data_ptr(), maxp)
    app_rows = B
    if chunk_kv is not None:
        # one append per step takes every new row that the decode launch does not: the chunk's, and
        # without the fused step the decode batch's own too
        nb = 0 if fuse else B
        ck = to_dev(np.concatenate([chunk_kv[0]] + ([] if fuse else [np.stack(last_k)])))
        cv = to_dev(np.concatenate([chunk_kv[1]] + ([] if fuse else [np.stack(last_v)])))
        cs = to_dev(np.concatenate([np.full(W.chunk_tokens, W.batch, np.int32), np.arange(nb, dtype=np.int32)]))
        cp = to_dev(np.concatenate([np.arange(W.chunk_tokens, dtype=np.int32),
                                    (W.context_lens[:nb] - 1).astype(np.int32)]))
        keep = (ck, cv, cs, cp)  # noqa: F841  (alive for the step's pointers)
        app = (ck.data_ptr(), cv.data_ptr(), W.chunk_tokens + nb, cs.data_ptr(), cp.data_ptr(), bt.data_ptr(), maxp)
        app_rows = W.chunk_tokens + nb
        if fuse and bal is not None and args.chunk_append == "decode":
            # the chunk's rows ride in the decode launch, appended by workgroups after its units
            chunk = (ck.data_ptr(), cv.data_ptr(), W.chunk_tokens, cs.data_ptr(), cp.data_ptr())
            app = None
    elif fuse:
        app = None
    # the host plan: long and short sequences share SIMDs (identity where it cannot help)
    order = None
    if args.plan == "uniform":
        order = base.plan([int(x) for x in W.context_lens], hq, W.max_context_len, splits, device=dev)
    dec = (q.data_ptr(), B, hq, bt.data_ptr(), maxp, cl.data_ptr(), W.max_context_len,
           W.softmax_scale, splits, ws.data_ptr(), wsb, out.data_ptr(),
           None if order is None else order.data_ptr(), 0 if order is None else int(order.numel()),
           (new_k.data_ptr(), new_v.data_ptr()) if fuse else None,
           None if bal is None else (bal[0], bal[1].data_ptr(), bal[2].data_ptr()), chunk)
    runners = [Step(lib, c.layout, c, app, dec) for c in caches]

    log(f"{R} pool replicas of {footprint} bytes; timing")
    K, Wm = args.steps, args.warmup

    def eager_step(i):
        r = runners[i % R]
        r.run(sp)
        r.decode(sp)

    Wm = warm(eager_step, Wm, stream)

    ev = event_pairs(K)
    app_ev = event_pairs(K) if app is not None else None
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        r = runners[(Wm + i) % R]
        if app_ev is not None:
            app_ev[i][0].record(stream)
        r.run(sp)
        if app_ev is not None:
            app_ev[i][1].record(stream)
        ev[i][0].record(stream)
        r.decode(sp)
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / K
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec_avg_ms = float(dec_ms.mean())
    app_avg_ms = float(np.mean([a.elapsed_time(b) for a, b in app_ev])) if app_ev is not None else None

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
        Wg = warm(lambda i: graphs[i % NG].replay(), args.warmup, stream)
        gstart, gstop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gstart.record(stream)
        for i in range(K):
            graphs[(Wg + i) % NG].replay()
        gstop.record(stream)
        torch.cuda.synchronize()
        g_ms = gstart.elapsed_time(gstop) / K
        graph = {"ms_per_step": round(g_ms, 5), "replicas": NG}
        log(f"graph replay: {g_ms * 1e3:.1f} us/step")
        # One graph holding S steps back to back, a step on every replica in turn (S = R), or 8
        # steps on the one replica whose pools outgrow the Infinity Cache (S = 8), as a model's
        # decode graph holds one step per layer (the replicas' pools stand for the layers'
        # caches): K steps are K // S replays of it plus K % S single-step replays.
        S = R if R > 1 else 8
        if NG == R and S <= 64:
            layers = torch.cuda.CUDAGraph()
            with torch.cuda.graph(layers):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(S):
                    runners[i % R].run(cs)
                    runners[i % R].decode(cs)
            torch.cuda.synchronize()
            warm(lambda i: layers.replay(), max(1, args.warmup // S), stream)
            gstart.record(stream)
            for _ in range(K // S):
                layers.replay()
            for i in range(K % S):
                graphs[i % NG].replay()
            gstop.record(stream)
            torch.cuda.synchronize()
            m_ms = gstart.elapsed_time(gstop) / K
            graph["multi_step_ms_per_step"] = round(m_ms, 5)
            graph["steps_per_graph"] = S
            log(f"graph of {S} steps: {m_ms * 1e3:.1f} us/step")
            del layers
        del graphs
        # The decode call alone: one graph holding M decode calls back to back (one per pool
        # replica in turn, or 8 calls on the one replica), replayed so that about K calls run,
        # with one HIP event pair on the stream around them all; the mean carries neither host
        # launch gaps, nor per-call event markers, nor a graph launch per call.
        M = min(64, R if R > 1 else 8)
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(M):
                runners[i % R].decode(cs)
        torch.cuda.synchronize()
        warm(lambda i: dgraph.replay(), max(1, args.warmup // M), stream)
        nrep = max(1, K // M)
        gstart.record(stream)
        for _ in range(nrep):
            dgraph.replay()
        gstop.record(stream)
        torch.cuda.synchronize()
        dg_us = gstart.elapsed_time(gstop) / (nrep * M) * 1e3
        graph["decode_call_us"] = round(dg_us, 2)
        graph["decode_calls_timed"] = nrep * M
        log(f"decode call, {M} a graph: {dg_us:.1f} us")
        del dgraph

    kv_bytes = int(W.context_lens.astype(np.int64).sum()) * hkv * 2 * rb
    tokens = int(W.context_lens.astype(np.int64).sum())
    nsplits = bal[0] if bal is not None else xq.xq_decode_num_splits(base.layout, B, hq, W.max_context_len, splits)
    by_graph = graph is not None and graph["replicas"] == R
    by_layers = by_graph and "multi_step_ms_per_step" in graph
    timed_ms = graph["multi_step_ms_per_step"] if by_layers else graph["ms_per_step"] if by_graph else step_ms
    value = kv_bytes / (timed_ms * 1e-3) / 1e9
    # the decode launch's algorithmic bytes: the KV rows it reads, plus the chunk's rows (bf16 in,
    # codes and scale out) where it appends them too
    chunk_bytes = W.chunk_tokens * hkv * 2 * (256 + rb) if chunk is not None else 0
    launch_bytes = kv_bytes + chunk_bytes
    # the decode call's duration: replayed alone from a graph where there is one, else eager
    call_ms = graph["decode_call_us"] * 1e-3 if graph is not None else dec_avg_ms
    achieved = launch_bytes / (call_ms * 1e-3) / 1e9
    tag = f"decode_call_{workloads.DTYPE_NAMES[W.dtype]}_{W.name}"
    prof = committed_profile(tag)
    kernel_us = prof.get("decode_call_kernel_us")

    # the append kernel's own rate: bf16 rows in, code rows and scales out
    append = {"bytes_per_row": 256 + rb,
              "fill_rows": fill_rows, "fill_ms": round(fill_ms, 4),
              "fill_GBps": round(fill_rows * (256 + rb) / (fill_ms * 1e-3) / 1e9, 1)}
    if app_avg_ms is not None:
        rows = app_rows * hkv * 2
        append.update({"step_rows": rows, "step_call_us": round(app_avg_ms * 1e3, 2),
                       "step_GBps": round(rows * (256 + rb) / (app_avg_ms * 1e-3) / 1e9, 1)})

    result = {
        "metric": "quantized paged decode attn: KV GB/s (% of HBM peak) and seq-tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(timed_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {4: "i4xi8->i32 QK (3 query digits), f32 softmax, f16 PV->f32",
                  3: "i3xi8->i32 QK (3 query digits), f32 softmax, f16 PV->f32",
                  2: "i2xi8->i32 QK (3 query digits), f32 softmax, f16 PV->f32",
                  8: "i8xi8->i32 QK (3 query digits), f32 softmax, f16 PV->f32",
                  0: "bf16xbf16->f32", workloads.FP8: "e4m3->bf16, bf16xbf16->f32"}[W.dtype],
        "data": "synthetic",
        "config": {
            "workload": W.name, "description": W.note, "cache": workloads.DTYPE_NAMES[W.dtype],
            "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
            "page_size": W.page_size, "context_tokens": tokens, "max_context": W.max_context_len,
            "splits": nsplits, "chunk_append_tokens": W.chunk_tokens, "pool_replicas": R,
            "plan": ("length-aware partitions (xq_decode_plan_balanced)" if bal is not None else
                     None if order is None else "permutation of the batch" if int(order.numel()) == B
                     else "unit placement (longest first, balanced SIMDs)"),
            "fused_append": fuse,
            "chunk_append": (None if not W.chunk_tokens else "in the decode launch" if chunk is not None
                             else "separate append kernel"),
        },
        "step_timing": {"method": ((f"hip graph replay, {R} steps (one per pool replica, as one per layer) per graph"
                                    if R > 1 else "hip graph replay, 8 steps on the one pool replica per graph")
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
                           "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                           "method": "HIP events around each eager call in the timed steps"},
        "decode_call_graph_us": graph["decode_call_us"] if graph is not None else None,
        "decode_calls_graph_timed": graph["decode_calls_timed"] if graph is not None else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "duration": ("decode_call_graph_us: one HIP event pair around replays of a graph "
                                  "holding only decode calls, back to back" if graph is not None
                                  else "decode_call_us (eager)"),
                     "traffic": prof.get("hbm_bytes_per_launch"),
                     "frac_kernel_trace": (round(launch_bytes / (kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                           if kernel_us else None),
                     "kernel_trace_us": kernel_us,
                     "kernel": ("xq_decode_attention_balanced" if bal is not None else
                                "xq_append_decode_attention" if fuse else "xq_paged_decode_attention")
                               + " call (decode_split_kernel"
                               + (" + decode_combine_kernel)" if nsplits > 1 else ")"),
                     "bytes_per_launch": launch_bytes,
                     "bytes_note": "algorithmic: sum_b L_b x Hkv x (K row + V row), a row being "
                                   f"{rb} B (codes + fp16 scale)"
                                   + (f"; plus the chunk's {W.chunk_tokens} x Hkv x (K, V) rows appended in "
                                      f"the launch, {256 + rb} B each (bf16 in, codes + scale out)"
                                      if chunk is not None else "")},
        "append": append,
    }
    if chunk_kv is not None and not args.no_prefill:
        result["prefill"] = time_prefill(base, W, bt, to_dev, stream, K, args.warmup)
    if not args.no_probe:
        del caches, runners
        result["hbm_reference"] = hbm_reference(xq, stream)
    log(f"GPU: {step_ms * 1e3:.1f} us/step eager, "
        f"{'%.1f' % (graph['ms_per_step'] * 1e3) if graph is not None else '-'} us/step graph, "
        f"decode call {dec_avg_ms * 1e3:.1f} us")
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
